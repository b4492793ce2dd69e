"""The seeded workloads do what their descriptions say (CPU only).

These check the generator's planting against the oracle's verification:
the tiny workload accepts the rank-0 chain to depth 3, the geometric
workload's accept lengths follow the planted draw (mean emitted tokens per
step (1 - 0.6^7) / 0.4 = 2.430 by the expected-tokens-per-pass formula), the
cycle workload's top-8 rows are all cycle ids, and the first-order workload
is lossless.
"""
import numpy as np
import torch

from oracle import tr_oracle as O
from synth import workloads as W


def test_shapes_and_caps():
    for w in W.WORKLOADS.values():
        t = O.template_from_levels(w.levels)
        assert t.n_nodes == w.T and t.parent.tolist() == w.parent
        assert w.cap() >= w.prefix[1] + w.steps * (t.max_depth + 1)
    assert W.WORKLOADS["tiny"].T == 16 and W.WORKLOADS["vicuna7b"].T == 81


def test_initial_state_is_seeded():
    w = W.WORKLOADS["tiny"].scaled(V=500)
    a, b = W.initial_state(w), W.initial_state(w)
    assert torch.equal(a.M, b.M) and torch.equal(a.k_cache, b.k_cache)
    assert a.M.dtype == torch.int64 and int(a.M.max()) < 500
    assert int(a.prefix_len[0]) == 256
    assert (a.k_cache[0, :, 256:] == 0).all()


def test_varlen_prefix_zero_tail():
    w = W.WORKLOADS["largevocab"].scaled(V=300, B=4, prefix=(10, 40), Hkv=2, Hq=4, steps=2)
    s = W.initial_state(w)
    for b in range(4):
        P = int(s.prefix_len[b])
        assert 10 <= P <= 40
        assert (s.k_cache[b, :, P:] == 0).all() and (s.k_cache[b, :, :P] != 0).any()


def test_tiny_plants_depth3_chain():
    w = W.WORKLOADS["tiny"]
    t = O.template_from_levels(w.levels)
    st = W.initial_state(w)
    tok = O.retrieve(t, st.M[0].numpy(), int(st.root[0]))
    z = W.step_logits(w, 0, torch.from_numpy(tok)[None]).numpy()[0]
    top = O.topk_rows(z, w.k)
    v = O.verify(t, tok, top[:, 0])
    assert v.accept_len == 3 and v.path.tolist() == [0, 1, 5, 13]


def test_geometric_accept_lengths():
    w = W.WORKLOADS["vicuna13b"]
    t = O.template_from_levels(w.levels)
    rng = np.random.default_rng(0)
    total, n = 0, 1500
    for s in range(n):
        tok = rng.integers(0, 40, size=w.T)            # tiny id range: many duplicate siblings
        tgt = W.plant_targets(w, s, torch.from_numpy(tok)[None])[0].numpy()
        v = O.verify(t, tok, tgt)
        u = torch.rand((1,), generator=W._gen("cpu", w.seed, W._S_PLANT, s), dtype=torch.float64)
        Lstar = min(int(np.floor(np.log(float(u[0])) / np.log(0.6))), 6)
        assert v.accept_len == Lstar
        total += v.accept_len + 1
    assert abs(total / n - (1 - 0.6 ** 7) / 0.4) < 0.15


def test_cycle_rows_top8_are_cycle_ids():
    w = W.WORKLOADS["codellama34b"]
    S = set(W.cycle_ids(w).tolist())
    tok = torch.tensor([list(S)[:10] + [5] * (w.T - 10)])
    z = W.step_logits(w, 3, tok).float().numpy()[0]
    top = O.topk_rows(z, 8)
    assert set(top.ravel().tolist()) <= S
    assert all(len(set(r)) == 8 for r in top.tolist())


def test_first_order_loop_is_lossless():
    w = W.WORKLOADS["vicuna7b"].scaled(V=2000, Hq=1, Hkv=1, prefix=(4, 4), steps=6)
    t = O.template_from_levels(w.levels)
    st = W.initial_state(w)
    M = st.M[0].numpy().astype(np.int64)
    H = W.first_order_map(w)[0].numpy()
    tok = O.retrieve(t, M, int(st.root[0]))
    stream = []
    for s in range(w.steps):
        z = W.step_logits(w, s, torch.from_numpy(tok)[None]).float().numpy()[0]
        res, _ = O.step_after_forward(t, M, tok, z, w.k)
        stream += res.verdict.emitted.tolist()
        tok = res.next_tok
    want = [int(st.root[0])]
    for _ in stream:
        want.append(int(H[want[-1]]))
    assert stream == want[1:]
