"""Whole-loop parity on the five seeded workloads, at full size (MI355X only).

The HIP path runs exactly what the benchmark times: per step one
tr_tree_attn call and one fused tr_step call, on the workload's shapes and
step count.  The oracle runs the same trajectory on the host from the same
seeded inputs: the logits of every step are drawn from the ORACLE's tree
tokens, after checking that the GPU's tree equals them.

Checked bit for bit on every step of every followed sequence: tree tokens,
top-k of every node, accepted length, path, emitted tokens, next root,
prefix length; at the end: every row of M and every committed key/value
row.  Attention is checked within 2e-2 absolute (bf16) or 1e-5 relative per
row (fp32) on every step of the single-sequence workloads and on steps {0,
1, every 8th, last} of the 32-sequence batch, whose 32 sequences are all
followed.  The attention checks run after the loop, against the oracle's
final cache cut to each step's prefix length (committed rows never change
afterwards), in a pool of threads (numpy releases the GIL in the heavy
calls; BLAS is held to one thread per worker).
"""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch
from threadpoolctl import threadpool_limits

from oracle import tr_oracle as O
from synth import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def tr():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from draft_tree_retrieval_amd import tr as _tr
    _tr.load()
    return _tr


def attn_ok(t, out, q, kt, vt, kc, vc, P, dtype):
    want = O.tree_attention(t, q, kt, vt, kc, vc, P)
    if dtype == torch.float32:
        rel = np.abs(out - want).max(-1) / np.maximum(np.abs(want).max(-1), 1e-30)
        return float(rel.max()), rel.max() <= 1e-5
    err = float(np.abs(out - want).max())
    return err, err <= 2e-2


MARGIN = 2e-5      # a uniform this close to a threshold could go either way in float32
POOL = max(1, min(16, os.cpu_count() or 1))


def run_loop(tr, w, steps, track, attn_steps, update="all", temperature=0.0):
    with threadpool_limits(1), ThreadPoolExecutor(POOL) as ex:
        return _run_loop(tr, w, steps, track, attn_steps, update, temperature, ex)


def _run_loop(tr, w, steps, track, attn_steps, update, temperature, ex):
    from draft_tree_retrieval_amd.loop import TRDecoder
    t = O.template_from_levels(w.levels)
    st = W.initial_state(w, DEV)
    host = st.to("cpu")
    tree = tr.Tree.from_levels(w.levels, w.k)
    dec = TRDecoder(tree, st.M, st.k_cache, st.v_cache, st.prefix_len, st.root, Hq=w.Hq,
                    update=update)
    # oracle state of the tracked sequences
    oM = {b: host.M[b].numpy().astype(np.int64).copy() for b in track}
    okc = {b: host.k_cache[b].float().numpy().copy() for b in track}
    ovc = {b: host.v_cache[b].float().numpy().copy() for b in track}
    oP = {b: int(host.prefix_len[b]) for b in track}
    otok = {b: O.retrieve(t, oM[b], int(host.root[b])) for b in track}
    P0 = dict(oP)
    pending = []                                    # attention checks, run after the loop
    out = torch.empty((w.B, w.T, w.Hq, w.d), dtype=w.kv_dtype, device=DEV)
    for s in range(steps):
        gtok = dec.tree_tok.cpu().numpy()
        for b in track:
            assert (gtok[b] == otok[b]).all(), f"step {s} seq {b}: tree differs"
        q, kt, vt = W.step_qkv(w, s, DEV)
        dec.attend(q, kt, vt, out)
        if s in attn_steps:
            oh, qh, kh, vh = (x.cpu() for x in (out, q, kt, vt))
            pending += [(s, b, oh[b], qh[b], kh[b], vh[b], oP[b]) for b in track]
        gen_tok = dec.tree_tok.clone()
        for b in track:
            gen_tok[b] = torch.from_numpy(otok[b]).to(torch.int32)
        logits = W.step_logits(w, s, gen_tok, DEV)
        lh = logits.cpu()
        zl = {b: lh[b].float().numpy() for b in track}
        if temperature > 0:
            # uniforms of every sequence; those of the followed ones redrawn
            # until every decision clears its threshold
            ug = torch.Generator().manual_seed(7000 + s)
            U = torch.rand((w.B, w.T, 2), generator=ug)
            for b in track:
                while O.verify_sample(t, otok[b], zl[b], temperature,
                                      U[b].double().numpy()).margin <= MARGIN:
                    U[b] = torch.rand((w.T, 2), generator=ug)
            dec.step_sample(logits, kt, vt, temperature, U.to(DEV))
        else:
            dec.step(logits, kt, vt)
        kth, vth = kt.float().cpu().numpy(), vt.float().cpu().numpy()

        def oracle_step(b):
            # sequences are independent: each thread mutates only its own state
            return O.step_after_forward(t, oM[b], otok[b], zl[b], w.k, okc[b], ovc[b], kth[b],
                                        vth[b], oP[b], update_mode=update, temperature=temperature,
                                        uniforms=U[b].double().numpy() if temperature > 0 else None)

        results = dict(zip(track, ex.map(oracle_step, track)))
        gk = dec.topk.cpu().numpy()
        gL, gem, groot, gP = (x.cpu().numpy() for x in (dec.accept_len, dec.emitted, dec.root_tok,
                                                        dec.prefix_len))
        for b in track:
            res, oP[b] = results[b]
            assert (gk[b] == res.topk).all(), f"step {s} seq {b}: top-k differs"
            v = res.verdict
            assert int(gL[b]) == v.accept_len, f"step {s} seq {b}: accept length"
            em = v.emitted.tolist() + [-1] * (t.max_depth + 1 - len(v.emitted))
            assert gem[b].tolist() == em, f"step {s} seq {b}: emitted"
            assert int(groot[b]) == v.bonus and int(gP[b]) == oP[b]
            otok[b] = res.next_tok
    assert dec.device_flags() == 0
    Mh = dec.M.cpu()
    for b in track:
        assert (Mh[b].numpy().astype(np.int64) == oM[b]).all(), f"seq {b}: M differs"
        kc = dec.k_cache[b, :, P0[b]:oP[b]].float().cpu().numpy()
        vc = dec.v_cache[b, :, P0[b]:oP[b]].float().cpu().numpy()
        assert (kc == okc[b][:, P0[b]:oP[b]]).all() and (vc == ovc[b][:, P0[b]:oP[b]]).all()

    def check(item):
        s, b, o, qq, kk, vv, P = item
        err, ok = attn_ok(t, o.float().numpy(), qq.float().numpy(), kk.float().numpy(),
                          vv.float().numpy(), okc[b], ovc[b], P, w.kv_dtype)
        return s, b, err, ok

    worst = 0.0
    for s, b, err, ok in ex.map(check, pending):
        worst = max(worst, err)
        assert ok, f"step {s} seq {b}: attention error {err}"
    assert len(pending) == len(attn_steps & set(range(steps))) * len(track)
    return worst


def test_tiny_full(tr):
    w = W.WORKLOADS["tiny"]
    run_loop(tr, w, w.steps, [0], {0})


def test_vicuna7b_full(tr):
    w = W.WORKLOADS["vicuna7b"]
    run_loop(tr, w, w.steps, [0], set(range(w.steps)))


def test_vicuna13b_full(tr):
    w = W.WORKLOADS["vicuna13b"]
    run_loop(tr, w, w.steps, [0], set(range(w.steps)))


def test_codellama34b_full(tr):
    w = W.WORKLOADS["codellama34b"]
    run_loop(tr, w, w.steps, [0], set(range(w.steps)))


def test_tiny_accepted_only_update(tr):
    # the ablation that recycles the accepted path only (tr_step_ex)
    w = W.WORKLOADS["tiny"]
    run_loop(tr, w, w.steps, [0], {0}, update="accepted")


def test_vicuna7b_accepted_only_update(tr):
    w = W.WORKLOADS["vicuna7b"]
    run_loop(tr, w, 64, [0], {0, 63}, update="accepted")


def test_vicuna7b_sampling(tr):
    # verification by sampling at temperature 1 (tr_step_sample)
    w = W.WORKLOADS["vicuna7b"]
    run_loop(tr, w, 48, [0], {0, 47}, temperature=1.0)


def test_largevocab_sampling_sampled_sequences(tr):
    w = W.WORKLOADS["largevocab"]
    run_loop(tr, w, 16, [0, 31], {0}, temperature=0.8)


@pytest.mark.parametrize("wl,ps,steps", [("vicuna7b", 64, 256), ("largevocab", 128, 24)])
def test_paged_loop_equals_contiguous(tr, wl, ps, steps):
    # the paged cache (shuffled pages) runs the same trajectory bit for bit:
    # attention outputs, trees, verdicts, M and the committed rows
    from draft_tree_retrieval_amd.loop import TRDecoder, from_pages
    w = W.WORKLOADS[wl]
    cap = -(-w.cap(steps) // ps) * ps
    tree = tr.Tree.from_levels(w.levels, w.k)
    sa, sb = W.initial_state(w, DEV, cap=cap), W.initial_state(w, DEV, cap=cap)
    da = TRDecoder(tree, sa.M, sa.k_cache, sa.v_cache, sa.prefix_len, sa.root, Hq=w.Hq)
    db = TRDecoder(tree, sb.M, sb.k_cache, sb.v_cache, sb.prefix_len, sb.root, Hq=w.Hq,
                   page_size=ps)
    oa = torch.empty((w.B, w.T, w.Hq, w.d), dtype=w.kv_dtype, device=DEV)
    ob = torch.empty_like(oa)
    for s in range(steps):
        q, kt, vt = W.step_qkv(w, s, DEV)
        da.attend(q, kt, vt, oa)
        db.attend(q, kt, vt, ob)
        assert torch.equal(oa, ob), f"step {s}: attention differs"
        z = W.step_logits(w, s, da.tree_tok, DEV)
        da.step(z, kt, vt)
        db.step(z, kt, vt)
        assert torch.equal(da.tree_tok, db.tree_tok) and torch.equal(da.prefix_len, db.prefix_len)
        assert torch.equal(da.emitted, db.emitted), f"step {s}"
    assert torch.equal(da.M, db.M)
    assert torch.equal(from_pages(db.k_pages, db.block_table), da.k_cache)
    assert torch.equal(from_pages(db.v_pages, db.block_table), da.v_cache)
    assert da.device_flags() == 0 and db.device_flags() == 0


def test_largevocab_full_all_sequences(tr):
    # every sequence's integer results on every step; attention on steps
    # 0, 1, every 8th and the last
    w = W.WORKLOADS["largevocab"]
    run_loop(tr, w, w.steps, list(range(w.B)), {0, 1, w.steps - 1} | set(range(0, w.steps, 8)))
