"""The greedy step for few logit rows (fewer than 256 rows of at most 32768
logits: one block per row, a tail block per sequence that polls the rows'
results, commit blocks that copy the accepted rows).

Checked against the CPU oracle bit for bit (top-k ids, M, verdict, next
tree, prefix length, committed cache rows) on rows chosen to stress the
selection (ties, signed zeros, infinities, unaligned and odd lengths, the
longest rows the kernel holds), on several sequences per launch and on one
workspace reused across launches of different shapes; and bit-identical to
the general kernel (diagnostic switch TR_FEW_ROW_STEP=0) on the same
inputs.  MI355X only.
"""
import math

import numpy as np
import pytest
import torch

from oracle import tr_oracle as O

pytestmark = pytest.mark.gpu
DEV = "cuda"
TREE_81 = [[8], [6, 4, 3, 2, 2, 1, 1, 1], [5, 4, 3, 2, 2, 2, 1, 1, 1, 1],
           [4, 3, 2, 2, 2, 1, 1, 1, 1, 1], [3, 2, 2, 1, 1, 1], [2]]


@pytest.fixture(scope="module")
def tr():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from draft_tree_retrieval_amd import tr as _tr
    _tr.load()
    return _tr


def rows_cases():
    g = torch.Generator().manual_seed(12)
    cases = []
    z = (torch.randint(-3, 4, (9, 5003), generator=g).float() * 0.5)
    z[0, ::7] = -0.0
    z[1, 100] = math.inf
    z[2, :] = -math.inf
    z[2, 4000] = 0.0
    z[3, :] = 0.0                       # every element tied: the list overflows
    z[3, 17] = -0.0
    z[4, :] = -0.0
    z[4, 4999] = 0.0
    cases.append(("ties_f32", z))
    cases.append(("ties_bf16", z.to(torch.bfloat16)))
    cases.append(("bf16_32000", (torch.randn((81, 32000), generator=g) * 3).to(torch.bfloat16)))
    cases.append(("bf16_longest", (torch.randn((7, 32768), generator=g) * 3).to(torch.bfloat16)))
    cases.append(("f32_longest_odd", torch.randn((5, 32767), generator=g) * 2))
    cases.append(("bf16_odd", (torch.randn((5, 1037), generator=g) * 3).to(torch.bfloat16)))
    cases.append(("f32_tiny", torch.randn((6, 16), generator=g)))
    # the best values in the last elements (the loose tail) and a tie there
    z = (torch.randn((4, 32001), generator=g) * 3).to(torch.bfloat16)
    z[:, 32000] = 100.0
    z[:, 31999] = 90.0
    z[:, 0] = 90.0
    cases.append(("bf16_tail_best", z))
    return cases


def set_kernel(monkeypatch, few):
    if few:
        monkeypatch.delenv("TR_FEW_ROW_STEP", raising=False)
    else:
        monkeypatch.setenv("TR_FEW_ROW_STEP", "0")


@pytest.mark.parametrize("k", [1, 3, 8, 16])
def test_update_rows_parity(tr, monkeypatch, k):
    # tr_update_topk with M: the kernel's update-only tail
    rng = np.random.default_rng(k)
    for name, z in rows_cases():
        rows, V = z.shape
        if V < k:
            continue
        tree = tr.Tree.from_levels([[1]] * (rows - 1), k)     # a chain: rows nodes
        tok = rng.integers(0, min(V, 12), size=(1, rows)).astype(np.int32)   # repeats
        M0 = torch.from_numpy(rng.integers(0, V, size=(1, V, k))).to(torch.int32)
        got = {}
        for few in (True, False):
            set_kernel(monkeypatch, few)
            ws = tr.new_workspace(tree, 1, V, k, 0, 0, 0, 0, device=DEV)
            Md = M0.to(DEV)
            out = torch.empty((1, rows, k), dtype=torch.int32, device=DEV)
            tr.tr_update_topk(tree, z[None].to(DEV), torch.from_numpy(tok).to(DEV), Md, out, ws)
            got[few] = (out.cpu(), Md.cpu())
            assert tr.tr_read_device_status(ws) == 0
        want = O.topk_rows(z.float().numpy(), k)
        ids = got[True][0][0].numpy()
        bad = np.flatnonzero((ids != want).any(axis=1))
        assert len(bad) == 0, f"{name} k={k}: rows {bad[:5]} got {ids[bad[0]]} want {want[bad[0]]}"
        Mo = M0[0].numpy().astype(np.int64).copy()
        O.update(Mo, tok[0], want)
        assert (got[True][1][0].numpy() == Mo).all(), name
        assert torch.equal(got[True][0], got[False][0]) and torch.equal(got[True][1], got[False][1])


def planted_step_inputs(tr, g, rng, levels, B, V, k, Hkv, cap, P):
    t = O.template_from_levels(levels)
    tree = tr.Tree.from_levels(levels, k)
    M = torch.randint(0, V, (B, V, k), generator=g, dtype=torch.int32)
    root = torch.randint(0, V, (B,), generator=g, dtype=torch.int32)
    tok = torch.empty((B, t.n_nodes), dtype=torch.int32, device=DEV)
    ws = tr.new_workspace(tree, B, V, k, 0, 0, 0, 0, device=DEV)
    tr.tr_retrieve(tree, M.to(DEV), root.to(DEV), tok, ws)
    tok_h = tok.cpu().numpy().astype(np.int64)
    z = (torch.randn((B, t.n_nodes, V), generator=g) * 3)
    for b in range(B):                                  # accept along random edges
        for n in range(1, t.n_nodes):
            if rng.random() < 0.6:
                z[b, t.parent[n], tok_h[b, n]] = 40.0 + float(rng.random())
    z = z.to(torch.bfloat16)
    kc = torch.randn((B, Hkv, cap, 128), generator=g).to(torch.bfloat16)
    vc = torch.randn((B, Hkv, cap, 128), generator=g).to(torch.bfloat16)
    kt = torch.randn((B, t.n_nodes, Hkv, 128), generator=g).to(torch.bfloat16)
    vt = torch.randn((B, t.n_nodes, Hkv, 128), generator=g).to(torch.bfloat16)
    Pt = torch.tensor(P, dtype=torch.int32)
    return t, tree, M, root, tok_h, z, kc, vc, kt, vt, Pt


def run_step(tr, tree, t, M, root, tok_h, z, kc, vc, kt, vt, P, ws=None):
    B, T, V = z.shape
    k = M.shape[2]
    if ws is None:
        ws = tr.new_workspace(tree, B, V, k, 0, 0, 0, 0, device=DEV)
    dM, droot, dkc, dvc, dP = (x.to(DEV) for x in (M, root, kc, vc, P))
    tok = torch.from_numpy(tok_h.astype(np.int32)).to(DEV)
    L = torch.empty((B,), dtype=torch.int32, device=DEV)
    path = torch.empty((B, t.max_depth + 1), dtype=torch.int32, device=DEV)
    em = torch.empty((B, t.max_depth + 1), dtype=torch.int32, device=DEV)
    topk = torch.empty((B, T, k), dtype=torch.int32, device=DEV)
    tr.tr_step(tree, z.to(DEV), dM, tok, droot, L, path, em, ws, kt.to(DEV), vt.to(DEV), dkc, dvc,
               dP, topk_out=topk)
    flags = tr.tr_read_device_status(ws)
    return dict(M=dM.cpu(), root=droot.cpu(), kc=dkc.cpu(), vc=dvc.cpu(), P=dP.cpu(), tok=tok.cpu(),
                L=L.cpu(), path=path.cpu(), em=em.cpu(), topk=topk.cpu(), flags=flags)


def check_vs_oracle(t, M, tok_h, z, kc, vc, kt, vt, P, got):
    B = z.shape[0]
    k = M.shape[2]
    for b in range(B):
        Mo = M[b].numpy().astype(np.int64).copy()
        kco, vco = kc[b].float().numpy().copy(), vc[b].float().numpy().copy()
        res, newP = O.step_after_forward(t, Mo, tok_h[b], z[b].float().numpy(), k, kco, vco,
                                         kt[b].float().numpy(), vt[b].float().numpy(), int(P[b]))
        v = res.verdict
        assert (got["topk"][b].numpy() == res.topk).all(), b
        assert (got["M"][b].numpy().astype(np.int64) == Mo).all(), b
        assert int(got["L"][b]) == v.accept_len and int(got["root"][b]) == v.bonus
        assert got["path"][b, :v.accept_len + 1].tolist() == v.path.tolist()
        em = v.emitted.tolist() + [-1] * (t.max_depth + 1 - len(v.emitted))
        assert got["em"][b].tolist() == em
        assert got["tok"][b].numpy().tolist() == res.next_tok.tolist()
        assert int(got["P"][b]) == newP
        assert (got["kc"][b].float().numpy() == kco).all() and (got["vc"][b].float().numpy() == vco).all()


@pytest.mark.parametrize("B,Hkv", [(1, 32), (3, 8), (3, 40)])
def test_step_sequences_commit(tr, monkeypatch, B, Hkv):
    # B sequences of the 81-node tree (243 rows at B = 3), commit blocks
    # sized for Hkv heads; the general kernel must give the same bits
    g = torch.Generator().manual_seed(100 + B * Hkv)
    rng = np.random.default_rng(B * Hkv)
    V, k, cap = 32000, 8, 64
    P = [int(x) for x in rng.integers(0, cap - 7, size=B)]
    t, tree, M, root, tok_h, z, kc, vc, kt, vt, Pt = planted_step_inputs(tr, g, rng, TREE_81, B, V,
                                                                         k, Hkv, cap, P)
    set_kernel(monkeypatch, True)
    few = run_step(tr, tree, t, M, root, tok_h, z, kc, vc, kt, vt, Pt)
    assert few["flags"] == 0
    assert int(few["L"].max()) >= 2                        # the plants were accepted
    check_vs_oracle(t, M, tok_h, z, kc, vc, kt, vt, Pt, few)
    set_kernel(monkeypatch, False)
    gen = run_step(tr, tree, t, M, root, tok_h, z, kc, vc, kt, vt, Pt)
    for key in few:
        if key == "flags":
            assert gen[key] == few[key]
        else:
            assert torch.equal(gen[key], few[key]), key


def test_workspace_reused_across_shapes(tr, monkeypatch):
    # one workspace, launches of different (B, tree) in a row: the mailbox,
    # verdict words and counters each launch leaves must not leak into the
    # next; the last launch overflows one cache (flag, no commit)
    set_kernel(monkeypatch, True)
    g = torch.Generator().manual_seed(7)
    rng = np.random.default_rng(7)
    V, k, Hkv, cap = 5000, 8, 4, 48
    big = tr.Tree.from_levels(TREE_81, k)
    ws = tr.new_workspace(big, 3, V, k, 0, 0, 0, 0, device=DEV)
    shapes = [(TREE_81, 3, [3, 10, 20]), ([[4], [4, 2, 1, 1], [2, 1]], 1, [5]),
              (TREE_81, 2, [0, 30]), ([[1]] * 9, 2, [1, 2]), (TREE_81, 1, [44])]
    for i, (levels, B, P) in enumerate(shapes):
        t, tree, M, root, tok_h, z, kc, vc, kt, vt, Pt = planted_step_inputs(tr, g, rng, levels, B,
                                                                             V, k, Hkv, cap, P)
        got = run_step(tr, tree, t, M, root, tok_h, z, kc, vc, kt, vt, Pt, ws=ws)
        if i < len(shapes) - 1:
            assert got["flags"] == 0, i
            check_vs_oracle(t, M, tok_h, z, kc, vc, kt, vt, Pt, got)
        else:
            fits = int(got["L"][0]) + 1 + 44 <= cap
            assert bool(got["flags"] & tr.TR_FLAG_CACHE_FULL) == (not fits)
            if not fits:
                assert int(got["P"][0]) == 44 and torch.equal(got["kc"], kc)


@pytest.mark.parametrize("B,Hkv", [(1, 32), (3, 8)])
def test_step_lmhead_paths_commit(tr, monkeypatch, B, Hkv):
    # the fused LM head's step through the few-row step kernel (the slice
    # lists merged in its row blocks) and through the merge kernel (one block
    # per row, the tail in the last one of a sequence): the same bits, cache
    # commits included
    g = torch.Generator().manual_seed(300 + B)
    rng = np.random.default_rng(300 + B)
    V, k, cap, H = 32000, 8, 64, 256
    P = [int(x) for x in rng.integers(0, cap - 7, size=B)]
    t, tree, M, root, tok_h, _, kc, vc, kt, vt, Pt = planted_step_inputs(tr, g, rng, TREE_81, B, V,
                                                                         k, Hkv, cap, P)
    T = t.n_nodes
    W = (torch.randn((V, H), generator=g) / H ** 0.5).to(torch.bfloat16)
    # hidden states leaning towards the W row of a child's token, so that
    # drafts are accepted along random edges
    h = torch.randn((B, T, H), generator=g) * 0.3
    for b in range(B):
        for n in range(T):
            ch = t.children(n)
            if ch and rng.random() < 0.7:
                h[b, n] += W[tok_h[b, ch[int(rng.integers(len(ch)))]]].float() * 4.0
    h = h.to(torch.bfloat16)

    def run(few):
        set_kernel(monkeypatch, few)
        ws = tr.new_lmhead_workspace(B * T, V, k)
        dM, droot, dkc, dvc, dP = (x.to(DEV) for x in (M, root, kc, vc, Pt))
        tok = torch.from_numpy(tok_h.astype(np.int32)).to(DEV)
        L = torch.empty((B,), dtype=torch.int32, device=DEV)
        path = torch.empty((B, t.max_depth + 1), dtype=torch.int32, device=DEV)
        em = torch.empty((B, t.max_depth + 1), dtype=torch.int32, device=DEV)
        topk = torch.empty((B, T, k), dtype=torch.int32, device=DEV)
        tr.tr_step_lmhead(tree, h.to(DEV), W.to(DEV), dM, tok, droot, L, path, em, ws, kt.to(DEV),
                          vt.to(DEV), dkc, dvc, dP, topk_out=topk)
        return dict(M=dM.cpu(), root=droot.cpu(), kc=dkc.cpu(), vc=dvc.cpu(), P=dP.cpu(),
                    tok=tok.cpu(), L=L.cpu(), path=path.cpu(), em=em.cpu(), topk=topk.cpu(),
                    flags=tr.tr_read_device_status(ws))

    few, merged = run(True), run(False)
    assert few["flags"] == 0 and merged["flags"] == 0
    assert int(few["L"].max()) >= 2                        # drafts were accepted
    for key in few:
        if key != "flags":
            assert torch.equal(few[key], merged[key]), key
