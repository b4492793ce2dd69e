"""Per-call parity of the HIP path against the CPU oracle (MI355X only).

Integer results (trees, top-k ids, verification, M, committed rows) must
match bit for bit.  Attention must match the float64 oracle within 1e-5
relative per output row (float32 inputs; max |diff| / max |oracle| over the
row) and within 2e-2 absolute per element (bfloat16 inputs).
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import tr_oracle as O

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module")
def tr():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from draft_tree_retrieval_amd import tr as _tr
    _tr.load()
    return _tr


def ws_for(tr, tree, B, V=0, k=0, Hq=0, Hkv=0, cap=0):
    return tr.new_workspace(tree, B, V, k, Hq, Hkv, 128 if Hq else 0, cap, device=DEV)


def otree(levels):
    return O.template_from_levels(levels)


RAND_LEVELS = [[[3], [2, 1]], [[4], [4, 2, 1, 1], [2, 1]], [[1]] * 9, [],
               [[8], [6, 4, 3, 2, 2, 1, 1, 1], [5, 4, 3, 2, 2, 2, 1, 1, 1, 1],
                [4, 3, 2, 2, 2, 1, 1, 1, 1, 1], [3, 2, 2, 1, 1, 1], [2]]]


# ------------------------------------------------------------------ worked example
def test_worked_example_through_abi(tr):
    with open(os.path.join(os.path.dirname(__file__), "golden", "worked_example.json")) as f:
        ex = json.load(f)
    ids = {n: i for i, n in enumerate(ex["vocab"])}
    V, k = len(ex["vocab"]), ex["k"]
    M = torch.full((1, V, k), ids["pad"], dtype=torch.int64)
    for name, row in ex["M_pre"].items():
        M[0, ids[name]] = torch.tensor([ids[x] for x in row])
    logits = torch.zeros((1, 7, V), dtype=torch.float32)
    for n, row in enumerate(ex["logits"]):
        for name, val in row.items():
            logits[0, n, ids[name]] = val
    tree = tr.Tree.from_levels(ex["levels"], k)
    ws = ws_for(tr, tree, 1, V, k)
    M_d, root = M.to(DEV), torch.tensor([ids[ex["root"]]], dtype=torch.int32, device=DEV)
    tok = torch.empty((1, 7), dtype=torch.int32, device=DEV)
    tr.tr_retrieve(tree, M_d, root, tok, ws)
    assert [ex["vocab"][x] for x in tok[0].tolist()] == ex["merged_sequence"]
    # verify through the stand-alone calls
    topk = torch.empty((1, 7, k), dtype=torch.int32, device=DEV)
    tr.tr_update_topk(tree, logits.to(DEV), None, None, topk, ws)
    L = torch.empty((1,), dtype=torch.int32, device=DEV)
    path = torch.empty((1, 3), dtype=torch.int32, device=DEV)
    bonus = torch.empty((1,), dtype=torch.int32, device=DEV)
    emitted = torch.empty((1, 3), dtype=torch.int32, device=DEV)
    tr.tr_verify(tree, topk, tok, L, path, bonus, emitted)
    e = ex["expected"]
    assert int(L[0]) == e["accept_len"] and path[0].tolist() == e["path"]
    assert ex["vocab"][int(bonus[0])] == e["bonus"]
    assert [ex["vocab"][x] for x in emitted[0].tolist()] == e["emitted"]
    # and through the fused step
    tree_tok, root2 = tok.clone(), root.clone()
    tr.tr_step(tree, logits.to(DEV), M_d, tree_tok, root2, L, path, emitted, ws)
    Mh = M_d.cpu()[0]
    for name, row in e["M_post"].items():
        assert [ex["vocab"][x] for x in Mh[ids[name]].tolist()] == row
    assert ex["vocab"][int(root2[0])] == e["next_root"]
    assert [ex["vocab"][x] for x in tree_tok[0].tolist()] == e["next_tree"]
    assert tr.tr_read_device_status(ws) == 0


# ------------------------------------------------------------------ retrieval
@pytest.mark.parametrize("m_dtype", [torch.int32, torch.int64])
def test_retrieve_parity(tr, m_dtype):
    g = torch.Generator().manual_seed(1)
    for levels in RAND_LEVELS:
        t = otree(levels)
        for V, k, B in ((7, 8, 3), (1000, 8, 5), (32000, 8, 2)):
            tree = tr.Tree.from_levels(levels, k)
            M = torch.randint(0, V, (B, V, k), generator=g).to(m_dtype)
            root = torch.randint(0, V, (B,), generator=g).to(torch.int32)
            ws = ws_for(tr, tree, B)
            tok = torch.empty((B, t.n_nodes), dtype=torch.int32, device=DEV)
            tr.tr_retrieve(tree, M.to(DEV), root.to(DEV), tok, ws)
            got = tok.cpu().numpy()
            for b in range(B):
                assert (got[b] == O.retrieve(t, M[b].numpy(), int(root[b]))).all()
            assert tr.tr_read_device_status(ws) == 0


def test_retrieve_flags_bad_root(tr):
    tree = tr.Tree.from_levels([[2], [1]], 2)
    ws = ws_for(tr, tree, 1)
    M = torch.zeros((1, 10, 2), dtype=torch.int32, device=DEV)
    tok = torch.empty((1, 4), dtype=torch.int32, device=DEV)
    tr.tr_retrieve(tree, M, torch.tensor([12], dtype=torch.int32, device=DEV), tok, ws)
    assert tr.tr_read_device_status(ws) & tr.TR_FLAG_BAD_TOKEN
    assert tok[0, 1:].tolist() == [-1, -1, -1]
    assert tr.tr_read_device_status(ws) == 0          # reading clears the word


# ------------------------------------------------------------------ top-k
def topk_cases():
    g = torch.Generator().manual_seed(2)
    cases = []
    # heavy ties: values from a tiny set; signed zeros; infinities
    z = (torch.randint(-3, 4, (9, 5003), generator=g).float() * 0.5)
    z[0, ::7] = -0.0
    z[1, 100] = math.inf
    z[2, :] = -math.inf
    z[2, 4000] = 0.0
    z[3, :] = 0.0
    z[3, 17] = -0.0
    cases.append(("ties_f32", z))
    cases.append(("ties_bf16", z.to(torch.bfloat16)))
    cases.append(("normal_bf16_32000", (torch.randn((81, 32000), generator=g) * 3).to(torch.bfloat16)))
    cases.append(("normal_f32_odd", torch.randn((17, 32003), generator=g) * 2))
    cases.append(("normal_bf16_odd", (torch.randn((5, 1037), generator=g) * 3).to(torch.bfloat16)))
    cases.append(("large_vocab", (torch.randn((3, 128256), generator=g) * 3).to(torch.bfloat16)))
    cases.append(("tiny_vocab", torch.randn((6, 16), generator=g)))
    return cases


@pytest.mark.parametrize("k", [1, 3, 8, 16])
def test_topk_parity(tr, k):
    for name, z in topk_cases():
        rows, V = z.shape
        if V < k:
            continue
        tree = tr.Tree.from_levels([[1]] * (rows - 1), k)       # chain: rows nodes, B = 1
        ws = ws_for(tr, tree, 1, V, k)
        out = torch.empty((1, rows, k), dtype=torch.int32, device=DEV)
        tr.tr_update_topk(tree, z[None].to(DEV), None, None, out, ws)
        want = O.topk_rows(z.float().numpy(), k)
        got = out[0].cpu().numpy()
        bad = np.flatnonzero((got != want).any(axis=1))
        assert len(bad) == 0, f"{name} k={k}: rows {bad[:5]} got {got[bad[0]]} want {want[bad[0]]}"


def test_topk_unaligned_rows(tr):
    # rows start at odd element offsets: a sliced view of a wider tensor
    g = torch.Generator().manual_seed(3)
    base = (torch.randn((4, 2 * 4001 + 3), generator=g) * 3).to(torch.bfloat16).to(DEV)
    z = base.view(-1)[1: 1 + 8 * 4001].view(1, 8, 4001)           # odd element offset
    tree = tr.Tree.from_levels([[1]] * 7, 8)
    ws = ws_for(tr, tree, 1, 4001, 8)
    out = torch.empty((1, 8, 8), dtype=torch.int32, device=DEV)
    tr.tr_update_topk(tree, z, None, None, out, ws)
    want = O.topk_rows(z[0].float().cpu().numpy(), 8)
    assert (out[0].cpu().numpy() == want).all()


@pytest.mark.parametrize("dtype,V,k,rows", [(torch.float32, 524288, 8, 3),
                                             (torch.bfloat16, 1048576, 8, 3),
                                             (torch.bfloat16, 524288, 16, 2),
                                             (torch.float32, 262144, 16, 300)])
def test_topk_at_row_limit(tr, dtype, V, k, rows):
    # the longest rows the plan holds (one row per block and many rows per
    # launch): the best values sit in the last elements of each row, where a
    # segment that dropped its tail would miss them; a tie at the very end
    # goes to the lower id
    g = torch.Generator().manual_seed(V + k)
    z = (torch.randn((rows, V), generator=g) * 3).to(dtype)
    for r in range(rows):
        z[r, V - 1] = 100.0
        z[r, V - 3] = 90.0
        z[r, V - 2] = 90.0
        z[r, (r * 7919) % (V // 2)] = 95.0
    T = min(rows, 100)                              # B sequences of a T-node chain
    B = rows // T
    tree = tr.Tree.from_levels([[1]] * (T - 1), k)
    ws = ws_for(tr, tree, B, V, k)
    out = torch.empty((B, T, k), dtype=torch.int32, device=DEV)
    tr.tr_update_topk(tree, z.view(B, T, V).to(DEV), None, None, out, ws)
    want = O.topk_rows(z.float().numpy(), k)
    got = out.view(rows, k).cpu().numpy()
    assert (got == want).all()
    assert (got[:, 0] == V - 1).all() and (got[:, 2] == V - 3).all() and (got[:, 3] == V - 2).all()


# ------------------------------------------------------------------ verify + update
def test_verify_parity_duplicates(tr):
    rng = np.random.default_rng(4)
    for levels in RAND_LEVELS:
        t = otree(levels)
        tree = tr.Tree.from_levels(levels, 8)
        B = 16
        tok = rng.integers(0, 4, size=(B, t.n_nodes)).astype(np.int32)   # many duplicates
        top = rng.integers(0, 4, size=(B, t.n_nodes, 8)).astype(np.int32)
        W = t.max_depth + 1
        L = torch.empty((B,), dtype=torch.int32, device=DEV)
        path = torch.empty((B, W), dtype=torch.int32, device=DEV)
        bonus = torch.empty((B,), dtype=torch.int32, device=DEV)
        em = torch.empty((B, W), dtype=torch.int32, device=DEV)
        tr.tr_verify(tree, torch.from_numpy(top).to(DEV), torch.from_numpy(tok).to(DEV), L, path,
                     bonus, em)
        for b in range(B):
            v = O.verify(t, tok[b].astype(np.int64), top[b, :, 0].astype(np.int64))
            assert int(L[b]) == v.accept_len and int(bonus[b]) == v.bonus
            assert path[b].tolist() == v.path.tolist() + [-1] * (W - len(v.path))
            assert em[b].tolist() == v.emitted.tolist() + [-1] * (W - len(v.emitted))


@pytest.mark.parametrize("m_dtype", [torch.int32, torch.int64])
def test_update_parity_duplicate_rows(tr, m_dtype):
    rng = np.random.default_rng(5)
    levels = RAND_LEVELS[4]
    t = otree(levels)
    tree = tr.Tree.from_levels(levels, 8)
    B, V = 3, 50
    tok = rng.integers(0, 12, size=(B, t.n_nodes)).astype(np.int32)     # tokens repeat often
    z = torch.from_numpy(rng.standard_normal((B, t.n_nodes, V)).astype(np.float32))
    M0 = torch.from_numpy(rng.integers(0, V, size=(B, V, 8))).to(m_dtype)
    Md = M0.to(DEV)
    ws = ws_for(tr, tree, B, V, 8)
    tr.tr_update_topk(tree, z.to(DEV), torch.from_numpy(tok).to(DEV), Md, None, ws)
    for b in range(B):
        Mo = M0[b].numpy().astype(np.int64).copy()
        O.update(Mo, tok[b], O.topk_rows(z[b].numpy(), 8))
        assert (Md[b].cpu().numpy() == Mo).all()


@pytest.mark.parametrize("k,m_dtype", [(3, torch.int32), (16, torch.int64)])
def test_update_long_rows_segments(tr, k, m_dtype):
    # rows longer than one block holds: each row's segments meet in the
    # per-sequence merge launch, which then runs the update (tie-prone bf16
    # rows, tokens that repeat, k = 3 and the 16-key lists)
    rng = np.random.default_rng(40 + k)
    levels = RAND_LEVELS[4] if k >= 8 else [[1]] * 80      # 81 nodes either way
    t = otree(levels)
    tree = tr.Tree.from_levels(levels, k)
    B, V = 2, 128256
    g = torch.Generator().manual_seed(41 + k)
    z = (torch.randn((B, t.n_nodes, V), generator=g) * 3).to(torch.bfloat16)
    tok = rng.integers(0, 40, size=(B, t.n_nodes)).astype(np.int32)
    M0 = torch.from_numpy(rng.integers(0, V, size=(B, V, k))).to(m_dtype)
    Md = M0.to(DEV)
    out = torch.empty((B, t.n_nodes, k), dtype=torch.int32, device=DEV)
    ws = ws_for(tr, tree, B, V, k)
    tr.tr_update_topk(tree, z.to(DEV), torch.from_numpy(tok).to(DEV), Md, out, ws)
    assert tr.tr_read_device_status(ws) == 0
    for b in range(B):
        want = O.topk_rows(z[b].float().numpy(), k)
        assert (out[b].cpu().numpy() == want).all(), b
        Mo = M0[b].numpy().astype(np.int64).copy()
        O.update(Mo, tok[b], want)
        assert (Md[b].cpu().numpy().astype(np.int64) == Mo).all(), b


def test_step_long_rows_k16(tr):
    # the greedy step with 16-key segment lists at a long vocabulary: top-k,
    # verdict, M and the next tree against the oracle
    rng = np.random.default_rng(77)
    levels = RAND_LEVELS[4]
    t = otree(levels)
    k, B, V = 16, 2, 128256
    tree = tr.Tree.from_levels(levels, k)
    M = torch.from_numpy(rng.integers(0, V, size=(B, V, k))).to(torch.int32)
    root = torch.from_numpy(rng.integers(0, V, size=(B,))).to(torch.int32)
    ws = ws_for(tr, tree, B, V, k)
    dM, droot = M.to(DEV), root.to(DEV)
    tok = torch.empty((B, t.n_nodes), dtype=torch.int32, device=DEV)
    tr.tr_retrieve(tree, dM, droot, tok, ws)
    tok_h = tok.cpu().numpy().astype(np.int64)
    g = torch.Generator().manual_seed(78)
    z = torch.randn((B, t.n_nodes, V), generator=g) * 3
    for b in range(B):                                  # accept along random edges
        for n in range(1, t.n_nodes):
            if rng.random() < 0.6:
                z[b, t.parent[n], tok_h[b, n]] = 40.0 + float(rng.random())
    z = z.to(torch.bfloat16)
    L = torch.empty((B,), dtype=torch.int32, device=DEV)
    path = torch.empty((B, t.max_depth + 1), dtype=torch.int32, device=DEV)
    em = torch.empty((B, t.max_depth + 1), dtype=torch.int32, device=DEV)
    topk = torch.empty((B, t.n_nodes, k), dtype=torch.int32, device=DEV)
    tr.tr_step(tree, z.to(DEV), dM, tok, droot, L, path, em, ws, topk_out=topk)
    assert tr.tr_read_device_status(ws) == 0
    lengths = []
    for b in range(B):
        Mo = M[b].numpy().astype(np.int64).copy()
        res, _ = O.step_after_forward(t, Mo, tok_h[b], z[b].float().numpy(), k)
        v = res.verdict
        assert (topk[b].cpu().numpy() == res.topk).all(), b
        assert int(L[b]) == v.accept_len and int(droot[b]) == v.bonus
        assert path[b, :v.accept_len + 1].cpu().tolist() == v.path.tolist()
        assert (dM[b].cpu().numpy().astype(np.int64) == Mo).all(), b
        assert tok[b].cpu().numpy().tolist() == res.next_tok.tolist()
        lengths.append(v.accept_len)
    assert max(lengths) >= 2                            # the plants were accepted


# ------------------------------------------------------------------ attention
def attn_inputs(g, B, T, Hq, Hkv, P, cap, dtype):
    q = torch.randn((B, T, Hq, 128), generator=g).to(dtype)
    kt = torch.randn((B, T, Hkv, 128), generator=g).to(dtype)
    vt = torch.randn((B, T, Hkv, 128), generator=g).to(dtype)
    kc = torch.randn((B, Hkv, cap, 128), generator=g).to(dtype)
    vc = torch.randn((B, Hkv, cap, 128), generator=g).to(dtype)
    return q, kt, vt, kc, vc


def check_attn(t, got, q, kt, vt, kc, vc, P, dtype, rows=None):
    B = q.shape[0]
    for b in range(B):
        want = O.tree_attention(t, q[b].double().numpy(), kt[b].double().numpy(), vt[b].double().numpy(),
                                kc[b].double().numpy(), vc[b].double().numpy(), int(P[b]))
        gb = got[b].double().numpy()
        if dtype == torch.float32:
            num = np.abs(gb - want).max(axis=-1)
            den = np.maximum(np.abs(want).max(axis=-1), 1e-30)
            assert (num / den).max() <= 1e-5, (num / den).max()
        else:
            assert np.abs(gb - want).max() <= 2e-2, np.abs(gb - want).max()


ATTN_CASES = [
    # levels, B, Hq, Hkv, P list, cap
    (RAND_LEVELS[1], 1, 8, 8, [256], 300),
    (RAND_LEVELS[0], 2, 4, 2, [0, 5], 70),
    (RAND_LEVELS[4], 1, 32, 32, [1000], 1100),
    (RAND_LEVELS[4], 3, 16, 2, [63, 700, 1], 800),
    (RAND_LEVELS[2], 2, 8, 8, [130, 64], 200),
    (RAND_LEVELS[3], 2, 8, 1, [77, 3000], 3100),
    (RAND_LEVELS[4], 1, 64, 8, [1500], 1600),
    # 64 x 4 (sequence, kv head) pairs fill 256 blocks with one chunk each:
    # the bf16 plan still splits the keys in two so the prefix pass takes
    # the tree keys; ragged prefixes, 0 and the full capacity among them
    (RAND_LEVELS[2], 64, 8, 4, [0, 300] + [(37 * i) % 301 for i in range(62)], 300),
]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("case", range(len(ATTN_CASES)))
def test_tree_attention_parity(tr, dtype, case):
    levels, B, Hq, Hkv, Ps, cap = ATTN_CASES[case]
    t = otree(levels)
    tree = tr.Tree.from_levels(levels, 8)
    g = torch.Generator().manual_seed(100 + case)
    q, kt, vt, kc, vc = attn_inputs(g, B, t.n_nodes, Hq, Hkv, max(Ps), cap, dtype)
    P = torch.tensor(Ps, dtype=torch.int32)
    ws = ws_for(tr, tree, B, Hq=Hq, Hkv=Hkv, cap=cap)
    out = torch.empty_like(q, device=DEV)
    tr.tr_tree_attn(tree, q.to(DEV), kt.to(DEV), vt.to(DEV), kc.to(DEV), vc.to(DEV), P.to(DEV), out, ws)
    check_attn(t, out.cpu(), q, kt, vt, kc, vc, P, dtype)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_attention_siblings_and_determinism(tr, dtype):
    levels = RAND_LEVELS[4]
    t = otree(levels)
    tree = tr.Tree.from_levels(levels, 8)
    g = torch.Generator().manual_seed(7)
    q, kt, vt, kc, vc = [x.to(DEV) for x in attn_inputs(g, 1, t.n_nodes, 16, 4, 900, 1000, dtype)]
    P = torch.tensor([900], dtype=torch.int32, device=DEV)
    ws = ws_for(tr, tree, 1, Hq=16, Hkv=4, cap=1000)
    base = torch.empty_like(q)
    tr.tr_tree_attn(tree, q, kt, vt, kc, vc, P, base, ws)
    again = torch.empty_like(q)
    tr.tr_tree_attn(tree, q, kt, vt, kc, vc, P, again, ws)
    assert torch.equal(base.view(torch.int16) if dtype == torch.bfloat16 else base.view(torch.int32),
                       again.view(torch.int16) if dtype == torch.bfloat16 else again.view(torch.int32))
    mask = O.ancestor_mask(t)
    for j in (1, 9, 40, 80):
        kt2, vt2 = kt.clone(), vt.clone()
        kt2[0, j] += 3.0
        vt2[0, j] -= 2.0
        out = torch.empty_like(q)
        tr.tr_tree_attn(tree, q, kt2, vt2, kc, vc, P, out, ws)
        changed = []
        for n in range(t.n_nodes):
            same = torch.equal(out[0, n], base[0, n])
            if not mask[n, j]:
                assert same, (j, n)             # a non-ancestor never matters, bit for bit
            else:
                changed.append(not same)
        # an ancestor's key/value always moves the fp32 result; bf16 rounding may hide a few
        assert all(changed) if dtype == torch.float32 else np.mean(changed) >= 0.9


# ------------------------------------------------------------------ accepted-only update
@pytest.mark.parametrize("m_dtype", [torch.int32, torch.int64])
def test_step_ex_accepted_only_duplicates(tr, m_dtype):
    # Tiny vocabularies: tokens repeat along the accepted path and off it, so
    # a node off the path often carries a path token with a higher index
    # (the all-nodes update would let it win; this one must not).
    g = torch.Generator().manual_seed(21)
    rng = np.random.default_rng(21)
    for levels in RAND_LEVELS:
        t = otree(levels)
        T, D = t.n_nodes, t.max_depth
        widest = max((max(l) for l in levels), default=0)
        # k = 16: the 16-wide tail (row prefetch of 16 ids per node)
        for V, k, B in ((5, 3, 4), (9, 8, 3), (300, 8, 2), (40, 16, 2)):
            if k < widest:
                continue
            tree = tr.Tree.from_levels(levels, k)
            M = torch.randint(0, V, (B, V, k), generator=g).to(m_dtype)
            root = torch.randint(0, V, (B,), generator=g).to(torch.int32)
            ws = ws_for(tr, tree, B, V, k)
            dM, droot = M.to(DEV), root.to(DEV)
            tok = torch.empty((B, T), dtype=torch.int32, device=DEV)
            tr.tr_retrieve(tree, dM, droot, tok, ws)
            tok_h = tok.cpu().numpy().astype(np.int64)
            z = torch.randn((B, T, V), generator=g)
            for b in range(B):                      # plant acceptance on most edges
                for n in range(1, T):
                    if rng.random() < 0.8:
                        z[b, t.parent[n], tok_h[b, n]] = 20.0 + float(rng.random())
            L = torch.empty((B,), dtype=torch.int32, device=DEV)
            path = torch.empty((B, D + 1), dtype=torch.int32, device=DEV)
            em = torch.empty((B, D + 1), dtype=torch.int32, device=DEV)
            tr.tr_step_ex(tree, z.to(DEV), dM, tok, droot, L, path, em, ws, update="accepted")
            for b in range(B):
                Mo = M[b].numpy().astype(np.int64).copy()
                res, _ = O.step_after_forward(t, Mo, tok_h[b], z[b].numpy(), k,
                                              update_mode="accepted")
                assert (dM[b].cpu().numpy().astype(np.int64) == Mo).all(), (levels, V, b)
                assert int(L[b]) == res.verdict.accept_len
                assert path[b, :res.verdict.accept_len + 1].cpu().tolist() == res.verdict.path.tolist()
                assert tok[b].cpu().numpy().tolist() == res.next_tok.tolist()
                assert int(droot[b]) == res.verdict.bonus
            assert tr.tr_read_device_status(ws) == 0


# ------------------------------------------------------------------ sampling verification
MARGIN = 2e-5      # a uniform this close to a threshold could go either way in float32


def clear_uniforms(t, M, tok, z, k, temp, g, update="all"):
    """Uniforms [T][2] whose every decision clears its threshold by MARGIN
    in the oracle, and the oracle's step result on them."""
    for _ in range(50):
        u = torch.rand((t.n_nodes, 2), generator=g, dtype=torch.float64).to(torch.float32)
        Mo = M.copy()
        res, _ = O.step_after_forward(t, Mo, tok, z, k, update_mode=update, temperature=temp,
                                      uniforms=u.double().numpy())
        if res.verdict.margin > MARGIN:
            return u, res, Mo
    raise AssertionError("no clear uniforms")


@pytest.mark.parametrize("l_dtype", [torch.bfloat16, torch.float32])
def test_step_sample_parity(tr, l_dtype):
    g = torch.Generator().manual_seed(51)
    rng = np.random.default_rng(51)
    lengths = []
    for li, levels in enumerate(RAND_LEVELS):
        t = otree(levels)
        T, D = t.n_nodes, t.max_depth
        for V, B, temp in ((300, 3, 1.0), (32000, 2, 0.7), (1001, 2, 1.6)):
            k = 8
            tree = tr.Tree.from_levels(levels, k)
            M = torch.randint(0, V, (B, V, k), generator=g, dtype=torch.int32)
            root = torch.randint(0, V, (B,), generator=g).to(torch.int32)
            ws = ws_for(tr, tree, B, V, k)
            dM, droot = M.to(DEV), root.to(DEV)
            tok = torch.empty((B, T), dtype=torch.int32, device=DEV)
            tr.tr_retrieve(tree, dM, droot, tok, ws)
            tok_h = tok.cpu().numpy().astype(np.int64)
            z = torch.randn((B, T, V), generator=g) * 2.0
            for b in range(B):                      # deep paths: boost most drafts
                for n in range(1, T):
                    if rng.random() < 0.7:
                        z[b, t.parent[n], tok_h[b, n]] += 10.0
            z = z.to(l_dtype)
            zh = z.float().numpy()
            us, want = [], []
            for b in range(B):
                u, res, Mo = clear_uniforms(t, M[b].numpy().astype(np.int64), tok_h[b], zh[b], k,
                                            temp, g)
                us.append(u)
                want.append((res, Mo))
            U = torch.stack(us).to(DEV)
            L = torch.empty((B,), dtype=torch.int32, device=DEV)
            path = torch.empty((B, D + 1), dtype=torch.int32, device=DEV)
            em = torch.empty((B, D + 1), dtype=torch.int32, device=DEV)
            topk = torch.empty((B, T, k), dtype=torch.int32, device=DEV)
            tr.tr_step_sample(tree, z.to(DEV), temp, U, dM, tok, droot, L, path, em, ws,
                              topk_out=topk)
            for b, (res, Mo) in enumerate(want):
                v = res.verdict
                case = (li, V, b)
                assert int(L[b]) == v.accept_len, case
                assert path[b, :v.accept_len + 1].cpu().tolist() == v.path.tolist(), case
                assert int(droot[b]) == v.bonus, case
                emw = v.emitted.tolist() + [-1] * (D + 1 - len(v.emitted))
                assert em[b].cpu().tolist() == emw, case
                assert (topk[b].cpu().numpy() == res.topk).all(), case
                assert (dM[b].cpu().numpy().astype(np.int64) == Mo).all(), case
                assert tok[b].cpu().numpy().tolist() == res.next_tok.tolist(), case
                lengths.append(v.accept_len)
            assert tr.tr_read_device_status(ws) == 0
    # the cases reach past the first layer and also stop at the root
    assert max(lengths) >= 3 and min(lengths) == 0


def test_step_sample_draw_covers_the_row(tr):
    # one node (a leaf root): the bonus is the inverse-CDF draw from p_root;
    # uniforms spread over [0, 1) reach ids all over the row, and each
    # matches the oracle's draw
    g = torch.Generator().manual_seed(52)
    tree = tr.Tree.from_levels([], 8)
    t = otree([])
    V, B, temp = 5000, 64, 3.0
    z = (torch.randn((1, 1, V), generator=g) * 0.5).to(torch.bfloat16).repeat(B, 1, 1)
    zh = z.float().numpy()
    M = torch.zeros((B, V, 8), dtype=torch.int32)
    ws = ws_for(tr, tree, B, V, 8)
    us = []
    for b in range(B):
        while True:
            u = torch.tensor([[0.0, (b + float(torch.rand((), generator=g))) / B]])
            v = O.verify_sample(t, np.zeros(1, dtype=np.int64), zh[b], temp, u.double().numpy())
            if v.margin > MARGIN:
                break
        us.append((u, v.bonus))
    U = torch.stack([u for u, _ in us]).to(DEV)
    tok = torch.zeros((B, 1), dtype=torch.int32, device=DEV)
    root = torch.zeros((B,), dtype=torch.int32, device=DEV)
    L = torch.empty((B,), dtype=torch.int32, device=DEV)
    path = torch.empty((B, 1), dtype=torch.int32, device=DEV)
    em = torch.empty((B, 1), dtype=torch.int32, device=DEV)
    tr.tr_step_sample(tree, z.to(DEV), temp, U, M.to(DEV), tok, root, L, path, em, ws)
    got = root.cpu().tolist()
    assert got == [bonus for _, bonus in us]
    assert got == sorted(got) and got[-1] - got[0] > V // 2   # increasing uniforms, increasing ids


# ------------------------------------------------------------------ paged cache
def paged_from_contiguous(g, kc, ps, spare=3, layers=1):
    """Pools [layers][num_pages][Hkv][ps][d] holding the contiguous caches kc
    [layers][B][Hkv][cap][d] in shuffled pages (junk in the spare pages) and
    the block table [B][cap / ps]."""
    L, B, Hkv, cap, d = kc.shape
    mp = cap // ps
    n = B * mp + spare
    perm = torch.randperm(n, generator=g)
    table = perm[:B * mp].reshape(B, mp).to(torch.int32)
    pool = (torch.randn((L, n, Hkv, ps, d), generator=g) * 50).to(kc.dtype)
    for b in range(B):
        for j in range(mp):
            pool[:, table[b, j]] = kc[:, b, :, j * ps:(j + 1) * ps]
    return pool, table


@pytest.mark.parametrize("ps", [64, 128])
def test_paged_attention_parity(tr, ps):
    g = torch.Generator().manual_seed(71)
    levels = RAND_LEVELS[1]
    t = otree(levels)
    tree = tr.Tree.from_levels(levels, 8)
    B, Hq, Hkv, d, cap = 2, 8, 4, 128, 512
    P = torch.tensor([200, 391], dtype=torch.int32)
    mk = lambda *sh: torch.randn(sh, generator=g).to(torch.bfloat16)
    q, kt, vt = mk(B, t.n_nodes, Hq, d), mk(1, B, t.n_nodes, Hkv, d), mk(1, B, t.n_nodes, Hkv, d)
    kc, vc = mk(1, B, Hkv, cap, d), mk(1, B, Hkv, cap, d)
    kp, table = paged_from_contiguous(g, kc, ps)
    vp = torch.empty_like(kp)
    for b in range(B):
        for j in range(cap // ps):
            vp[:, table[b, j]] = vc[:, b, :, j * ps:(j + 1) * ps]
    D = [x.to(DEV) for x in (q, kt, vt, kc, vc, kp, vp, table, P)]
    dq, dkt, dvt, dkc, dvc, dkp, dvp, dtab, dP = D
    ws = ws_for(tr, tree, B, 0, 0, Hq, Hkv, cap)
    kv = tr.PagedKV(dkp, dvp, dtab, dkt, dvt, dP)
    out_p = torch.empty_like(dq)
    tr.tr_tree_attn_paged(tree, dq, kv, 0, out_p, ws)
    out_c = torch.empty_like(dq)
    tr.tr_tree_attn(tree, dq, dkt[0], dvt[0], dkc[0], dvc[0], dP, out_c, ws)
    assert torch.equal(out_p, out_c)                 # the same arithmetic in the same order
    for b in range(B):
        want = O.tree_attention_paged(t, q[b].float().numpy(), kt[0, b].float().numpy(),
                                      vt[0, b].float().numpy(), kp[0].float().numpy(),
                                      vp[0].float().numpy(), table[b].numpy(), ps, int(P[b]))
        assert np.abs(out_p[b].float().cpu().numpy() - want).max() <= 2e-2
    assert tr.tr_read_device_status(ws) == 0
    # a page id outside the pool reads page 0 and raises the flag
    bad = dtab.clone()
    bad[1, 2] = kp.shape[1] + 5
    kv_bad = tr.PagedKV(dkp, dvp, bad, dkt, dvt, dP)
    tr.tr_tree_attn_paged(tree, dq, kv_bad, 0, out_p, ws)
    assert tr.tr_read_device_status(ws) & tr.TR_FLAG_BAD_PAGE


@pytest.mark.parametrize("ps", [64, 256])
def test_paged_attention_later_layers(tr, ps):
    # a model's cache of 4 layers in shared page pools; attention at layer 1
    # and at the last layer reads that layer's pages and tree rows only
    # (every layer's data differs), checked against the oracle's paged
    # attention on that layer's pool and bit for bit against the contiguous
    # call on that layer's slices
    g = torch.Generator().manual_seed(73)
    levels = RAND_LEVELS[4]
    t = otree(levels)
    tree = tr.Tree.from_levels(levels, 8)
    L, B, Hq, Hkv, d, cap = 4, 3, 16, 4, 128, 1024
    P = torch.tensor([1000, 0, 517], dtype=torch.int32)
    mk = lambda *sh: torch.randn(sh, generator=g).to(torch.bfloat16)
    kt, vt = mk(L, B, t.n_nodes, Hkv, d), mk(L, B, t.n_nodes, Hkv, d)
    kc, vc = mk(L, B, Hkv, cap, d), mk(L, B, Hkv, cap, d)
    kp, table = paged_from_contiguous(g, kc, ps, layers=L)
    vp = torch.empty_like(kp)
    for b in range(B):
        for j in range(cap // ps):
            vp[:, table[b, j]] = vc[:, b, :, j * ps:(j + 1) * ps]
    dkt, dvt, dkc, dvc, dkp, dvp, dtab, dP = (x.to(DEV) for x in (kt, vt, kc, vc, kp, vp, table, P))
    ws = ws_for(tr, tree, B, 0, 0, Hq, Hkv, cap)
    kv = tr.PagedKV(dkp, dvp, dtab, dkt, dvt, dP)
    for layer in (1, L - 1):
        q = mk(B, t.n_nodes, Hq, d)
        dq = q.to(DEV)
        out_p = torch.empty_like(dq)
        tr.tr_tree_attn_paged(tree, dq, kv, layer, out_p, ws)
        out_c = torch.empty_like(dq)
        tr.tr_tree_attn(tree, dq, dkt[layer], dvt[layer], dkc[layer], dvc[layer], dP, out_c, ws)
        assert torch.equal(out_p, out_c), layer
        for b in range(B):
            want = O.tree_attention_paged(t, q[b].float().numpy(), kt[layer, b].float().numpy(),
                                          vt[layer, b].float().numpy(), kp[layer].float().numpy(),
                                          vp[layer].float().numpy(), table[b].numpy(), ps, int(P[b]))
            assert np.abs(out_p[b].float().cpu().numpy() - want).max() <= 2e-2, (layer, b)
    assert tr.tr_read_device_status(ws) == 0


def test_step_paged_commits_every_layer(tr):
    g = torch.Generator().manual_seed(72)
    levels = RAND_LEVELS[1]
    t = otree(levels)
    tree = tr.Tree.from_levels(levels, 8)
    T, D = t.n_nodes, t.max_depth
    V, B, Hkv, d, ps, L = 300, 3, 2, 128, 64, 3
    mp = 3                                          # capacity 192 positions
    M = torch.randint(0, V, (B, V, 8), generator=g, dtype=torch.int32)
    root = torch.tensor([3, 4, 5], dtype=torch.int32)
    P = torch.tensor([5, 62, 189], dtype=torch.int32)   # seq 1 crosses a page, seq 2 overflows
    kc = torch.zeros((L, B, Hkv, mp * ps, d), dtype=torch.bfloat16)
    kp, table = paged_from_contiguous(g, kc, ps, layers=L)
    vp = kp.clone()
    kt = torch.randn((L, B, T, Hkv, d), generator=g).to(torch.bfloat16)
    vt = torch.randn((L, B, T, Hkv, d), generator=g).to(torch.bfloat16)
    ws = ws_for(tr, tree, B, V, 8)
    dM, droot, dP, dkp, dvp, dtab, dkt, dvt = (x.to(DEV) for x in (M, root, P, kp, vp, table, kt, vt))
    tok = torch.empty((B, T), dtype=torch.int32, device=DEV)
    tr.tr_retrieve(tree, dM, droot, tok, ws)
    tok_h = tok.cpu().numpy().astype(np.int64)
    z = torch.randn((B, T, V), generator=g)
    for b in range(B):                              # accept the rank-0 chain 0 -> 1 -> 5 -> 13
        for a, c in ((0, 1), (1, 5), (5, 13)):
            z[b, a, tok_h[b, c]] = 50.0
    Ld = torch.empty((B,), dtype=torch.int32, device=DEV)
    path = torch.empty((B, D + 1), dtype=torch.int32, device=DEV)
    em = torch.empty((B, D + 1), dtype=torch.int32, device=DEV)
    kv = tr.PagedKV(dkp, dvp, dtab, dkt, dvt, dP)
    tr.tr_step_paged(tree, z.to(DEV), dM, tok, droot, Ld, path, em, ws, kv)
    flags = tr.tr_read_device_status(ws)
    assert flags & tr.TR_FLAG_CACHE_FULL            # seq 2: 189 + 4 > 192
    okp, ovp = kp.float().numpy(), vp.float().numpy()
    for b in range(B):
        Mo = M[b].numpy().astype(np.int64).copy()
        res, _ = O.step_after_forward(t, Mo, tok_h[b], z[b].numpy(), 8)
        assert int(Ld[b]) == res.verdict.accept_len == 3
        assert (dM[b].cpu().numpy() == Mo).all()
        assert tok[b].cpu().numpy().tolist() == res.next_tok.tolist()
        if b < 2:
            newP = O.commit_paged(okp, ovp, kt[:, b].float().numpy(), vt[:, b].float().numpy(),
                                  table[b].numpy(), ps, int(P[b]), res.verdict.path)
            assert int(dP[b]) == newP
        else:
            assert int(dP[b]) == int(P[b])
    assert (dkp.float().cpu().numpy() == okp).all() and (dvp.float().cpu().numpy() == ovp).all()


# ------------------------------------------------------------------ fused LM head
def lmhead_tol(H):
    # twice a worst-case float32 accumulation bound for a length-H dot product
    # of N(0,1) bf16 entries: (H/32 + 8) roundings (32-term MFMA products,
    # then one accumulation per k step) of at most eps * sum|h w|, with
    # sum|h w| ~ 0.64 H
    return 2 * 6e-8 * (H / 32 + 8) * 0.64 * H


def check_lmhead_rows(z, ids, k, tol):
    """z [rows][V] float64 oracle logits, ids [rows][k] from the GPU: rows
    whose k+1 best are separated by more than tol must match exactly (value
    descending, ties to the lower id); the others must be a valid top-k
    within tol.  Returns the number of rows checked exactly."""
    exact = 0
    for r in range(z.shape[0]):
        order = np.lexsort((np.arange(z.shape[1]), -z[r]))
        top = z[r][order[:k + 1]]
        if len(top) <= k or (np.diff(-top) > tol).all():
            assert ids[r].tolist() == order[:k].tolist(), r
            exact += 1
        else:
            got = z[r][ids[r]]
            assert len(set(ids[r].tolist())) == k
            assert (got >= z[r][order[k - 1]] - tol).all() and (np.diff(got) <= tol).all(), r
    return exact


@pytest.mark.parametrize("rows,H,V,k", [(81, 4096, 32000, 8), (5, 256, 1000, 8), (100, 512, 777, 3),
                                         (1, 128, 130, 1), (200, 256, 4096, 8)])
def test_lmhead_topk_parity(tr, rows, H, V, k):
    g = torch.Generator().manual_seed(91 + rows)
    h = torch.randn((rows, H), generator=g).to(torch.bfloat16)
    W = torch.randn((V, H), generator=g).to(torch.bfloat16)
    ws = tr.new_lmhead_workspace(rows, V, k)
    out = torch.empty((rows, k), dtype=torch.int32, device=DEV)
    tr.tr_lmhead_topk(h.to(DEV), W.to(DEV), k, out, ws)
    z = O.lmhead_logits(h.float().numpy(), W.float().numpy())
    exact = check_lmhead_rows(z, out.cpu().numpy(), k, lmhead_tol(H))
    # the bound leaves every row of the short products separated (so each
    # must match exactly) and 72 of 81 at H = 4096; the rest: valid within it
    assert exact == rows if H <= 512 else exact >= int(rows * 0.85)


def test_lmhead_topk_large_vocab_sampled_rows(tr):
    # 32 sequences x 81 nodes against a 128256 x 4096 output embedding (27
    # row tiles, W streamed once per tile); the oracle follows sampled rows
    rows, H, V, k = 2592, 4096, 128256, 8
    g = torch.Generator(device=DEV).manual_seed(92)
    h = torch.randn((rows, H), generator=g, device=DEV).to(torch.bfloat16)
    W = torch.randn((V, H), generator=g, device=DEV).to(torch.bfloat16)
    ws = tr.new_lmhead_workspace(rows, V, k)
    out = torch.empty((rows, k), dtype=torch.int32, device=DEV)
    tr.tr_lmhead_topk(h, W, k, out, ws)
    pick = [0, 95, 96, 1295, 2591]
    z = O.lmhead_logits(h[pick].float().cpu().numpy(), W.float().cpu().numpy())
    check_lmhead_rows(z, out[pick].cpu().numpy(), k, lmhead_tol(H))


@pytest.mark.parametrize("path", ["few_row", "merge"])
def test_step_lmhead_parity(tr, path, monkeypatch):
    # few rows go through the few-row step kernel's slice-list row blocks;
    # with that kernel switched off, through one merge block per row
    if path == "merge":
        monkeypatch.setenv("TR_FEW_ROW_STEP", "0")
    levels = RAND_LEVELS[4]
    t = otree(levels)
    T, D = t.n_nodes, t.max_depth
    B, H, V, k = 2, 512, 3000, 8
    g = torch.Generator().manual_seed(93)
    tree = tr.Tree.from_levels(levels, k)
    W = torch.randn((V, H), generator=g).to(torch.bfloat16)
    M = torch.randint(0, V, (B, V, k), generator=g, dtype=torch.int32)
    root = torch.randint(0, V, (B,), generator=g).to(torch.int32)
    ws = tr.new_lmhead_workspace(B * T, V, k)
    dM, droot, dW = M.to(DEV), root.to(DEV), W.to(DEV)
    tok = torch.empty((B, T), dtype=torch.int32, device=DEV)
    tr.tr_retrieve(tree, dM, droot, tok, ws)
    tok_h = tok.cpu().numpy().astype(np.int64)
    # hidden states: noise, and for most nodes the W row of their rank-0
    # child's token (that token then wins by far: accepted paths run deep)
    rng = np.random.default_rng(93)
    Wf = W.float().numpy()
    plant = [[bool(t.children(n)) and rng.random() < 0.85 for n in range(T)] for b in range(B)]

    def draw(b, n):
        x = torch.randn((H,), generator=g) * (0.02 if plant[b][n] else 1.0)
        if plant[b][n]:
            x += W[tok_h[b, t.children(n)[0]]].float() * 0.1
        return x.to(torch.bfloat16)

    def clear(row):
        # the k + 1 best oracle logits of the row are separated beyond the bound
        z = O.lmhead_logits(row.float().numpy()[None], Wf)[0]
        top = np.sort(z)[::-1][:k + 1]
        return (np.diff(-top) > lmhead_tol(H)).all()

    h = torch.empty((B, T, H), dtype=torch.bfloat16)
    for b in range(B):
        for n in range(T):
            h[b, n] = draw(b, n)
            while not clear(h[b, n]):                 # a near tie in the k+1 best: redraw
                h[b, n] = draw(b, n)
    L = torch.empty((B,), dtype=torch.int32, device=DEV)
    path = torch.empty((B, D + 1), dtype=torch.int32, device=DEV)
    em = torch.empty((B, D + 1), dtype=torch.int32, device=DEV)
    topk = torch.empty((B, T, k), dtype=torch.int32, device=DEV)
    tr.tr_step_lmhead(tree, h.to(DEV), dW, dM, tok, droot, L, path, em, ws, topk_out=topk)
    lengths = []
    for b in range(B):
        z = O.lmhead_logits(h[b].float().numpy(), W.float().numpy())
        assert check_lmhead_rows(z, topk[b].cpu().numpy(), k, lmhead_tol(H)) == T   # all exact
        Mo = M[b].numpy().astype(np.int64).copy()
        res, _ = O.step_after_forward(t, Mo, tok_h[b], z, k)
        assert int(L[b]) == res.verdict.accept_len
        lengths.append(res.verdict.accept_len)
        assert path[b, :res.verdict.accept_len + 1].cpu().tolist() == res.verdict.path.tolist()
        assert int(droot[b]) == res.verdict.bonus
        assert (dM[b].cpu().numpy().astype(np.int64) == Mo).all()
        assert tok[b].cpu().numpy().tolist() == res.next_tok.tolist()
    assert max(lengths) >= 4                          # the planted states reach deep
    assert tr.tr_read_device_status(ws) == 0


# ------------------------------------------------------------------ initial M
@pytest.mark.parametrize("m_dtype", [torch.int32, torch.int64])
def test_init_matrix_parity(tr, m_dtype):
    # odd V*k (one id per store) and V*k % 4 == 0 (16-byte groups), one
    # sequence and several, one prior for all and one per sequence
    g = torch.Generator().manual_seed(31)
    for B, V, k in ((1, 7, 3), (3, 1001, 5), (5, 13, 1), (2, 32000, 8), (4, 6, 2)):
        M = torch.full((B, V, k), -7, dtype=m_dtype, device=DEV)
        tr.tr_init_matrix(M, "zero")
        assert (M == 0).all()
        for seed in (0, 12345, 2 ** 64 - 1):
            tr.tr_init_matrix(M, "random", seed=seed)
            want = O.init_matrix(B, V, k, "random", seed=seed)
            assert np.array_equal(M.cpu().numpy().astype(np.int64), want), (B, V, k, seed)
        for p_dtype in (torch.int32, torch.int64):
            for pb in sorted({1, B}):
                prior = torch.randint(0, V, (pb, V, k), generator=g).to(p_dtype)
                tr.tr_init_matrix(M, "prior", prior.to(DEV))
                want = O.init_matrix(B, V, k, "prior", prior.numpy())
                assert np.array_equal(M.cpu().numpy().astype(np.int64), want), (B, V, k, pb)


def test_init_matrix_random_full_size(tr):
    # the large-vocabulary batch: 32 sequences of 128256 x 8 int32 ids
    B, V, k = 32, 128256, 8
    M = torch.empty((B, V, k), dtype=torch.int32, device=DEV)
    tr.tr_init_matrix(M, "random", seed=2024)
    assert np.array_equal(M.cpu().numpy().astype(np.int64), O.init_matrix(B, V, k, "random", seed=2024))


# ------------------------------------------------------------------ step + commit
def test_step_commit_and_cache_full_flag(tr):
    levels = RAND_LEVELS[1]
    t = otree(levels)
    tree = tr.Tree.from_levels(levels, 8)
    V, B, Hkv = 300, 2, 2
    g = torch.Generator().manual_seed(9)
    M = torch.randint(0, V, (B, V, 8), generator=g, dtype=torch.int32)
    kc = torch.zeros((B, Hkv, 40, 128), dtype=torch.bfloat16)
    vc = torch.zeros_like(kc)
    P = torch.tensor([5, 37], dtype=torch.int32)       # sequence 1 will overflow its cache
    root = torch.tensor([3, 4], dtype=torch.int32)
    kt = torch.randn((B, t.n_nodes, Hkv, 128), generator=g).to(torch.bfloat16)
    vt = torch.randn((B, t.n_nodes, Hkv, 128), generator=g).to(torch.bfloat16)
    ws = ws_for(tr, tree, B, V, 8)
    dM, dkc, dvc, dP, droot = (x.to(DEV) for x in (M, kc, vc, P, root))
    tok = torch.empty((B, t.n_nodes), dtype=torch.int32, device=DEV)
    tr.tr_retrieve(tree, dM, droot, tok, ws)
    tok_h = tok.cpu().numpy()
    # logits whose greedy continuation follows the rank-0 chain: accept 3 drafts
    z = torch.randn((B, t.n_nodes, V), generator=g)
    for b in range(B):
        for a, c in ((0, 1), (1, 5), (5, 13)):
            z[b, a, tok_h[b, c]] = 50.0
    L = torch.empty((B,), dtype=torch.int32, device=DEV)
    path = torch.empty((B, 4), dtype=torch.int32, device=DEV)
    em = torch.empty((B, 4), dtype=torch.int32, device=DEV)
    tr.tr_step(tree, z.to(DEV), dM, tok, droot, L, path, em, ws, kt.to(DEV), vt.to(DEV), dkc, dvc, dP)
    flags = tr.tr_read_device_status(ws)
    for b in range(B):
        Mo = M[b].numpy().astype(np.int64).copy()
        if b == 0:      # fits: the oracle commits too
            res, newP = O.step_after_forward(t, Mo, tok_h[b].astype(np.int64), z[b].numpy(), 8,
                                             kc[b].float().numpy(), vc[b].float().numpy(),
                                             kt[b].float().numpy(), vt[b].float().numpy(), int(P[b]))
        else:           # 37 + 4 > 40: no commit, prefix unchanged, flag raised
            res, newP = O.step_after_forward(t, Mo, tok_h[b].astype(np.int64), z[b].numpy(), 8)[0], int(P[b])
        assert int(L[b]) == 3 == res.verdict.accept_len
        assert (dM[b].cpu().numpy() == Mo).all()
        assert tok[b].cpu().numpy().tolist() == res.next_tok.tolist()
        assert int(droot[b]) == res.verdict.bonus
        assert int(dP[b]) == newP
    assert torch.equal(dkc[0, :, 5:9].cpu(), kt[0, [0, 1, 5, 13]].transpose(0, 1))
    assert torch.equal(dvc[0, :, 5:9].cpu(), vt[0, [0, 1, 5, 13]].transpose(0, 1))
    assert (dkc[0, :, 9:].cpu() == 0).all() and (dkc[1].cpu() == 0).all()
    assert flags & tr.TR_FLAG_CACHE_FULL
