"""The allocation-free tree attention (tr_tree_attn_noalloc) against the
workspace entry point it varies (tr_tree_attn): the same kernels on the
same inputs, so the outputs must be bit-identical.  Two calls in a row on
the library's per-GPU scratch, the second with a smaller input (the array
keeps the first call's contents), plus an fp32 call and a call whose
prefix length is out of range (the flag lands in the caller's word)."""
import os
import sys

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

pytestmark = pytest.mark.gpu
DEV = "cuda"

# levels, B, Hq, Hkv, prefix lengths, cap, dtype: the second call is smaller
CASES = [
    ([[8], [6, 4, 3, 2, 2, 1, 1, 1], [5, 4, 3, 2, 2, 2, 1, 1, 1, 1], [4, 3, 2, 2, 2, 1, 1, 1, 1, 1],
      [3, 2, 2, 1, 1, 1], [2]], 8, 32, 8, [1500, 300, 1024, 777, 64, 0, 2000, 1999], 2048,
     torch.bfloat16),
    ([[4], [4, 2, 1, 1], [2, 1]], 2, 8, 4, [130, 17], 200, torch.bfloat16),
    ([[4], [4, 2, 1, 1], [2, 1]], 1, 8, 8, [256], 300, torch.float32),
]


@pytest.fixture(scope="module")
def tr():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    from draft_tree_retrieval_amd import tr as _tr
    _tr.load()
    return _tr


def _inputs(g, B, T, Hq, Hkv, cap, dtype):
    mk = lambda *s: torch.randn(s, generator=g).to(dtype).to(DEV)
    return (mk(B, T, Hq, 128), mk(B, T, Hkv, 128), mk(B, T, Hkv, 128), mk(B, Hkv, cap, 128),
            mk(B, Hkv, cap, 128))


def _same(a, b):
    view = torch.int16 if a.dtype == torch.bfloat16 else torch.int32
    return torch.equal(a.view(view), b.view(view))


def test_noalloc_equals_workspace_call(tr):
    for i, (levels, B, Hq, Hkv, Ps, cap, dtype) in enumerate(CASES):
        print(f"no-alloc case {i}: B={B} Hq={Hq} Hkv={Hkv} cap={cap} {dtype}", flush=True)
        tree = tr.Tree.from_levels(levels, 8)
        g = torch.Generator().manual_seed(500 + i)
        q, kt, vt, kc, vc = _inputs(g, B, tree.n_nodes, Hq, Hkv, cap, dtype)
        P = torch.tensor(Ps, dtype=torch.int32, device=DEV)
        ws = tr.new_workspace(tree, B, 0, 0, Hq, Hkv, 128, cap, device=DEV)
        want = torch.empty_like(q)
        tr.tr_tree_attn(tree, q, kt, vt, kc, vc, P, want, ws)
        got = torch.full_like(q, float("nan"))
        flags = torch.zeros(1, dtype=torch.int32, device=DEV)
        tr.tr_tree_attn_noalloc(tree, q, kt, vt, kc, vc, P, got, flags)
        torch.cuda.synchronize()
        assert _same(got, want), f"case {i}"
        assert int(flags[0]) == 0
        assert tr.tr_read_device_status(ws) == 0


def test_noalloc_flags_bad_prefix(tr):
    levels, B, Hq, Hkv, Ps, cap, dtype = CASES[1]
    tree = tr.Tree.from_levels(levels, 8)
    g = torch.Generator().manual_seed(77)
    q, kt, vt, kc, vc = _inputs(g, B, tree.n_nodes, Hq, Hkv, cap, dtype)
    bad = torch.tensor([cap + 5, 17], dtype=torch.int32, device=DEV)      # clamped to cap
    ok = torch.tensor([cap, 17], dtype=torch.int32, device=DEV)
    ws = tr.new_workspace(tree, B, 0, 0, Hq, Hkv, 128, cap, device=DEV)
    want = torch.empty_like(q)
    tr.tr_tree_attn(tree, q, kt, vt, kc, vc, ok, want, ws)
    got = torch.empty_like(q)
    flags = torch.zeros(1, dtype=torch.int32, device=DEV)
    tr.tr_tree_attn_noalloc(tree, q, kt, vt, kc, vc, bad, got, flags)
    torch.cuda.synchronize()
    assert _same(got, want)
    assert int(flags[0]) == tr.TR_FLAG_BAD_PREFIX
