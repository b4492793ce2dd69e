"""The Python binding refuses tensors whose shape, dtype, layout or device do
not match what the C call assumes, before anything reaches the library (a
mismatched M or logits tensor would otherwise be read or written out of
bounds on the device).  CPU only: the tensors are host tensors, so every
call below must stop in the binding."""
import pytest
import torch

from draft_tree_retrieval_amd import tr

LEVELS = [[3], [2, 1]]        # 7 nodes, depth 2
K = 4


@pytest.fixture(scope="module")
def tree():
    tr.load()
    return tr.Tree.from_levels(LEVELS, K)


def step_tensors(tree, B=2, V=50, dtype=torch.float32):
    T, W = tree.n_nodes, tree.depth + 1
    i32 = dict(dtype=torch.int32)
    return dict(logits=torch.zeros((B, T, V), dtype=dtype), M=torch.zeros((B, V, K), **i32),
                tree_tok=torch.zeros((B, T), **i32), root_tok=torch.zeros((B,), **i32),
                accept_len=torch.zeros((B,), **i32), accept_path=torch.zeros((B, W), **i32),
                emitted=torch.zeros((B, W), **i32), ws=torch.zeros(1024, dtype=torch.uint8))


def call_step(tree, t, **kw):
    args = dict(t)
    args.update(kw)
    tr.tr_step(tree, args["logits"], args["M"], args["tree_tok"], args["root_tok"],
               args["accept_len"], args["accept_path"], args["emitted"], args["ws"],
               **{k: v for k, v in args.items() if k in ("k_tree", "v_tree", "k_cache", "v_cache",
                                                         "prefix_len", "topk_out")})


@pytest.mark.parametrize("field,bad,msg", [
    ("M", torch.zeros((2, 50, K + 1), dtype=torch.int32), "M has shape"),          # k != tree.k
    ("M", torch.zeros((2, 49, K), dtype=torch.int32), "M has shape"),              # V != logits V
    ("M", torch.zeros((2, 50, K), dtype=torch.float32), "M has dtype"),
    ("logits", torch.zeros((2, 6, 50)), "rows per sequence"),                      # T != nodes
    ("logits", torch.zeros((2, 7, 50), dtype=torch.float16), "logits has dtype"),
    ("tree_tok", torch.zeros((2, 7), dtype=torch.int64), "tree_tok has dtype"),
    ("root_tok", torch.zeros((3,), dtype=torch.int32), "root_tok has shape"),
    ("accept_path", torch.zeros((2, 2), dtype=torch.int32), "accept_path has shape"),
    ("topk_out", torch.zeros((2, 7, K - 1), dtype=torch.int32), "topk_out has shape"),
    ("ws", torch.zeros(16, dtype=torch.int32), "ws has dtype"),
])
def test_step_mismatches_are_refused(tree, field, bad, msg):
    t = step_tensors(tree)
    with pytest.raises(ValueError, match=msg):
        call_step(tree, t, **{field: bad})


def test_step_host_tensors_and_strides_are_refused(tree):
    t = step_tensors(tree)
    with pytest.raises(ValueError, match="takes GPU memory"):
        call_step(tree, t)                                   # right shapes, host memory
    strided = torch.zeros((2, 50, 2 * K), dtype=torch.int32)[:, :, ::2]
    with pytest.raises(ValueError, match="contiguous"):
        call_step(tree, t, M=strided)


def test_step_cache_mismatches_are_refused(tree):
    t = step_tensors(tree)
    B, T = 2, tree.n_nodes
    kc = torch.zeros((B, 2, 16, 128), dtype=torch.bfloat16)
    good = dict(k_cache=kc, v_cache=kc.clone(), k_tree=torch.zeros((B, T, 2, 128), dtype=torch.bfloat16),
                v_tree=torch.zeros((B, T, 2, 128), dtype=torch.bfloat16),
                prefix_len=torch.zeros((B,), dtype=torch.int32))
    with pytest.raises(ValueError, match="v_cache has shape"):
        call_step(tree, t, **{**good, "v_cache": torch.zeros((B, 2, 15, 128), dtype=torch.bfloat16)})
    with pytest.raises(ValueError, match="k_tree has shape"):
        call_step(tree, t, **{**good, "k_tree": torch.zeros((B, T, 3, 128), dtype=torch.bfloat16)})
    with pytest.raises(ValueError, match="has dtype"):
        call_step(tree, t, **{**good, "v_tree": torch.zeros((B, T, 2, 128))})
    with pytest.raises(ValueError, match="prefix_len is required"):
        call_step(tree, t, **{**good, "prefix_len": None})


def test_step_sample_uniforms_are_checked(tree):
    t = step_tensors(tree)
    with pytest.raises(ValueError, match="uniforms has shape"):
        tr.tr_step_sample(tree, t["logits"], 1.0, torch.zeros((2, 7, 3)), t["M"], t["tree_tok"],
                          t["root_tok"], t["accept_len"], t["accept_path"], t["emitted"], t["ws"])


def test_attention_mismatches_are_refused(tree):
    B, T, Hq, Hkv, cap = 2, tree.n_nodes, 8, 2, 32
    bf = dict(dtype=torch.bfloat16)
    q = torch.zeros((B, T, Hq, 128), **bf)
    kt, vt = torch.zeros((B, T, Hkv, 128), **bf), torch.zeros((B, T, Hkv, 128), **bf)
    kc, vc = torch.zeros((B, Hkv, cap, 128), **bf), torch.zeros((B, Hkv, cap, 128), **bf)
    P = torch.zeros((B,), dtype=torch.int32)
    out = torch.zeros_like(q)
    ws = torch.zeros(1024, dtype=torch.uint8)
    with pytest.raises(ValueError, match="rows per sequence"):
        tr.tr_tree_attn(tree, q[:, :5], kt, vt, kc, vc, P, out, ws)
    with pytest.raises(ValueError, match="out has shape"):
        tr.tr_tree_attn(tree, q, kt, vt, kc, vc, P, out[:, :, :4], ws)
    with pytest.raises(ValueError, match="v_tree has shape"):
        tr.tr_tree_attn(tree, q, kt, vt[:1], kc, vc, P, out, ws)
    with pytest.raises(ValueError, match="has dtype"):
        tr.tr_tree_attn(tree, q, kt.float(), vt, kc, vc, P, out, ws)
    with pytest.raises(ValueError, match="takes GPU memory"):
        tr.tr_tree_attn(tree, q, kt, vt, kc, vc, P, out, ws)
    with pytest.raises(ValueError, match="flags has dtype"):
        tr.tr_tree_attn_noalloc(tree, q, kt, vt, kc, vc, P, out, flags=torch.zeros(1))


def test_paged_descriptor_is_checked(tree):
    L, npg, Hkv, ps, B, T = 2, 8, 2, 64, 2, tree.n_nodes
    bf = dict(dtype=torch.bfloat16)
    pages = torch.zeros((L, npg, Hkv, ps, 128), **bf)
    ktr = torch.zeros((L, B, T, Hkv, 128), **bf)
    with pytest.raises(ValueError, match="block_table has dtype"):
        tr.PagedKV(pages, pages.clone(), torch.zeros((B, 4), dtype=torch.int64), ktr, ktr.clone(),
                   torch.zeros((B,), dtype=torch.int32))
    with pytest.raises(ValueError, match="v_pages has shape"):
        tr.PagedKV(pages, pages[:, :4], torch.zeros((B, 4), dtype=torch.int32), ktr, ktr.clone(),
                   torch.zeros((B,), dtype=torch.int32))


def test_other_calls_are_checked(tree):
    i32 = dict(dtype=torch.int32)
    ws = torch.zeros(1024, dtype=torch.uint8)
    with pytest.raises(ValueError, match="M has shape"):
        tr.tr_retrieve(tree, torch.zeros((2, 50, K + 2), **i32), torch.zeros((2,), **i32),
                       torch.zeros((2, 7), **i32), ws)
    with pytest.raises(ValueError, match="tree_tok has shape"):
        tr.tr_retrieve(tree, torch.zeros((2, 50, K), **i32), torch.zeros((2,), **i32),
                       torch.zeros((2, 6), **i32), ws)
    with pytest.raises(ValueError, match="topk_out is required"):           # nothing to write
        tr.tr_update_topk(tree, torch.zeros((1, 7, 50)), None, None, None, ws)
    with pytest.raises(ValueError, match="topk has shape"):
        tr.tr_verify(tree, torch.zeros((1, 7, K + 1), **i32), torch.zeros((1, 7), **i32),
                     torch.zeros((1,), **i32), None, torch.zeros((1,), **i32), None)
    with pytest.raises(ValueError, match="W has shape"):
        tr.tr_lmhead_topk(torch.zeros((3, 64), dtype=torch.bfloat16),
                          torch.zeros((100, 32), dtype=torch.bfloat16), 8,
                          torch.zeros((3, 8), **i32), ws)
    with pytest.raises(ValueError, match="prior has shape"):
        tr.tr_init_matrix(torch.zeros((2, 50, K), **i32), "prior", prior=torch.zeros((3, 50, K), **i32))
    with pytest.raises(ValueError, match="ws has dtype"):
        tr.tr_read_device_status(torch.zeros(16, **i32))
