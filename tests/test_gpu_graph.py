"""The step loop captured into a HIP graph (MI355X only).

Every library call launches its kernels on the caller's stream, so a
capture of tr_tree_attn + tr_step turns each launch into a kernel node with
its arguments fixed.  The graph is replayed several times, the state reset
in place between replays by ordinary eager work (copies and a retrieval
call), and every replay must end bit for bit where the eager run of the
same steps ended: tree tokens, M, both caches, prefix length, verdicts and
the last attention output.  A launch that left state behind it (a counter
not returned to zero, a memset node) would make a later replay differ.
"""
import pytest
import torch

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


@pytest.mark.parametrize("name", ["vicuna7b", "largevocab"])
def test_graph_replays_match_eager(tr, name):
    from draft_tree_retrieval_amd.loop import TRDecoder
    w = W.WORKLOADS[name]
    steps = 6
    st0 = W.initial_state(w, DEV, cap=w.cap(steps + 2))
    tree = tr.Tree.from_levels(w.levels, w.k)
    out = torch.empty((w.B, w.T, w.Hq, w.d), dtype=w.kv_dtype, device=DEV)

    # eager run; the inputs of every step are kept (the logits plant a
    # continuation of the tree each step built)
    st = st0.clone()
    dec = TRDecoder(tree, st.M, st.k_cache, st.v_cache, st.prefix_len, st.root, Hq=w.Hq)
    inputs = []
    for s in range(steps):
        q, kt, vt = W.step_qkv(w, s, DEV)
        z = W.step_logits(w, s, dec.tree_tok, DEV)
        dec.attend(q, kt, vt, out)
        dec.step(z, kt, vt)
        inputs.append((q, kt, vt, z))
    torch.cuda.synchronize()
    want = {"tree_tok": dec.tree_tok.clone(), "M": st.M.clone(), "k_cache": st.k_cache.clone(),
            "v_cache": st.v_cache.clone(), "prefix_len": st.prefix_len.clone(),
            "root": st.root.clone(), "accept_len": dec.accept_len.clone(),
            "accept_path": dec.accept_path.clone(), "emitted": dec.emitted.clone(),
            "out": out.clone()}
    assert dec.device_flags() == 0

    # the same steps captured once on fixed state tensors
    sg = st0.clone()
    gdec = TRDecoder(tree, sg.M, sg.k_cache, sg.v_cache, sg.prefix_len, sg.root, Hq=w.Hq)
    gout = torch.empty_like(out)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for q, kt, vt, z in inputs:
            gdec.attend(q, kt, vt, gout)
            gdec.step(z, kt, vt)
    torch.cuda.synchronize()
    for rep in range(3):
        # eager work between replays: the state back to its start, in place
        sg.M.copy_(st0.M)
        sg.k_cache.copy_(st0.k_cache)
        sg.v_cache.copy_(st0.v_cache)
        sg.prefix_len.copy_(st0.prefix_len)
        sg.root.copy_(st0.root)
        tr.tr_retrieve(tree, sg.M, sg.root, gdec.tree_tok, gdec.ws)
        gout.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = {"tree_tok": gdec.tree_tok, "M": sg.M, "k_cache": sg.k_cache, "v_cache": sg.v_cache,
               "prefix_len": sg.prefix_len, "root": sg.root, "accept_len": gdec.accept_len,
               "accept_path": gdec.accept_path, "emitted": gdec.emitted, "out": gout}
        for key, ref in want.items():
            assert torch.equal(got[key], ref), f"{name} replay {rep}: {key} differs from the eager run"
        assert gdec.device_flags() == 0
    del graph
