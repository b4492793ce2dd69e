"""A TR decoding loop on one GPU: device state plus the two calls of a step.

One step of Token Recycling ("Token Recycling" summary, Method; walk-through
"why it is called Token Recycling"): the target model's forward pass over
the merged tree sequence calls tree attention once per layer
(`attend`); after the forward pass, `step` takes the logits of every tree
node and runs top-k, verification, the update of M, the commit of the
accepted path's key/value rows and the retrieval of the next tree, in one
fused launch.  The state never leaves the GPU; nothing here synchronises.
"""
from __future__ import annotations

import torch

from . import tr


def to_pages(cache, page_size, spare_pages=0, seed=0):
    """A page pool [1][num_pages][Hkv][page_size][d] holding a contiguous
    cache [B][Hkv][cap][d] (cap a multiple of page_size) in shuffled pages,
    and its block table [B][cap / page_size] (int32, same device)."""
    B, Hkv, cap, d = cache.shape
    if cap % page_size:
        raise ValueError("cap must be a multiple of page_size")
    mp = cap // page_size
    n = B * mp + spare_pages
    perm = torch.randperm(n, generator=torch.Generator().manual_seed(seed))
    table = perm[:B * mp].reshape(B, mp).to(torch.int32).to(cache.device)
    pool = torch.zeros((1, n, Hkv, page_size, d), dtype=cache.dtype, device=cache.device)
    src = cache.reshape(B, Hkv, mp, page_size, d).permute(0, 2, 1, 3, 4).reshape(B * mp, Hkv,
                                                                                  page_size, d)
    pool[0, table.reshape(-1).long()] = src
    return pool, table


def from_pages(pool, table, layer=0):
    """The contiguous cache [B][Hkv][cap][d] of one layer of a page pool."""
    B, mp = table.shape
    _, n, Hkv, ps, d = pool.shape
    x = pool[layer, table.reshape(-1).long()].reshape(B, mp, Hkv, ps, d)
    return x.permute(0, 2, 1, 3, 4).reshape(B, Hkv, mp * ps, d)


class TRDecoder:
    def __init__(self, tree: tr.Tree, M, k_cache, v_cache, prefix_len, root_tok, Hq,
                 V=None, stream=None, update="all", page_size=None):
        self.tree = tree
        self.update = update          # "all" (the method) or "accepted" (its ablation)
        # page_size: keep the prefix in a paged cache (one layer) built from
        # k_cache/v_cache in shuffled pages, and use the paged calls
        self.page_size = page_size
        if page_size:
            self.k_pages, self.block_table = to_pages(k_cache, page_size, spare_pages=3, seed=1)
            self.v_pages, _ = to_pages(v_cache, page_size, spare_pages=3, seed=1)
        self.M, self.k_cache, self.v_cache = M, k_cache, v_cache
        self.prefix_len, self.root_tok = prefix_len, root_tok
        self.stream = stream
        B, Vm, k = M.shape
        self.B, self.V, self.k = B, (V or Vm), k
        T, D = tree.n_nodes, tree.depth
        self.Hq, self.Hkv, self.cap, self.d = Hq, k_cache.shape[1], k_cache.shape[2], k_cache.shape[3]
        dev = M.device
        i32 = dict(dtype=torch.int32, device=dev)
        self.tree_tok = torch.empty((B, T), **i32)
        self.accept_len = torch.zeros((B,), **i32)
        self.accept_path = torch.full((B, D + 1), -1, **i32)
        self.emitted = torch.full((B, D + 1), -1, **i32)
        self.topk = torch.empty((B, T, k), **i32)
        self.ws = tr.new_workspace(tree, B, self.V, k, Hq, self.Hkv, self.d, self.cap, device=dev,
                                   stream=stream)
        tr.tr_retrieve(tree, M, root_tok, self.tree_tok, self.ws, stream)

    def _kv(self, k_tree, v_tree):
        return tr.PagedKV(self.k_pages, self.v_pages, self.block_table, k_tree.unsqueeze(0),
                          v_tree.unsqueeze(0), self.prefix_len)

    def attend(self, q, k_tree, v_tree, out, scale=None):
        if self.page_size:
            tr.tr_tree_attn_paged(self.tree, q, self._kv(k_tree, v_tree), 0, out, self.ws, scale,
                                  self.stream)
            return
        tr.tr_tree_attn(self.tree, q, k_tree, v_tree, self.k_cache, self.v_cache, self.prefix_len,
                        out, self.ws, scale, self.stream)

    def step(self, logits, k_tree, v_tree):
        if self.page_size:
            tr.tr_step_paged(self.tree, logits, self.M, self.tree_tok, self.root_tok,
                             self.accept_len, self.accept_path, self.emitted, self.ws,
                             self._kv(k_tree, v_tree), self.topk, self.update, self.stream)
            return
        if self.update == "all":
            tr.tr_step(self.tree, logits, self.M, self.tree_tok, self.root_tok, self.accept_len,
                       self.accept_path, self.emitted, self.ws, k_tree, v_tree, self.k_cache,
                       self.v_cache, self.prefix_len, self.topk, self.stream)
        else:
            tr.tr_step_ex(self.tree, logits, self.M, self.tree_tok, self.root_tok,
                          self.accept_len, self.accept_path, self.emitted, self.ws, k_tree,
                          v_tree, self.k_cache, self.v_cache, self.prefix_len, self.topk,
                          self.update, self.stream)

    def step_sample(self, logits, k_tree, v_tree, temperature, uniforms):
        """The step verifying by sampling; uniforms [B][T][2] float32 in [0, 1)."""
        if self.page_size:
            raise NotImplementedError("sampling verification takes the contiguous cache")
        tr.tr_step_sample(self.tree, logits, temperature, uniforms, self.M, self.tree_tok,
                          self.root_tok, self.accept_len, self.accept_path, self.emitted, self.ws,
                          k_tree, v_tree, self.k_cache, self.v_cache, self.prefix_len, self.topk,
                          self.update, self.stream)

    def device_flags(self):
        return tr.tr_read_device_status(self.ws, self.stream)
