"""Seeded synthetic inputs for Token Recycling steps.

This module is the stand-in for the target language model: it draws the
adjacency-matrix start state, the prefix key/value cache, the per-step
query/key/value rows of the tree tokens and the per-step next-token logits
with a planted greedy continuation.  It does none of the method's own
arithmetic (no retrieval, attention, top-k, verification or update): where a
planting rule needs the tree, the caller passes the tree tokens and the
parent array in.

Both the HIP path and the CPU oracle consume exactly the tensors drawn here
(the oracle gets host copies).  Draws use torch generators seeded from
(config seed, step, stream), so a given device reproduces them bit for bit.

The five workloads follow the shapes of the method's evaluation models
(Vicuna 7B/13B, Code Llama 34B with grouped key/value heads, a 128k-vocabulary
batched case); the public benchmark suites the pages evaluate on are not
used: synthetic rows of the same shapes and the distributions given per
workload stand in for them.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

# Per-layer child-count lists of the static trees.  Layer d lists the number
# of children of each node of that layer, earlier nodes first.
TREE_16 = [[4], [4, 2, 1, 1], [2, 1]]                         # 15 drafts, depth 3
TREE_81 = [[8], [6, 4, 3, 2, 2, 1, 1, 1], [5, 4, 3, 2, 2, 2, 1, 1, 1, 1],
           [4, 3, 2, 2, 2, 1, 1, 1, 1, 1], [3, 2, 2, 1, 1, 1], [2]]   # 80 drafts, depth 6


def levels_to_parent_rank(levels):
    """Parent/rank arrays of a per-layer child-count list (plain bookkeeping
    of the config format: children of a node take ranks 0..c-1)."""
    parent, rank, layer = [-1], [-1], [0]
    for counts in levels:
        nxt = []
        for i, c in enumerate(counts):
            for r in range(c):
                parent.append(layer[i])
                rank.append(r)
                nxt.append(len(parent) - 1)
        layer = nxt
    return parent, rank


@dataclass
class Workload:
    name: str
    V: int
    k: int
    B: int
    levels: list
    Hq: int
    Hkv: int
    d: int
    kv_dtype: torch.dtype
    logit_dtype: torch.dtype
    m_dtype: torch.dtype
    prefix: tuple            # (lo, hi) inclusive range of initial prefix lengths
    steps: int
    logit_std: float
    plant: str               # "chain3" | "first_order" | "geometric" | "cycle"
    seed: int
    description: str = ""
    parent: list = field(init=False)
    rank: list = field(init=False)

    def __post_init__(self):
        self.parent, self.rank = levels_to_parent_rank(self.levels)

    @property
    def T(self):
        return len(self.parent)

    @property
    def depth(self):
        return len(self.levels)

    def cap(self, steps=None):
        steps = self.steps if steps is None else steps
        return self.prefix[1] + steps * (self.depth + 1)

    def scaled(self, **over):
        """A copy with some fields replaced (smaller parity cases)."""
        kw = {f: getattr(self, f) for f in self.__dataclass_fields__ if self.__dataclass_fields__[f].init}
        kw.update(over)
        return Workload(**kw)


WORKLOADS = {
    "tiny": Workload(
        "tiny", V=32000, k=8, B=1, levels=TREE_16, Hq=8, Hkv=8, d=128,
        kv_dtype=torch.float32, logit_dtype=torch.float32, m_dtype=torch.int64,
        prefix=(256, 256), steps=1, logit_std=2.0, plant="chain3", seed=1000,
        description="tiny single step: V=32000 k=8 int64 M, 16-node depth-3 tree, "
                    "8 heads x d=128 fp32, prefix 256"),
    "vicuna7b": Workload(
        "vicuna7b", V=32000, k=8, B=1, levels=TREE_81, Hq=32, Hkv=32, d=128,
        kv_dtype=torch.bfloat16, logit_dtype=torch.bfloat16, m_dtype=torch.int32,
        prefix=(2048, 2048), steps=256, logit_std=3.0, plant="first_order", seed=1001,
        description="Vicuna-7B-shaped step loop: V=32000 k=8 int32 M, 81-node depth-6 tree, "
                    "32 heads x d=128 bf16, prefix 2048, 256 steps"),
    "vicuna13b": Workload(
        "vicuna13b", V=32000, k=8, B=1, levels=TREE_81, Hq=40, Hkv=40, d=128,
        kv_dtype=torch.bfloat16, logit_dtype=torch.bfloat16, m_dtype=torch.int32,
        prefix=(4096, 4096), steps=512, logit_std=3.0, plant="geometric", seed=1002,
        description="Vicuna-13B-shaped: 40 heads x d=128 bf16, prefix 4096, geometric(0.4) "
                    "accept lengths, Zipf(1.1) targets, 512 steps"),
    "codellama34b": Workload(
        "codellama34b", V=32000, k=8, B=1, levels=TREE_81, Hq=64, Hkv=8, d=128,
        kv_dtype=torch.bfloat16, logit_dtype=torch.bfloat16, m_dtype=torch.int32,
        prefix=(8192, 8192), steps=512, logit_std=3.0, plant="cycle", seed=1003,
        description="Code-Llama-34B-shaped GQA 64/8 x d=128 bf16, prefix 8192, "
                    "repeated-substring targets, 512 steps"),
    "largevocab": Workload(
        "largevocab", V=128256, k=8, B=32, levels=TREE_81, Hq=32, Hkv=8, d=128,
        kv_dtype=torch.bfloat16, logit_dtype=torch.bfloat16, m_dtype=torch.int32,
        prefix=(1024, 4096), steps=128, logit_std=3.0, plant="first_order", seed=1004,
        description="large-vocab batched: V=128256, 32 sequences, GQA 32/8 x d=128 bf16, "
                    "prefixes U[1024,4096], 128 steps"),
}


def _gen(device, *key):
    g = torch.Generator(device=device)
    h = 0
    for x in key:
        h = (h * 1_000_003 + int(x)) % (2 ** 61 - 1)
    g.manual_seed(h)
    return g


# stream ids
_S_STATE, _S_QKV, _S_LOGITS, _S_PLANT, _S_MAP = 1, 2, 3, 4, 5


@dataclass
class State:
    """Decoding state carried from step to step (plain tensors)."""
    M: torch.Tensor              # [B, V, k]
    k_cache: torch.Tensor        # [B, Hkv, cap, d]
    v_cache: torch.Tensor
    prefix_len: torch.Tensor     # [B] int32
    root: torch.Tensor           # [B] int32, last committed token

    def clone(self):
        return State(*(x.clone() for x in (self.M, self.k_cache, self.v_cache,
                                           self.prefix_len, self.root)))

    def to(self, device):
        return State(*(x.to(device) for x in (self.M, self.k_cache, self.v_cache,
                                              self.prefix_len, self.root)))


def initial_state(w: Workload, device="cpu", cap=None) -> State:
    """Hot-started M (seeded uniform ids), a seeded prefix cache and root."""
    g = _gen(device, w.seed, _S_STATE)
    cap = w.cap() if cap is None else cap
    M = torch.randint(0, w.V, (w.B, w.V, w.k), generator=g, device=device,
                      dtype=torch.int64).to(w.m_dtype)
    lo, hi = w.prefix
    P = torch.randint(lo, hi + 1, (w.B,), generator=g, device=device, dtype=torch.int64)
    kc = torch.zeros((w.B, w.Hkv, cap, w.d), dtype=w.kv_dtype, device=device)
    vc = torch.zeros_like(kc)
    Pm = int(P.max())
    kc[:, :, :Pm] = torch.randn((w.B, w.Hkv, Pm, w.d), generator=g, device=device).to(w.kv_dtype)
    vc[:, :, :Pm] = torch.randn((w.B, w.Hkv, Pm, w.d), generator=g, device=device).to(w.kv_dtype)
    for b in range(w.B):                    # positions past each prefix stay zero
        kc[b, :, int(P[b]):] = 0
        vc[b, :, int(P[b]):] = 0
    root = torch.randint(0, w.V, (w.B,), generator=g, device=device, dtype=torch.int64)
    return State(M, kc, vc, P.to(torch.int32), root.to(torch.int32))


def step_qkv(w: Workload, step: int, device="cpu"):
    """Query rows of the tree tokens [B,T,Hq,d] and their key/value rows
    [B,T,Hkv,d], ~N(0,1) rounded to the workload's dtype."""
    g = _gen(device, w.seed, _S_QKV, step)
    q = torch.randn((w.B, w.T, w.Hq, w.d), generator=g, device=device).to(w.kv_dtype)
    kt = torch.randn((w.B, w.T, w.Hkv, w.d), generator=g, device=device).to(w.kv_dtype)
    vt = torch.randn((w.B, w.T, w.Hkv, w.d), generator=g, device=device).to(w.kv_dtype)
    return q, kt, vt


def first_order_map(w: Workload, device="cpu"):
    """Seeded map [B][V] -> V: the synthetic target's greedy next token of a
    token, whatever the context (a first-order target)."""
    g = _gen(device, w.seed, _S_MAP)
    return torch.randint(0, w.V, (w.B, w.V), generator=g, device=device, dtype=torch.int64)


def cycle_ids(w: Workload, device="cpu"):
    """Seeded cycle of 24 distinct token ids (the repeated substring)."""
    g = _gen(device, w.seed, _S_MAP)
    return torch.randperm(w.V, generator=g, device=device)[:24]


def _zipf_cdf(V, s, device):
    r = torch.arange(1, V + 1, dtype=torch.float64, device=device)
    pmf = r.pow(-s)
    return torch.cumsum(pmf / pmf.sum(), 0)


def _children_tokens(parent, tok):
    """[B,T,8] tokens of each node's children (-1 padded); structure only."""
    B, T = tok.shape
    ch = torch.full((B, T, 8), -1, dtype=torch.int64, device=tok.device)
    fill = [0] * T
    for n in range(1, T):
        p = parent[n]
        ch[:, p, fill[p]] = tok[:, n]
        fill[p] += 1
    return ch


def plant_targets(w: Workload, step: int, tree_tok: torch.Tensor, device=None):
    """The synthetic target's greedy token t(n) after every tree node [B,T].

    first_order: t(n) = H_b(tok n), a seeded map that M can learn.
    chain3: the rank-0 chain 0->1->5->13 is planted; other nodes random.
    geometric: a chain to depth L* ~ Geometric(0.4) (failures before the first
      success, clamped to the depth) is planted; every other node, and the last
      chain node, gets a Zipf(1.1)-ranked token that is none of its children's.
    cycle: a repeated substring of 24 ids: t(n) is the id after tok n in the
      cycle (the cycle's first id when tok n is not in it).
    """
    device = tree_tok.device if device is None else device
    tok = tree_tok.to(device=device, dtype=torch.int64)
    B, T = tok.shape
    g = _gen(device, w.seed, _S_PLANT, step)
    if w.plant == "first_order":
        H = first_order_map(w, device)
        return torch.gather(H, 1, tok)
    if w.plant == "chain3":
        t = torch.randint(0, w.V, (B, T), generator=g, device=device, dtype=torch.int64)
        for a, c in ((0, 1), (1, 5), (5, 13)):
            t[:, a] = tok[:, c]
        return t
    if w.plant == "cycle":
        S = cycle_ids(w, device)
        pos = torch.full((w.V,), -1, dtype=torch.int64, device=device)
        pos[S] = torch.arange(24, device=device)
        p = pos[tok]
        return torch.where(p >= 0, S[(p + 1) % 24], S[0].expand_as(p))
    if w.plant == "geometric":
        u = torch.rand((B,), generator=g, device=device, dtype=torch.float64)
        Ls = torch.clamp(torch.floor(torch.log(u) / math.log(0.6)), 0, w.depth).to(torch.int64)
        cdf = _zipf_cdf(w.V, 1.1, device)
        cand = torch.searchsorted(cdf, torch.rand((B, T, 8), generator=g, device=device,
                                                  dtype=torch.float64)).clamp_(max=w.V - 1)
        ch = _children_tokens(w.parent, tok)
        clash = (cand[:, :, :, None] == ch[:, :, None, :]).any(-1)          # [B,T,8]
        first_ok = torch.argmax((~clash).to(torch.int8), dim=-1)            # first usable draw
        t = torch.gather(cand, 2, first_ok[..., None])[..., 0]
        none_ok = clash.all(-1)
        if bool(none_ok.any()):                 # practically never: smallest id not a child's
            for b, n in none_ok.nonzero().tolist():
                used = set(ch[b, n].tolist())
                t[b, n] = next(x for x in range(w.V) if x not in used)
        chain = [0]
        for _ in range(w.depth):
            chain.append(w.parent.index(chain[-1]))     # rank-0 child: first child in order
        for b in range(B):
            for i in range(int(Ls[b])):
                t[b, chain[i]] = tok[b, chain[i + 1]]
        return t
    raise ValueError(w.plant)


def step_logits(w: Workload, step: int, tree_tok: torch.Tensor, device="cpu"):
    """Next-token logits of every tree node [B,T,V] in the workload's dtype:
    N(0, std^2) noise with the planted token set to rowmax + 1 (a unique
    maximum); the cycle rule also plants the seven next ranks at
    rowmax + 1 - 0.125 j with ids drawn from the rest of the cycle."""
    B, T, V = w.B, w.T, w.V
    g = _gen(device, w.seed, _S_LOGITS, step)
    z = (torch.randn((B, T, V), generator=g, device=device) * w.logit_std).to(w.logit_dtype)
    t = plant_targets(w, step, tree_tok.to(device))
    rowmax = z.amax(dim=-1).float()                                        # [B,T]
    z.scatter_(2, t[..., None], (rowmax + 1.0).to(w.logit_dtype)[..., None])
    if w.plant == "cycle":
        S = cycle_ids(w, device)
        gp = _gen(device, w.seed, _S_PLANT, step, 7)
        keys = torch.rand((B, T, 24), generator=gp, device=device)
        keys[S[None, None, :].expand(B, T, 24) == t[..., None]] = 2.0     # exclude t(n)
        pick = S[torch.argsort(keys, dim=-1)[..., :7]]                     # 7 distinct ids
        vals = rowmax[..., None] + 1.0 - 0.125 * torch.arange(1, 8, device=device)
        z.scatter_(2, pick, vals.to(w.logit_dtype))
    return z
