"""Plain CPU oracle for one Token Recycling (TR) step.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library (``draft_tree_retrieval_amd``) and imports nothing from it.

Everything here is written for readability, not speed: numpy arrays, float64
for every floating-point result, sequential loops where the method is
sequential.  Each function cites the passage of the source pages it follows:

* [TR-en]  "Token Recycling" summary page (hyper.ai/fr), sections Method and
  Experiment.
* [TR-zh]  the Chinese version of the same summary (hyper.ai/cn), section
  方法 (Method) -- the only page that prints the update equation
  M[x~_i] = argtopk(p~_{i+1}).
* [Blog]   "Token Recycling" walk-through (blog-shf.pages.dev), sections
  核心数据结构：邻接矩阵 (adjacency matrix), 完整工作流程 steps 1-4
  (workflow), 为什么叫 Token Recycling (why "recycling"), 为什么一个很小的矩阵
  就够用 (storage).
* [SD]     "Speculative decoding" lesson (anylearn.cc): acceptance rule,
  expected tokens per pass, the draft/verify loop and tree drafting.

Readings taken where the pages are silent are marked READING and listed, with
reasons, in the design notes of the repository.

Parity status: every function below is pinned by tests in
``tests/test_oracle_*.py`` (worked example, brute force, closed forms,
library special cases); attention numerics beyond the stated tolerance are
pinned only by the brute-force and library special cases.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np


# --------------------------------------------------------------------------
# a1: the static tree template
# --------------------------------------------------------------------------
@dataclass
class Template:
    """Static, imbalanced draft-tree template.

    [TR-en] Method: the number of children of every node is fixed across
    decoding steps (static) and earlier, higher-probability nodes of a layer
    get more children and reach deeper (imbalanced).  [Blog] workflow step 2:
    the node total is fixed so the attention mask can be prepared in advance.

    Node 0 is the root (the last committed token).  Nodes are numbered in
    the layer-by-layer order of the merged sequence ([TR-en] Method, "merged
    sequence through layer by layer traversal"; [Blog] workflow step 3).
    READING: inside a layer, order is (parent index, rank).
    """
    parent: np.ndarray          # [T] int, parent[0] = -1
    rank: np.ndarray            # [T] int, candidate column of the parent's row; rank[0] = -1
    depth: np.ndarray = field(init=False)
    ancestors: list = field(init=False)   # ancestors[n] = [0, ..., n] (root -> n)

    def __post_init__(self):
        parent = np.asarray(self.parent, dtype=np.int64)
        rank = np.asarray(self.rank, dtype=np.int64)
        T = len(parent)
        if T < 1 or len(rank) != T:
            raise ValueError("template needs at least the root and one rank per node")
        if parent[0] != -1 or rank[0] != -1:
            raise ValueError("node 0 must be the root (parent -1, rank -1)")
        depth = np.zeros(T, dtype=np.int64)
        anc = [[0]]
        seen = set()
        for n in range(1, T):
            p = int(parent[n])
            if not (0 <= p < n):
                raise ValueError(f"node {n}: parent {p} must precede it")
            if rank[n] < 0:
                raise ValueError(f"node {n}: negative rank")
            if (p, int(rank[n])) in seen:
                raise ValueError(f"node {n}: duplicate rank {rank[n]} under parent {p}")
            seen.add((p, int(rank[n])))
            depth[n] = depth[p] + 1
            anc.append(anc[p] + [n])
        # layer-by-layer numbering: (depth, parent, rank) must be increasing
        keys = [(int(depth[n]), int(parent[n]), int(rank[n])) for n in range(1, T)]
        if keys != sorted(keys):
            raise ValueError("nodes are not in layer order (depth, parent, rank)")
        self.parent, self.rank, self.depth, self.ancestors = parent, rank, depth, anc

    @property
    def n_nodes(self) -> int:
        return len(self.parent)

    @property
    def max_depth(self) -> int:
        return int(self.depth.max())

    def children(self, n: int) -> list:
        return [m for m in range(self.n_nodes) if self.parent[m] == n]


def template_from_levels(levels) -> Template:
    """Build a template from per-layer child-count lists.

    levels[d][i] = number of children of the i-th node of layer d (layer 0 is
    the root alone).  Missing entries mean no children.  A node with c
    children takes the c best candidates (ranks 0..c-1) of its parent's row:
    READING of [TR-en] Method ("extracts the top k candidates ... then
    recursively expands each candidate") and of the [Blog] step-2 example
    (guest expands ranks 0,1,2; speaker ranks 0,1; speak rank 0).
    """
    parent, rank = [-1], [-1]
    layer = [0]                       # node ids of the current layer
    for counts in levels:
        if len(counts) > len(layer):
            raise ValueError("more child counts than nodes in the layer")
        nxt = []
        for i, c in enumerate(counts):
            for r in range(int(c)):
                parent.append(layer[i])
                rank.append(r)
                nxt.append(len(parent) - 1)
        layer = nxt
    return Template(np.array(parent), np.array(rank))


def ancestor_mask(t: Template) -> np.ndarray:
    """Tree-attention visibility: mask[n, j] is True iff node j is node n or
    one of its ancestors.  [TR-en] Method / [Blog] workflow step 3: each node
    sees only its own path back to the root; sibling branches are invisible.
    [SD] tree drafting: each node attends only to its ancestors.
    READING: a node also sees itself (the usual causal convention; the blog's
    list of what "at" sees includes "at")."""
    T = t.n_nodes
    mask = np.zeros((T, T), dtype=bool)
    for n in range(T):
        mask[n, t.ancestors[n]] = True
    return mask


# --------------------------------------------------------------------------
# a2: retrieval
# --------------------------------------------------------------------------
def retrieve(t: Template, M: np.ndarray, root: int) -> np.ndarray:
    """Draft tree retrieval from the adjacency matrix.

    [TR-en] Method, second module: the root is the last token of the current
    content; its top-k candidates are read from M and every candidate is
    expanded recursively according to the fixed tree structure.  [Blog]
    workflow steps 1-2 (guest -> M[guest] -> M[speaker], M[speak]).
    M[i, j] is the j-th candidate successor of token i ([TR-en] Method).
    Duplicates are kept (READING: the template's shape is static).
    """
    V = M.shape[0]
    tok = np.empty(t.n_nodes, dtype=np.int64)
    tok[0] = root
    for n in range(1, t.n_nodes):      # layer order: a parent is always filled first
        p = tok[t.parent[n]]
        if not (0 <= p < V):
            raise ValueError(f"token {p} outside the vocabulary")
        tok[n] = M[p, t.rank[n]]
    return tok


# --------------------------------------------------------------------------
# a3: tree attention
# --------------------------------------------------------------------------
def tree_attention(t: Template, q, k_tree, v_tree, k_cache, v_cache, prefix_len: int,
                   scale: float | None = None) -> np.ndarray:
    """Tree-attention verification of the merged sequence against the prefix.

    [TR-en] Method: the merged sequence is fed to the model together with
    the existing prefix and verified with tree attention; [Blog] workflow
    step 3: the mask lets each node see only its own path, never sibling
    branches.  For every tree node n and query head h:

        O[n, h] = sum_j softmax_j(q[n,h] . k_j * scale) v_j,
        j over prefix positions 0..P-1 and the tree nodes in anc(n).

    READING (pages silent): scale = 1/sqrt(d); query head h uses key/value
    head h // (Hq // Hkv); no positional rotation (inputs are synthetic).

    Shapes: q [T, Hq, d]; k_tree, v_tree [T, Hkv, d];
    k_cache, v_cache [Hkv, >=P, d].  Returns float64 [T, Hq, d].
    """
    q = np.asarray(q, dtype=np.float64)
    kt = np.asarray(k_tree, dtype=np.float64)
    vt = np.asarray(v_tree, dtype=np.float64)
    kc = np.asarray(k_cache, dtype=np.float64)[:, :prefix_len]
    vc = np.asarray(v_cache, dtype=np.float64)[:, :prefix_len]
    T, Hq, d = q.shape
    Hkv = kt.shape[1]
    if Hq % Hkv:
        raise ValueError("query heads must be a multiple of key/value heads")
    group = Hq // Hkv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    mask = ancestor_mask(t)
    out = np.empty((T, Hq, d), dtype=np.float64)
    for h in range(Hq):
        kh = h // group
        keys = np.concatenate([kc[kh], kt[:, kh]], axis=0)        # [P+T, d]
        vals = np.concatenate([vc[kh], vt[:, kh]], axis=0)
        s = (q[:, h] @ keys.T) * scale                               # [T, P+T]
        visible = np.concatenate([np.ones((T, prefix_len), dtype=bool), mask], axis=1)
        s = np.where(visible, s, -np.inf)
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p = p / p.sum(axis=1, keepdims=True)
        out[:, h] = p @ vals
    return out


# --------------------------------------------------------------------------
# a4: argtopk of each node's next-token distribution
# --------------------------------------------------------------------------
def topk_row(z, k: int) -> np.ndarray:
    """argtopk of one next-token distribution, best first.

    [TR-zh] Method: M[x~_i] = argtopk(p~_{i+1}); [Blog] "why recycling":
    the K most probable tokens of every node's distribution are kept.
    Softmax is strictly increasing, so the top-k of p~ are the top-k of the
    logits; ranking raw logits avoids ties that rounding in a softmax would
    create.  READING (pages silent): ties in value go to the lower token id;
    -0.0 equals +0.0 (plain value comparison).  Logits must not be NaN.
    """
    z = np.asarray(z, dtype=np.float64)
    V = z.shape[0]
    if not (1 <= k <= V):
        raise ValueError("need 1 <= k <= V")
    if np.isnan(z).any():
        raise ValueError("NaN logits are outside the contract")
    kth = np.partition(z, V - k)[V - k]          # the k-th largest value
    above = np.flatnonzero(z > kth)
    equal = np.flatnonzero(z == kth)[: k - len(above)]   # lowest ids first
    ids = np.concatenate([above, equal])
    order = np.lexsort((ids, -z[ids]))           # value descending, then id ascending
    return ids[order].astype(np.int64)


def topk_rows(Z, k: int) -> np.ndarray:
    Z = np.asarray(Z)
    return np.stack([topk_row(Z[i], k) for i in range(Z.shape[0])])


def lmhead_logits(h, W) -> np.ndarray:
    """The target's next-token logits of every node from its last hidden
    state: z = h W^T (h [rows][H], W [V][H], the output embedding), float64.
    READING: the pages take the logits as given; the LM head is the plain
    linear map in front of the softmax whose top-k the update recycles."""
    return np.asarray(h, dtype=np.float64) @ np.asarray(W, dtype=np.float64).T


# --------------------------------------------------------------------------
# a5: verification (greedy)
# --------------------------------------------------------------------------
@dataclass
class Verdict:
    accept_len: int          # L, accepted draft tokens (root excluded)
    path: np.ndarray         # node ids root -> best, length L+1
    bonus: int               # target's token after the last accepted node
    emitted: np.ndarray      # tokens committed this step: accepted drafts then bonus
    margin: float = math.inf  # sampling only: closest distance of a uniform to its threshold


def verify(t: Template, tok: np.ndarray, greedy: np.ndarray) -> Verdict:
    """Longest correct path plus the bonus token (greedy verification).

    [TR-en] Method: tree attention checks every candidate path in one pass
    and the longest correct sequence is the step's output.  [Blog] workflow
    step 4: the matching path is extended with the target's own token at the
    first mismatch, so the output equals the target's own greedy decoding.
    [SD]: the bonus token is collected when every draft was accepted.

    greedy[n] is the target's top-1 token after node n.  A node is accepted
    iff its parent is accepted and its token equals greedy[parent]; the root
    is accepted.  READING: "longest" is taken over the whole tree (deepest
    accepted node), ties going to the smaller node index.
    """
    T = t.n_nodes
    acc = np.zeros(T, dtype=bool)
    acc[0] = True
    for n in range(1, T):
        p = t.parent[n]
        acc[n] = acc[p] and tok[n] == greedy[p]
    best = 0
    for n in range(1, T):
        if acc[n] and t.depth[n] > t.depth[best]:
            best = n
    path = np.array(t.ancestors[best], dtype=np.int64)
    L = len(path) - 1
    bonus = int(greedy[best])
    emitted = np.concatenate([tok[path[1:]], [bonus]]).astype(np.int64)
    return Verdict(L, path, bonus, emitted)


def softmax_rows(logits, temperature: float) -> np.ndarray:
    """p = softmax(z / temperature) per row, float64."""
    z = np.asarray(logits, dtype=np.float64) / float(temperature)
    z = z - z.max(axis=-1, keepdims=True)
    e = np.exp(z)
    return e / e.sum(axis=-1, keepdims=True)


def draw(dist: np.ndarray, r: float):
    """Inverse-CDF draw: the smallest id whose cumulative probability (ids
    in increasing order) exceeds r in [0, 1).  Returns (id, margin), margin
    = distance of r to the nearer end of that id's interval.  READING: the
    pages sample without naming a method; this one lets a caller's uniform
    decide the draw."""
    c = np.cumsum(dist)
    x = int(np.searchsorted(c, r, side="right"))
    nz = np.flatnonzero(dist > 0)
    x = min(x, int(nz[-1]))           # r within rounding of the total mass
    lo = c[x - 1] if x > 0 else 0.0
    return x, min(r - lo, c[x] - r)


def verify_sample(t: Template, tok: np.ndarray, logits: np.ndarray, temperature: float,
                  uniforms: np.ndarray) -> Verdict:
    """Stochastic tree verification ([SD] acceptance rule, residual
    resampling and the bonus token after a fully accepted draft; [TR-en]
    Experiment: TR is also run with sampling).

    p_n = softmax(z_n / temperature) is the target's distribution after node
    n.  READING (the pages give the rule for one chain of drafts): TR's
    drafts are read from M, not sampled, so each draft's q is a point mass
    on its token.  The walk starts at the root; at node n the children are
    tried in rank order as the drafts of the next position.  With the
    current residual r (initially p_n), child c with token x is accepted
    when u_c < min(1, r(x) / q(x)) = r(x); then the walk moves to c.  Else
    r becomes norm(max(0, r - q)) (r with x removed, renormalised) and the
    next child is tried.  When no child is accepted (a leaf has none) the
    bonus is drawn from r with the node's second uniform, and the walk ends.

    uniforms[n][0] decides node n's own acceptance as a child; uniforms[n][1]
    the draw at n if the walk ends there.  Returns the path root -> stop
    node, L = its depth, the bonus and the emitted tokens, as verify().
    """
    p = softmax_rows(logits, temperature)
    V = p.shape[1]
    margin = math.inf
    n, path = 0, [0]
    while True:
        r = p[n].copy()
        nxt = None
        for c in t.children(n):
            x = int(tok[c])
            if not (0 <= x < V):
                continue                      # READING: a token outside the vocabulary is rejected
            a = min(1.0, r[x])                # q(x) = 1
            u = float(uniforms[c][0])
            margin = min(margin, abs(u - a))
            if u < a:
                nxt = c
                break
            q = np.zeros(V)
            q[x] = 1.0
            r = np.maximum(0.0, r - q)
            r = r / r.sum()
        if nxt is None:
            bonus, m = draw(r, float(uniforms[n][1]))
            margin = min(margin, m)
            break
        n = nxt
        path.append(n)
    path = np.array(path, dtype=np.int64)
    emitted = np.concatenate([tok[path[1:]], [bonus]]).astype(np.int64)
    return Verdict(len(path) - 1, path, bonus, emitted, margin)


# --------------------------------------------------------------------------
# a6: recycling update of M
# --------------------------------------------------------------------------
def update(M: np.ndarray, tok: np.ndarray, topk: np.ndarray) -> None:
    """In-place matrix update M[x~_i] = argtopk(p~_{i+1}) for every tree node.

    [TR-zh] Method (the equation); [TR-en] Method: the new top-k overwrite the
    token's previous candidates, with no conflict resolution for duplicated
    tokens; [Blog] "why recycling": every verified node's top-k enters M,
    including nodes on rejected paths (speak in the example).
    READING: nodes are written in merged-sequence order, so on a duplicated
    token the node with the highest index wins.
    """
    for n in range(len(tok)):
        M[tok[n], :] = topk[n, : M.shape[1]]


def update_accepted(M: np.ndarray, tok: np.ndarray, topk: np.ndarray, path) -> None:
    """The ablation that updates with accepted tokens only: M[x~_i] =
    argtopk(p~_{i+1}) for the nodes of the accepted path (root included),
    in path order ([TR-en] Experiment, ablations: all draft tokens give a
    higher mean accepted length than only the accepted ones; [TR-zh] same
    section).  READING: "accepted tokens" are the root and the accepted
    drafts, the nodes whose top-k the verification pass used for the
    emitted tokens; on a repeated token the later (deeper) node wins, as
    in update().
    """
    for n in path:
        M[tok[n], :] = topk[n, : M.shape[1]]


# --------------------------------------------------------------------------
# initial contents of M
# --------------------------------------------------------------------------
_GAMMA = 0x9E3779B97F4A7C15
_MASK64 = (1 << 64) - 1


def splitmix64(seed: int, e) -> np.ndarray:
    """Output e of SplitMix64 seeded with seed (Steele, Lea and Flood,
    "Fast splittable pseudorandom number generators", OOPSLA 2014, with the
    finaliser of Vigna's published splitmix64): the state after e+1 steps,
    seed + (e+1)*gamma mod 2^64, through the xor-shift-multiply mixer.
    Vectorised over e in uint64, whose products wrap mod 2^64."""
    e = np.asarray(e, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = np.uint64(seed & _MASK64) + (e + np.uint64(1)) * np.uint64(_GAMMA)
        z = (z ^ (z >> np.uint64(30))) * np.uint64(0xBF58476D1CE4E5B9)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(0x94D049BB133111EB)
        return z ^ (z >> np.uint64(31))


def init_matrix(B: int, V: int, k: int, mode: str, prior=None, seed: int = 0) -> np.ndarray:
    """Initial M [B][V][k] ([TR-en] Method, first module: a hot start
    inherits the matrix of earlier inference rather than an empty one;
    [TR-en] Experiment, initialisation ablation: all-zero, random, and
    fixed / shuffled / inherited priors).

    READING: "zero" is every id 0; "random" draws every id uniformly from
    the vocabulary, id e (flat over [B][V][k]) = floor(u*V) with u the high
    32 bits of SplitMix64 output e over 2^32; "prior" copies a prior matrix
    into every sequence's slot (one prior for all sequences, or one each),
    which covers the fixed, shuffled and inherited settings: they differ
    only in where the prior comes from.
    """
    if mode == "zero":
        return np.zeros((B, V, k), dtype=np.int64)
    if mode == "random":
        z = splitmix64(seed, np.arange(B * V * k, dtype=np.uint64))
        u = z >> np.uint64(32)
        return ((u * np.uint64(V)) >> np.uint64(32)).astype(np.int64).reshape(B, V, k)
    if mode == "prior":
        prior = np.asarray(prior, dtype=np.int64).reshape(-1, V, k)
        assert prior.shape[0] in (1, B)
        return np.array([prior[0 if prior.shape[0] == 1 else b] for b in range(B)])
    raise ValueError(mode)


# --------------------------------------------------------------------------
# a7: commit of the accepted path
# --------------------------------------------------------------------------
def commit(k_cache, v_cache, k_tree, v_tree, prefix_len: int, path) -> int:
    """Append the key/value rows of the accepted path (root first) to the
    prefix cache and return the new prefix length.

    READING (pages silent): the root and the L accepted drafts become prefix
    positions P..P+L; the bonus token has no key/value yet and is the next
    step's root ([Blog] workflow step 4: the accepted path plus the target's
    token continue the text; [TR-en] Method: the root is the last token of
    the current content).
    Shapes: caches [Hkv, cap, d]; tree [T, Hkv, d].
    """
    cap = k_cache.shape[1]
    if prefix_len + len(path) > cap:
        raise ValueError("cache capacity exceeded")
    for i, n in enumerate(path):
        k_cache[:, prefix_len + i, :] = k_tree[n]
        v_cache[:, prefix_len + i, :] = v_tree[n]
    return prefix_len + len(path)


# --------------------------------------------------------------------------
# paged prefix cache (a storage layout of the same prefix)
# --------------------------------------------------------------------------
def page_slot(table_b, page_size: int, pos: int):
    """(page id, row inside the page) of prefix position pos of one
    sequence: the block table lists the sequence's pages in order.  READING:
    the pages fix no cache layout; a paged cache holds the same prefix rows,
    so every result equals the contiguous cache's."""
    return int(table_b[pos // page_size]), pos % page_size


def gather_pages(pages, table_b, page_size: int, P: int):
    """The contiguous [Hkv][P][d] prefix of one sequence and one layer from
    a page pool [num_pages][Hkv][page_size][d]."""
    Hkv, d = pages.shape[1], pages.shape[3]
    out = np.zeros((Hkv, P, d), dtype=np.float64)
    for pos in range(P):
        pg, r = page_slot(table_b, page_size, pos)
        out[:, pos, :] = pages[pg, :, r, :]
    return out


def tree_attention_paged(t: Template, q, k_tree, v_tree, k_pages, v_pages, table_b,
                         page_size: int, prefix_len: int, scale=None) -> np.ndarray:
    """Tree attention over a paged prefix: the prefix rows gathered in
    position order, then tree_attention."""
    kc = gather_pages(k_pages, table_b, page_size, prefix_len)
    vc = gather_pages(v_pages, table_b, page_size, prefix_len)
    return tree_attention(t, q, k_tree, v_tree, kc, vc, prefix_len, scale)


def commit_paged(k_pages, v_pages, k_tree, v_tree, table_b, page_size: int, prefix_len: int,
                 path) -> int:
    """commit() into a paged cache, for every layer: k_pages/v_pages
    [layers][num_pages][Hkv][page_size][d], k_tree/v_tree [layers][T][Hkv][d].
    Position prefix_len + i of every layer receives the rows of path[i]."""
    cap = len(table_b) * page_size
    if prefix_len + len(path) > cap:
        raise ValueError("cache capacity exceeded")
    for layer in range(k_pages.shape[0]):
        for i, n in enumerate(path):
            pg, r = page_slot(table_b, page_size, prefix_len + i)
            k_pages[layer, pg, :, r, :] = k_tree[layer, n]
            v_pages[layer, pg, :, r, :] = v_tree[layer, n]
    return prefix_len + len(path)


# --------------------------------------------------------------------------
# one whole step for one sequence
# --------------------------------------------------------------------------
@dataclass
class StepResult:
    tok: np.ndarray          # this step's tree tokens
    topk: np.ndarray         # [T, k]
    verdict: Verdict
    next_tok: np.ndarray     # the next step's tree, retrieved from the updated M


def step_after_forward(t: Template, M: np.ndarray, tok: np.ndarray, logits: np.ndarray, k: int,
                       k_cache=None, v_cache=None, k_tree=None, v_tree=None,
                       prefix_len: int = 0, update_mode: str = "all",
                       temperature: float = 0.0, uniforms=None):
    """The part of one TR step after the target's forward pass, in the order
    the pages give ([Blog] "why recycling" loop: query M, build the tree,
    verify, accept the longest path, recycle every node's top-k):

      top-k of every node -> verify -> update M -> commit -> next root = bonus
      -> retrieve the next tree from the updated M.

    The tree of this step was retrieved from M before the update ([Blog]
    workflow step 2: the old matrix builds the tree, the update serves the
    next round).  Mutates M (and the caches when given).  Returns the result
    and the new prefix length.  update_mode "accepted" takes the ablation
    that recycles only the accepted path's top-k (update_accepted).  A
    temperature above 0 verifies by sampling (verify_sample, with the given
    uniforms [T][2]); the update still recycles each node's top-k.
    """
    top = topk_rows(logits, k)
    if temperature > 0:
        v = verify_sample(t, tok, logits, temperature, uniforms)
    else:
        v = verify(t, tok, top[:, 0])
    if update_mode == "accepted":
        update_accepted(M, tok, top, v.path)
    else:
        update(M, tok, top)
    if k_cache is not None:
        prefix_len = commit(k_cache, v_cache, k_tree, v_tree, prefix_len, v.path)
    nxt = retrieve(t, M, v.bonus)
    return StepResult(tok, top, v, nxt), prefix_len


def storage_bytes(V: int, k: int, itemsize: int) -> int:
    """Extra storage of TR: the |V| x k matrix of token ids ([Blog] storage
    section; [TR-en] summary, under 2 MB)."""
    return V * k * itemsize
