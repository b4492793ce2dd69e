"""Pins of the CPU oracle against what the pages and mathematics fix.

Each test pins the oracle to something other than itself: the worked example
printed by the Token Recycling walk-through, closed forms, brute-force
definitions written a different way, and special cases that reduce to a
textbook or library routine.  CPU only.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import tr_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def load_example():
    with open(os.path.join(GOLDEN, "worked_example.json")) as f:
        ex = json.load(f)
    ids = {name: i for i, name in enumerate(ex["vocab"])}
    V, k = len(ex["vocab"]), ex["k"]
    M = np.full((V, k), ids["pad"], dtype=np.int64)
    for name, row in ex["M_pre"].items():
        M[ids[name]] = [ids[x] for x in row]
    logits = np.zeros((len(ex["logits"]), V), dtype=np.float32)
    for n, row in enumerate(ex["logits"]):
        for name, val in row.items():
            logits[n, ids[name]] = val
    return ex, ids, M, logits


# ---------------------------------------------------------------- worked example
def test_worked_example_template():
    ex, ids, M, _ = load_example()
    t = O.template_from_levels(ex["levels"])
    assert t.parent.tolist() == ex["parent"]
    assert t.rank.tolist() == ex["rank"]


def test_worked_example_retrieval_gives_merged_sequence():
    ex, ids, M, _ = load_example()
    t = O.template_from_levels(ex["levels"])
    tok = O.retrieve(t, M, ids[ex["root"]])
    assert [ex["vocab"][x] for x in tok] == ex["merged_sequence"]


def test_worked_example_mask():
    ex, ids, M, _ = load_example()
    t = O.template_from_levels(ex["levels"])
    tok = O.retrieve(t, M, ids[ex["root"]])
    mask = O.ancestor_mask(t)
    names = ex["merged_sequence"]
    for node_name, seen in ex["visible"].items():
        n = names.index(node_name)
        assert sorted(names[j] for j in np.flatnonzero(mask[n])) == sorted(seen)
    # siblings never see each other (speaker/speak/event; at/for)
    for a, b in ((1, 2), (1, 3), (2, 3), (4, 5)):
        assert not mask[a, b] and not mask[b, a]


def test_worked_example_verify_and_update():
    ex, ids, M, logits = load_example()
    t = O.template_from_levels(ex["levels"])
    tok = O.retrieve(t, M, ids[ex["root"]])
    res, _ = O.step_after_forward(t, M, tok, logits, ex["k"])
    e = ex["expected"]
    assert res.verdict.accept_len == e["accept_len"]
    assert res.verdict.path.tolist() == e["path"]
    assert ex["vocab"][res.verdict.bonus] == e["bonus"]
    assert [ex["vocab"][x] for x in res.verdict.emitted] == e["emitted"]
    for name, row in e["M_post"].items():
        assert [ex["vocab"][x] for x in M[ids[name]]] == row, name
    # rows of tokens outside the tree are untouched
    for name in ex["vocab"]:
        if name not in e["M_post"]:
            assert (M[ids[name]] == ids["pad"]).all()
    assert [ex["vocab"][x] for x in res.next_tok] == e["next_tree"]


def test_storage_closed_form():
    # V=32000, K=8, 64-bit ids: exactly 2,048,000 bytes, about 1.95 MiB, under 2 MB (MiB)
    assert O.storage_bytes(32000, 8, 8) == 2_048_000
    assert np.zeros((32000, 8), dtype=np.int64).nbytes == 2_048_000
    assert abs(2_048_000 / 2 ** 20 - 1.953) < 1e-3


# ---------------------------------------------------------------- templates
def test_workload_trees():
    from synth.workloads import TREE_16, TREE_81
    t16 = O.template_from_levels(TREE_16)
    assert t16.n_nodes == 16 and t16.max_depth == 3
    # rank-0 chain 0 -> 1 -> 5 -> 13
    assert [t16.parent[13], t16.parent[5], t16.parent[1]] == [5, 1, 0]
    assert t16.rank[13] == t16.rank[5] == t16.rank[1] == 0
    t81 = O.template_from_levels(TREE_81)
    assert t81.n_nodes == 81 and t81.max_depth == 6
    assert np.bincount(t81.depth).tolist() == [1, 8, 20, 22, 18, 10, 2]
    # imbalanced: within a layer, child counts never increase
    for d in range(6):
        layer = np.flatnonzero(t81.depth == d)
        counts = [len(t81.children(n)) for n in layer]
        assert counts == sorted(counts, reverse=True)


def random_levels(rng, k, max_depth=4, max_nodes=24):
    levels, width = [], 1
    for _ in range(rng.integers(1, max_depth + 1)):
        counts = [int(rng.integers(0, k + 1)) for _ in range(width)]
        counts = sorted(counts, reverse=True)
        if sum(counts) == 0 or 1 + sum(sum(l) for l in levels) + sum(counts) > max_nodes:
            break
        levels.append(counts)
        width = sum(counts)
    return levels or [[1]]


def test_mask_invariants_random():
    rng = np.random.default_rng(1)
    for _ in range(50):
        t = O.template_from_levels(random_levels(rng, 4))
        mask = O.ancestor_mask(t)
        for n in range(t.n_nodes):
            row = np.flatnonzero(mask[n])
            assert len(row) == t.depth[n] + 1
            assert row[0] == 0 and row[-1] == n and (row <= n).all()
            # a chain: each visible node's parent is visible too
            for j in row[1:]:
                assert mask[n, t.parent[j]]
            # siblings (other children of the same parent) are never visible
            if n:
                sib = [m for m in t.children(int(t.parent[n])) if m != n]
                assert not mask[n, sib].any()


def test_template_rejects_bad_input():
    with pytest.raises(ValueError):
        O.Template(np.array([-1, 1]), np.array([-1, 0]))        # parent after child
    with pytest.raises(ValueError):
        O.Template(np.array([-1, 0, 0]), np.array([-1, 0, 0]))  # duplicate rank
    with pytest.raises(ValueError):
        O.Template(np.array([-1, 0, 1, 0]), np.array([-1, 0, 0, 1]))  # not layer order


# ---------------------------------------------------------------- retrieval
def retrieve_recursive(t, M, root):
    """Brute-force definition: expand the tree depth-first, recursively."""
    tok = {}

    def expand(n, token):
        tok[n] = token
        for c in t.children(n):
            expand(c, M[token, t.rank[c]])
    expand(0, root)
    return np.array([tok[n] for n in range(t.n_nodes)])


def test_retrieve_matches_recursive_definition():
    rng = np.random.default_rng(2)
    for _ in range(100):
        k = int(rng.integers(1, 5))
        V = int(rng.integers(2, 12))
        t = O.template_from_levels(random_levels(rng, k))
        M = rng.integers(0, V, size=(V, k))
        root = int(rng.integers(0, V))
        assert (O.retrieve(t, M, root) == retrieve_recursive(t, M, root)).all()


# ---------------------------------------------------------------- top-k
def topk_full_sort(z, k):
    return [i for _, i in sorted(((-float(z[i]), i) for i in range(len(z))))[:k]]


def test_topk_matches_full_sort_with_ties():
    rng = np.random.default_rng(3)
    for _ in range(300):
        V = int(rng.integers(1, 60))
        k = int(rng.integers(1, V + 1))
        z = rng.integers(-3, 4, size=V).astype(np.float32) * 0.5     # many ties
        if rng.random() < 0.3:
            z[rng.integers(0, V, size=max(1, V // 4))] = -0.0
        if rng.random() < 0.2:
            z[rng.integers(0, V)] = np.inf
        if rng.random() < 0.2:
            z[rng.integers(0, V)] = -np.inf
        assert O.topk_row(z, k).tolist() == topk_full_sort(z, k)


def test_topk_signed_zero_and_infinities():
    z = np.array([-0.0, 0.0, -np.inf, -0.0, np.inf, -np.inf], dtype=np.float32)
    assert O.topk_row(z, 4).tolist() == [4, 0, 1, 3]
    assert O.topk_row(z, 6).tolist() == [4, 0, 1, 3, 2, 5]


def test_topk_bf16_rows_invariants():
    g = torch.Generator().manual_seed(4)
    Z = (torch.randn((8, 32000), generator=g) * 3).to(torch.bfloat16).float().numpy()
    for z in Z:
        ids = O.topk_row(z, 8)
        assert len(set(ids.tolist())) == 8
        rest = np.delete(z, ids)
        assert z[ids].min() >= rest.max()
        for a, b in zip(ids[:-1], ids[1:]):
            assert z[a] > z[b] or (z[a] == z[b] and a < b)
        assert ids.tolist() == topk_full_sort(z, 8)


# ---------------------------------------------------------------- verification
def verify_enumerate(t, tok, greedy):
    """Brute force: enumerate every root-to-node path, keep the correct ones
    (each token equals the target's greedy token after its predecessor), pick
    the longest, ties to the smaller end node."""
    best = (0, 0)
    for n in range(t.n_nodes):
        path = t.ancestors[n]
        ok = all(tok[path[i + 1]] == greedy[path[i]] for i in range(len(path) - 1))
        if ok and (len(path) - 1, -n) > (best[0], -best[1]):
            best = (len(path) - 1, n)
    L, n = best
    return L, list(t.ancestors[n]), int(greedy[n])


def test_verify_matches_path_enumeration():
    rng = np.random.default_rng(5)
    for _ in range(300):
        k = int(rng.integers(1, 5))
        V = int(rng.integers(2, 6))            # tiny vocab: many matches and duplicates
        t = O.template_from_levels(random_levels(rng, k))
        tok = rng.integers(0, V, size=t.n_nodes)
        greedy = rng.integers(0, V, size=t.n_nodes)
        v = O.verify(t, tok, greedy)
        L, path, bonus = verify_enumerate(t, tok, greedy)
        assert (v.accept_len, v.path.tolist(), v.bonus) == (L, path, bonus)
        assert v.emitted.tolist() == [int(tok[x]) for x in path[1:]] + [bonus]


def linear_greedy_loop(draft, target_next):
    """The draft/verify loop with the bonus token, greedy form: accept drafts
    while they equal the target's token; on the first miss emit the target's
    token and stop; if every draft passed, emit the target's next token."""
    out = []
    for j, tokn in enumerate(draft):
        if tokn == target_next[j]:
            out.append(tokn)
        else:
            out.append(target_next[j])
            break
    else:
        out.append(target_next[len(draft)])
    return out


def test_chain_tree_reduces_to_linear_loop():
    rng = np.random.default_rng(6)
    for gamma in range(1, 6):
        t = O.template_from_levels([[1]] * gamma)
        for _ in range(100):
            tok = rng.integers(0, 3, size=gamma + 1)
            greedy = rng.integers(0, 3, size=gamma + 1)
            v = O.verify(t, tok, greedy)
            assert v.emitted.tolist() == linear_greedy_loop(tok[1:].tolist(), greedy.tolist())


def test_expected_tokens_per_pass_closed_form():
    # (1 - a^(g+1)) / (1 - a) at a=0.8, g=4 is about 3.4 tokens per target pass
    alpha, gamma, trials = 0.8, 4, 40000
    expect = (1 - alpha ** (gamma + 1)) / (1 - alpha)
    assert abs(expect - 3.3616) < 1e-9
    rng = np.random.default_rng(7)
    t = O.template_from_levels([[1]] * gamma)
    total = 0
    for _ in range(trials):
        tok = np.arange(gamma + 1) + 10
        hit = rng.random(gamma) < alpha
        greedy = np.where(np.append(hit, False), np.append(tok[1:], 0), 0)
        total += len(O.verify(t, tok, greedy).emitted)
    assert abs(total / trials - expect) < 0.03


# ---------------------------------------------------------------- sampling verification
def _inverse_cdf(dist, r):
    return int(np.searchsorted(np.cumsum(dist), r, side="right"))


def _speculative_loop(p, draft, u_acc, u_res):
    """The draft/verify loop of the speculative-decoding lesson ([SD]) for
    one chain of drafts, with the draft distribution q a point mass on each
    drafted token: accept with min(1, p/q), else resample from the
    normalised positive part of p - q and stop, else the bonus from the
    last position."""
    V = p.shape[1]
    out = []
    for j, x in enumerate(draft):
        q = np.zeros(V)
        q[x] = 1.0
        if u_acc[j] < min(1.0, p[j][x] / q[x]):
            out.append(int(x))
        else:
            res = np.maximum(0.0, p[j] - q)
            out.append(_inverse_cdf(res / res.sum(), u_res[j]))
            return out
    out.append(_inverse_cdf(p[len(draft)], u_res[len(draft)]))
    return out


def test_sample_chain_is_the_speculative_loop():
    rng = np.random.default_rng(41)
    for trial in range(400):
        g = int(rng.integers(0, 6))
        t = O.template_from_levels([[1]] * g)
        V = int(rng.integers(2, 9))
        temp = float(rng.choice([0.5, 1.0, 2.0]))
        z = rng.standard_normal((g + 1, V)) * 2
        tok = rng.integers(0, V, size=g + 1)
        for j in range(g):                    # make acceptance likely on most positions
            if rng.random() < 0.7:
                z[j, tok[j + 1]] += 4.0
        u = rng.random((g + 1, 2))
        v = O.verify_sample(t, tok, z, temp, u)
        p = O.softmax_rows(z, temp)
        want = _speculative_loop(p, tok[1:], u[1:, 0], u[:, 1])
        assert v.emitted.tolist() == want, trial
        assert v.accept_len == len(want) - 1 and v.path.tolist() == list(range(len(want)))
        assert v.bonus == want[-1]


def _lossless_tree():
    # root with children carrying tokens 2, 0, 2 (a duplicate); child 0
    # has one child; V = 5
    t = O.template_from_levels([[3], [1, 0, 0]])
    tok = np.array([4, 2, 0, 2, 1])
    z = np.array([[0.3, 0.9, 1.1, -0.4, 0.2],
                  [0.5, -0.2, 0.1, 0.8, 0.0],
                  [1.0, 0.0, -1.0, 0.5, 0.2],
                  [0.0, 0.4, 0.3, -0.6, 0.9],
                  [0.2, 0.2, 0.7, -0.1, 0.0]])
    return t, tok, z


def _chi2(counts, probs):
    n = counts.sum()
    return float(((counts - n * probs) ** 2 / (n * probs)).sum())


def test_sample_is_lossless():
    # Emitted tokens follow the target: the first ~ p_root whatever the
    # drafts, and after an accepted draft the next ~ p of that node
    # (Stern, Leviathan and Chen, as the speculative-decoding lesson states).
    t, tok, z = _lossless_tree()
    temp, N = 1.0, 40000
    rng = np.random.default_rng(42)
    p = O.softmax_rows(z, temp)
    first = np.zeros(5)
    second = {2: np.zeros(5), 0: np.zeros(5)}      # after token 2 (node 1), token 0 (node 2)
    for _ in range(N):
        v = O.verify_sample(t, tok, z, temp, rng.random((5, 2)))
        first[v.emitted[0]] += 1
        if v.emitted[0] in second:
            assert len(v.emitted) >= 2               # a drafted token is only ever accepted
            second[v.emitted[0]][v.emitted[1]] += 1
    assert _chi2(first, p[0]) < 18.47                # 4 degrees of freedom, p = 0.001
    assert _chi2(second[2], p[1]) < 18.47
    assert _chi2(second[0], p[2]) < 18.47


def test_sample_low_temperature_is_greedy():
    # As the temperature falls, p becomes the point mass on the argmax, and
    # the walk accepts exactly the children carrying their parent's argmax.
    # Siblings carry distinct tokens here: with a duplicate the walk
    # descends into the first accepted sibling, greedy verification into
    # the one with the deepest accepted node.
    rng = np.random.default_rng(43)
    for trial in range(200):
        levels = random_levels(rng, 3)
        t = O.template_from_levels(levels)
        T, V = t.n_nodes, 7
        z = np.stack([rng.permutation(V) * 0.1 for _ in range(T)])   # distinct, 0.1 apart
        arg = np.argmax(z, axis=1)
        tok = rng.integers(0, V, size=T)
        for n in range(T):
            ch = t.children(n)
            if not ch:
                continue
            pick = rng.permutation(V)[:len(ch)]
            if rng.random() < 0.7 and arg[n] not in pick:
                pick[rng.integers(len(ch))] = arg[n]
            tok[ch] = pick
        u = rng.uniform(1e-9, 1 - 1e-9, size=(T, 2))
        v = O.verify_sample(t, tok, z, 1e-3, u)
        g = O.verify(t, tok, arg)
        assert v.path.tolist() == g.path.tolist() and v.bonus == g.bonus, trial
        assert v.emitted.tolist() == g.emitted.tolist()


# ---------------------------------------------------------------- LM head
def test_lmhead_logits_brute_force_and_one_hot_rows():
    rng = np.random.default_rng(81)
    h = rng.standard_normal((3, 5))
    W = rng.standard_normal((7, 5))
    z = O.lmhead_logits(h, W)
    for r in range(3):
        for v in range(7):
            assert abs(z[r, v] - sum(h[r, j] * W[v, j] for j in range(5))) < 1e-12
    # one-hot rows of W pick hidden coordinates: row v = e_(v mod 5)
    E = np.eye(5)[[v % 5 for v in range(7)]]
    np.testing.assert_array_equal(O.lmhead_logits(h, E), h[:, [v % 5 for v in range(7)]])


# ---------------------------------------------------------------- update
def test_update_last_writer_wins_brute_force():
    rng = np.random.default_rng(8)
    for _ in range(200):
        V, k, T = 6, 3, int(rng.integers(1, 12))
        M = rng.integers(0, V, size=(V, k))
        M0 = M.copy()
        tok = rng.integers(0, V, size=T)                 # many duplicated tokens
        top = rng.integers(0, V, size=(T, k))
        O.update(M, tok, top)
        for v in range(V):
            writers = [n for n in range(T) if tok[n] == v]
            want = top[max(writers)] if writers else M0[v]
            assert (M[v] == want).all()


def test_worked_example_accepted_only_update():
    # The ablation that recycles only the accepted tokens: of the page's
    # post-step rows, those of the accepted path guest -> speaker -> at are
    # written; speak (rejected) keeps its old row, event/for/ing stay empty.
    ex, ids, M, logits = load_example()
    t = O.template_from_levels(ex["levels"])
    tok = O.retrieve(t, M, ids[ex["root"]])
    res, _ = O.step_after_forward(t, M, tok, logits, ex["k"], update_mode="accepted")
    e = ex["expected"]
    assert res.verdict.path.tolist() == e["path"]
    for name in ("guest", "speaker", "at"):
        assert [ex["vocab"][x] for x in M[ids[name]]] == e["M_post"][name], name
    assert [ex["vocab"][x] for x in M[ids["speak"]]] == ex["M_pre"]["speak"]
    for name in ex["vocab"]:
        if name not in ex["M_pre"]:
            assert (M[ids[name]] == ids["pad"]).all(), name
    assert [ex["vocab"][x] for x in res.next_tok] == e["next_tree"]


def test_update_accepted_brute_force():
    # Expected rows from the definitions written another way: a node is
    # accepted when every edge above it carries its parent's argmax; best is
    # the deepest accepted node (lowest index on ties); the writers of token
    # v are the ancestors of best (itself included) carrying v, and the
    # deepest of them wins.
    rng = np.random.default_rng(18)
    for trial in range(300):
        levels = random_levels(rng, 3)
        t = O.template_from_levels(levels)
        T, V, k = t.n_nodes, 5, 3
        z = rng.standard_normal((T, V))
        arg = np.argmax(z, axis=1)
        tok = rng.integers(0, V, size=T)
        for n in range(1, T):                       # accept most edges
            if rng.random() < 0.7:
                tok[n] = arg[t.parent[n]]
        M = rng.integers(0, V, size=(V, k))
        M0 = M.copy()
        O.step_after_forward(t, M, tok.copy(), z, k, update_mode="accepted")

        def chain(n):
            out = [n]
            while out[-1] != 0:
                out.append(int(t.parent[out[-1]]))
            return out[::-1]

        acc = [n for n in range(T) if all(tok[c] == arg[t.parent[c]] for c in chain(n)[1:])]
        best = min(acc, key=lambda n: (-len(chain(n)), n))
        on_path = chain(best)
        top = np.argsort(-z, axis=1, kind="stable")[:, :k]
        for v in range(V):
            writers = [n for n in on_path if tok[n] == v]
            want = top[writers[-1]] if writers else M0[v]
            assert (M[v] == want).all(), (trial, v)


def test_update_accepted_equals_update_on_a_fully_accepted_chain():
    # a chain tree whose every draft is accepted: the path is the whole tree
    rng = np.random.default_rng(19)
    for _ in range(50):
        n, V, k = int(rng.integers(1, 8)), 6, 3
        t = O.template_from_levels([[1]] * (n - 1))
        z = rng.standard_normal((n, V))
        tok = np.empty(n, dtype=np.int64)
        tok[0] = rng.integers(0, V)
        tok[1:] = np.argmax(z, axis=1)[:-1]
        Ma = rng.integers(0, V, size=(V, k))
        Mb = Ma.copy()
        ra, _ = O.step_after_forward(t, Ma, tok.copy(), z, k)
        rb, _ = O.step_after_forward(t, Mb, tok.copy(), z, k, update_mode="accepted")
        assert ra.verdict.accept_len == n - 1
        assert (Ma == Mb).all() and (ra.next_tok == rb.next_tok).all()


# ---------------------------------------------------------------- initial M
def test_splitmix64_published_outputs():
    # the first three outputs of SplitMix64 from state 0, as printed with
    # the generator's published reference code
    assert [int(x) for x in O.splitmix64(0, [0, 1, 2])] == [
        0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_init_random_power_of_two_vocab_takes_top_bits():
    # floor(u * 2^m / 2^32) with u the high word is the top m bits of the draw
    for m in (1, 8, 13):
        M = O.init_matrix(2, 2 ** m, 3, "random", seed=77)
        z = O.splitmix64(77, np.arange(2 * 2 ** m * 3, dtype=np.uint64))
        assert (M.reshape(-1) == (z >> np.uint64(64 - m)).astype(np.int64)).all()


def test_init_random_is_uniform_over_the_vocabulary():
    V, n = 7, 7 * 3 * 4000
    M = O.init_matrix(4, V, 3 * 1000, "random", seed=3)
    counts = np.bincount(M.reshape(-1), minlength=V)
    assert M.min() >= 0 and M.max() < V and counts.sum() == n
    chi2 = float(((counts - n / V) ** 2 / (n / V)).sum())
    assert chi2 < 22.5                  # 6 degrees of freedom, p = 0.001
    assert not (O.init_matrix(4, V, 3000, "random", seed=4) == M).all()


def test_init_zero_and_prior():
    assert (O.init_matrix(3, 5, 2, "zero") == 0).all()
    rng = np.random.default_rng(5)
    one = rng.integers(0, 50, size=(1, 50, 4))
    M = O.init_matrix(3, 50, 4, "prior", one)
    assert all((M[b] == one[0]).all() for b in range(3))
    each = rng.integers(0, 50, size=(3, 50, 4))
    assert (O.init_matrix(3, 50, 4, "prior", each) == each).all()


# ---------------------------------------------------------------- attention
def attention_per_path(t, q, kt, vt, kc, vc, P, scale):
    """Textbook attention for one node at a time: its key sequence is the
    prefix followed by the tree nodes on its own path; plain loops."""
    T, Hq, d = q.shape
    G = Hq // kt.shape[1]
    out = np.zeros((T, Hq, d))
    for n in range(T):
        for h in range(Hq):
            kh = h // G
            keys = [kc[kh, j] for j in range(P)] + [kt[j, kh] for j in t.ancestors[n]]
            vals = [vc[kh, j] for j in range(P)] + [vt[j, kh] for j in t.ancestors[n]]
            s = [float(np.dot(q[n, h], kk)) * scale for kk in keys]
            m = max(s)
            w = [math.exp(x - m) for x in s]
            tot = sum(w)
            out[n, h] = sum(wi * vv for wi, vv in zip(w, vals)) / tot
    return out


def rand_attn(rng, T, Hq, Hkv, d, P, cap=None):
    cap = cap or P + 3
    return (rng.standard_normal((T, Hq, d)), rng.standard_normal((T, Hkv, d)),
            rng.standard_normal((T, Hkv, d)), rng.standard_normal((Hkv, cap, d)),
            rng.standard_normal((Hkv, cap, d)))


def test_attention_matches_per_path_brute_force():
    rng = np.random.default_rng(9)
    for levels, Hq, Hkv, P in (([[3], [2, 1]], 2, 2, 5), ([[2], [2, 1], [1]], 4, 2, 0),
                               ([[4], [1, 1, 1, 1]], 6, 3, 3)):
        t = O.template_from_levels(levels)
        q, kt, vt, kc, vc = rand_attn(rng, t.n_nodes, Hq, Hkv, 8, P)
        got = O.tree_attention(t, q, kt, vt, kc, vc, P, 0.3)
        want = attention_per_path(t, q, kt, vt, kc, vc, P, 0.3)
        np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def _paged_copy(rng, caches, page_size, spare=3):
    """Page pools [num_pages][Hkv][page_size][d] holding each of `caches`
    [Hkv][cap][d] in the same shuffled pages (spare pages hold junk), and
    the block table."""
    Hkv, cap, d = caches[0].shape
    n = -(-cap // page_size)
    table = rng.permutation(n + spare)[:n]
    pools = []
    for cache in caches:
        pool = rng.standard_normal((n + spare, Hkv, page_size, d)) * 100.0
        for pos in range(cap):
            pool[table[pos // page_size], :, pos % page_size, :] = cache[:, pos, :]
        pools.append(pool)
    return pools, table


def test_paged_attention_equals_contiguous_under_any_page_order():
    rng = np.random.default_rng(61)
    for levels, Hq, Hkv, P, ps in (([[3], [2, 1]], 4, 2, 11, 4), ([[2], [1, 1]], 2, 2, 7, 3),
                                   ([[1]] * 3, 2, 1, 1, 2), ([[4]], 2, 2, 0, 5)):
        t = O.template_from_levels(levels)
        q, kt, vt, kc, vc = rand_attn(rng, t.n_nodes, Hq, Hkv, 8, P, cap=P + 5)
        (kp, vp), table = _paged_copy(rng, [kc, vc], ps)
        want = O.tree_attention(t, q, kt, vt, kc, vc, P)
        got = O.tree_attention_paged(t, q, kt, vt, kp, vp, table, ps, P)
        np.testing.assert_array_equal(got, want)


def test_commit_paged_is_commit_per_layer():
    rng = np.random.default_rng(62)
    layers, T, Hkv, d, ps, cap = 3, 7, 2, 4, 4, 16
    kt = rng.standard_normal((layers, T, Hkv, d))
    vt = rng.standard_normal((layers, T, Hkv, d))
    table = rng.permutation(6)[:cap // ps]
    kp = np.zeros((layers, 6, Hkv, ps, d))
    vp = np.zeros_like(kp)
    kc = np.zeros((layers, Hkv, cap, d))
    vc = np.zeros_like(kc)
    P, path = 3, [0, 2, 5, 6]                   # rows 3..6 span two pages
    newP = O.commit_paged(kp, vp, kt, vt, table, ps, P, path)
    for layer in range(layers):
        for i, n in enumerate(path):              # position P+i: page table[(P+i) // ps], row (P+i) % ps
            pg, r = table[(P + i) // ps], (P + i) % ps
            np.testing.assert_array_equal(kp[layer, pg, :, r], kt[layer, n])
            np.testing.assert_array_equal(vp[layer, pg, :, r], vt[layer, n])
        assert O.commit(kc[layer], vc[layer], kt[layer], vt[layer], P, path) == newP == P + 4
        np.testing.assert_array_equal(O.gather_pages(kp[layer], table, ps, cap), kc[layer])
        np.testing.assert_array_equal(O.gather_pages(vp[layer], table, ps, cap), vc[layer])
    unused = [pg for pg in range(6) if pg not in table]
    assert (kp[:, unused] == 0).all()
    with pytest.raises(ValueError):
        O.commit_paged(kp, vp, kt, vt, table, ps, cap - 2, path)


def test_chain_tree_is_causal_attention():
    # a chain tree is ordinary causal attention over prefix ++ chain (library SDPA)
    rng = np.random.default_rng(10)
    T, H, d, P = 5, 3, 16, 7
    t = O.template_from_levels([[1]] * (T - 1))
    q, kt, vt, kc, vc = rand_attn(rng, T, H, H, d, P)
    got = O.tree_attention(t, q, kt, vt, kc, vc, P)
    Kseq = np.concatenate([kc[:, :P], kt.transpose(1, 0, 2)], axis=1)          # [H, P+T, d]
    Vseq = np.concatenate([vc[:, :P], vt.transpose(1, 0, 2)], axis=1)
    Qseq = np.concatenate([np.zeros((H, P, d)), q.transpose(1, 0, 2)], axis=1)  # queries at every position
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(Qseq)[None], torch.from_numpy(Kseq)[None], torch.from_numpy(Vseq)[None],
        is_causal=True)[0, :, P:].numpy().transpose(1, 0, 2)
    np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-12)


def test_single_node_is_decode_attention():
    rng = np.random.default_rng(11)
    t = O.template_from_levels([])
    q, kt, vt, kc, vc = rand_attn(rng, 1, 4, 4, 16, 9)
    got = O.tree_attention(t, q, kt, vt, kc, vc, 9)
    K = torch.from_numpy(np.concatenate([kc[:, :9], kt.transpose(1, 0, 2)], axis=1))
    V = torch.from_numpy(np.concatenate([vc[:, :9], vt.transpose(1, 0, 2)], axis=1))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q.transpose(1, 0, 2))[None], K[None], V[None])[0].numpy().transpose(1, 0, 2)
    np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-12)


def test_attention_ignores_non_ancestors():
    rng = np.random.default_rng(12)
    t = O.template_from_levels([[3], [2, 1], [1]])
    q, kt, vt, kc, vc = rand_attn(rng, t.n_nodes, 2, 1, 8, 4)
    base = O.tree_attention(t, q, kt, vt, kc, vc, 4)
    mask = O.ancestor_mask(t)
    for j in range(t.n_nodes):
        kt2, vt2 = kt.copy(), vt.copy()
        kt2[j] += 5.0
        vt2[j] -= 3.0
        out = O.tree_attention(t, q, kt2, vt2, kc, vc, 4)
        for n in range(t.n_nodes):
            if mask[n, j]:
                assert not np.allclose(out[n], base[n])
            else:
                assert (out[n] == base[n]).all()


def test_attention_gqa_grouping_uses_contiguous_heads():
    rng = np.random.default_rng(13)
    t = O.template_from_levels([[2]])
    q, kt, vt, kc, vc = rand_attn(rng, 3, 4, 2, 8, 3)
    out = O.tree_attention(t, q, kt, vt, kc, vc, 3)
    # heads 0,1 use kv head 0; heads 2,3 use kv head 1: compare with MHA on repeated kv
    mha = O.tree_attention(t, q, np.repeat(kt, 2, axis=1), np.repeat(vt, 2, axis=1),
                           np.repeat(kc, 2, axis=0), np.repeat(vc, 2, axis=0), 3)
    np.testing.assert_allclose(out, mha, rtol=1e-13)


# ---------------------------------------------------------------- whole loop
def test_lossless_first_order_target():
    """With a target whose greedy next token depends only on the last token,
    the stream the loop emits equals plain greedy decoding, token for token."""
    rng = np.random.default_rng(14)
    for trial in range(20):
        V, k = int(rng.integers(5, 40)), int(rng.integers(1, 5))
        t = O.template_from_levels(random_levels(rng, k, max_depth=4))
        H = rng.integers(0, V, size=V)
        M = rng.integers(0, V, size=(V, k))
        root = int(rng.integers(0, V))
        tok = O.retrieve(t, M, root)
        stream = []
        for s in range(15):
            logits = rng.standard_normal((t.n_nodes, V))
            logits[np.arange(t.n_nodes), H[tok]] = logits.max(axis=1) + 1.0
            res, _ = O.step_after_forward(t, M, tok, logits, k)
            stream += res.verdict.emitted.tolist()
            tok = res.next_tok
        greedy = [root]
        for _ in range(len(stream)):
            greedy.append(int(H[greedy[-1]]))
        assert stream == greedy[1:]


def test_commit_appends_path_rows():
    rng = np.random.default_rng(15)
    kc = np.zeros((2, 10, 4)); vc = np.zeros((2, 10, 4))
    kt = rng.standard_normal((5, 2, 4)); vt = rng.standard_normal((5, 2, 4))
    P = O.commit(kc, vc, kt, vt, 3, [0, 2, 4])
    assert P == 6
    assert (kc[:, 3] == kt[0]).all() and (kc[:, 4] == kt[2]).all() and (vc[:, 5] == vt[4]).all()
    assert (kc[:, :3] == 0).all() and (kc[:, 6:] == 0).all()
    with pytest.raises(ValueError):
        O.commit(kc, vc, kt, vt, 8, [0, 1, 2])
