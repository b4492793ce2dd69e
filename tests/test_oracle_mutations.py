"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each case swaps one oracle function for a plausibly wrong variant (dropped
term, wrong index, wrong tie rule, transposed operand) and runs the pins
that should catch it; the pins must fail.  The real oracle is restored
afterwards.
"""
import math

import numpy as np
import pytest

from oracle import tr_oracle as O
import tests.test_oracle_pins as P


def _bonus_from_parent(t, tok, greedy):
    v = ORIG["verify"](t, tok, greedy)
    par = v.path[-2] if len(v.path) > 1 else 0
    v.bonus = int(greedy[par])
    v.emitted = np.concatenate([tok[v.path[1:]], [v.bonus]])
    return v


def _first_match_walk(t, tok, greedy):
    # walks the first accepted child only (not the globally deepest node)
    n = 0
    while True:
        nxt = [c for c in t.children(n) if tok[c] == greedy[n]]
        if not nxt:
            break
        n = nxt[0]
    path = np.array(t.ancestors[n])
    return O.Verdict(len(path) - 1, path, int(greedy[n]),
                     np.concatenate([tok[path[1:]], [greedy[n]]]))


def _topk_ties_high_id(z, k):
    z = np.asarray(z, dtype=np.float64)
    ids = np.lexsort((-np.arange(len(z)), -z))[:k]
    return ids


def _update_first_writer(M, tok, topk):
    for n in reversed(range(len(tok))):
        M[tok[n], :] = topk[n, : M.shape[1]]


def _update_accepted_only_root(M, tok, topk):
    M[tok[0], :] = topk[0, : M.shape[1]]


def _accepted_shallow_wins(M, tok, topk, path):
    for n in reversed(list(path)):
        M[tok[n], :] = topk[n, : M.shape[1]]


def _accepted_without_root(M, tok, topk, path):
    for n in list(path)[1:]:
        M[tok[n], :] = topk[n, : M.shape[1]]


def _accepted_is_all(M, tok, topk, path):
    ORIG["update"](M, tok, topk)


def _splitmix_counter_from_zero(seed, e):
    # state seed + e*gamma instead of seed + (e+1)*gamma
    return ORIG["splitmix64"](seed - 0x9E3779B97F4A7C15, e)


def _splitmix_wrong_shift(seed, e):
    e = np.asarray(e, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = np.uint64(seed) + (e + np.uint64(1)) * np.uint64(0x9E3779B97F4A7C15)
        z = (z ^ (z >> np.uint64(31))) * np.uint64(0xBF58476D1CE4E5B9)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(0x94D049BB133111EB)
        return z ^ (z >> np.uint64(31))


def _init_low_word(B, V, k, mode, prior=None, seed=0):
    if mode != "random":
        return ORIG["init_matrix"](B, V, k, mode, prior, seed)
    z = O.splitmix64(seed, np.arange(B * V * k, dtype=np.uint64)) & np.uint64(0xFFFFFFFF)
    return ((z * np.uint64(V)) >> np.uint64(32)).astype(np.int64).reshape(B, V, k)


def _sampler(renormalise=True, residual_draw=True, swap_uniforms=False):
    # a compact walk with one of its parts done wrong
    def run(t, tok, logits, temperature, uniforms):
        p = O.softmax_rows(logits, temperature)
        V = p.shape[1]
        ua, ud = (1, 0) if swap_uniforms else (0, 1)
        n, path = 0, [0]
        while True:
            r, nxt = p[n].copy(), None
            for c in t.children(n):
                x = int(tok[c])
                if uniforms[c][ua] < min(1.0, r[x]):
                    nxt = c
                    break
                if renormalise:
                    r[x] = 0.0
                    r = r / r.sum()
            if nxt is None:
                dist = r if residual_draw else p[n]
                bonus = int(np.searchsorted(np.cumsum(dist), uniforms[n][ud], side="right"))
                bonus = min(bonus, V - 1)
                break
            n = nxt
            path.append(n)
        path = np.array(path)
        return O.Verdict(len(path) - 1, path, bonus,
                         np.concatenate([tok[path[1:]], [bonus]]).astype(np.int64))
    run.__name__ = ("_sample_no_residual_update" if not renormalise else
                    "_sample_draw_from_p" if not residual_draw else "_sample_swapped_uniforms")
    return run


def _page_slot_modulo(table_b, page_size, pos):
    # the page taken by position modulo the table length
    return int(table_b[pos % len(table_b)]), pos % page_size


def _page_slot_swapped(table_b, page_size, pos):
    return int(table_b[pos % page_size % len(table_b)]), pos // page_size % page_size


def _lmhead_drops_last_coordinate(h, W):
    return np.asarray(h, dtype=np.float64)[:, :-1] @ np.asarray(W, dtype=np.float64)[:, :-1].T


def _retrieve_rank_off(t, M, root):
    tok = np.empty(t.n_nodes, dtype=np.int64)
    tok[0] = root
    for n in range(1, t.n_nodes):
        tok[n] = M[tok[t.parent[n]], min(t.rank[n] + 1, M.shape[1] - 1)]
    return tok


def _mask_without_self(t):
    m = ORIG["ancestor_mask"](t)
    np.fill_diagonal(m, False)
    m[0, 0] = True
    return m


def _attention_no_scale(t, q, kt, vt, kc, vc, P_, scale=None):
    return ORIG["tree_attention"](t, q, kt, vt, kc, vc, P_, 1.0)


def _attention_wrong_group(t, q, kt, vt, kc, vc, P_, scale=None):
    # interleaved instead of contiguous head groups
    Hq, Hkv = q.shape[1], kt.shape[1]
    perm = [(h % Hkv) * (Hq // Hkv) + h // Hkv for h in range(Hq)]
    return ORIG["tree_attention"](t, q[:, perm], kt, vt, kc, vc, P_, scale)[:, np.argsort(perm)]


ORIG = {name: getattr(O, name) for name in
        ("verify", "topk_row", "update", "update_accepted", "retrieve", "ancestor_mask",
         "tree_attention", "splitmix64", "init_matrix", "verify_sample", "page_slot",
         "lmhead_logits")}

CASES = [
    ("verify", _bonus_from_parent, [P.test_worked_example_verify_and_update,
                                    P.test_verify_matches_path_enumeration,
                                    P.test_lossless_first_order_target]),
    ("verify", _first_match_walk, [P.test_verify_matches_path_enumeration]),
    ("topk_row", _topk_ties_high_id, [P.test_topk_matches_full_sort_with_ties]),
    ("update", _update_first_writer, [P.test_update_last_writer_wins_brute_force]),
    ("update", _update_accepted_only_root, [P.test_worked_example_verify_and_update]),
    ("update_accepted", _accepted_shallow_wins, [P.test_update_accepted_brute_force]),
    ("update_accepted", _accepted_without_root, [P.test_worked_example_accepted_only_update,
                                                 P.test_update_accepted_brute_force]),
    ("update_accepted", _accepted_is_all, [P.test_worked_example_accepted_only_update,
                                           P.test_update_accepted_brute_force]),
    ("splitmix64", _splitmix_counter_from_zero, [P.test_splitmix64_published_outputs]),
    ("splitmix64", _splitmix_wrong_shift, [P.test_splitmix64_published_outputs]),
    ("init_matrix", _init_low_word, [P.test_init_random_power_of_two_vocab_takes_top_bits]),
    ("verify_sample", _sampler(renormalise=False), [P.test_sample_chain_is_the_speculative_loop,
                                                     P.test_sample_is_lossless]),
    ("verify_sample", _sampler(residual_draw=False), [P.test_sample_chain_is_the_speculative_loop,
                                                      P.test_sample_is_lossless]),
    ("verify_sample", _sampler(swap_uniforms=True), [P.test_sample_chain_is_the_speculative_loop]),
    ("page_slot", _page_slot_modulo, [P.test_paged_attention_equals_contiguous_under_any_page_order,
                                      P.test_commit_paged_is_commit_per_layer]),
    ("page_slot", _page_slot_swapped, [P.test_paged_attention_equals_contiguous_under_any_page_order,
                                       P.test_commit_paged_is_commit_per_layer]),
    ("lmhead_logits", _lmhead_drops_last_coordinate, [P.test_lmhead_logits_brute_force_and_one_hot_rows]),
    ("retrieve", _retrieve_rank_off, [P.test_worked_example_retrieval_gives_merged_sequence,
                                      P.test_retrieve_matches_recursive_definition]),
    ("ancestor_mask", _mask_without_self, [P.test_worked_example_mask,
                                           P.test_mask_invariants_random,
                                           P.test_attention_matches_per_path_brute_force]),
    ("tree_attention", _attention_no_scale, [P.test_chain_tree_is_causal_attention,
                                             P.test_single_node_is_decode_attention]),
    ("tree_attention", _attention_wrong_group, [P.test_attention_gqa_grouping_uses_contiguous_heads,
                                                P.test_attention_matches_per_path_brute_force]),
]


@pytest.mark.parametrize("name,bad,pins", CASES, ids=[f"{c[0]}:{c[1].__name__}" for c in CASES])
def test_planted_mistake_is_caught(monkeypatch, name, bad, pins):
    monkeypatch.setattr(O, name, bad)
    for pin in pins:
        with pytest.raises(AssertionError):
            pin()
