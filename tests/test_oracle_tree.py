"""Pins for the oracle's DDTree builder (CPU only).

* brute force: sorting every prefix of the candidate universe by the
  canonical key and keeping the first B gives the heap's tree;
* optimality (DDTree page, method section): no prefix-closed tree of size B
  has a larger sum of prefix probabilities (exhaustive on tiny V/L; an
  independent tree-knapsack DP at the tiny-config scale);
* the theorem (same section): the sum of prefix probabilities equals the
  expected acceptance length, by exact enumeration of every target sequence;
* vanilla DFlash special case: k_tree = 1, B = L is the single top-1 path and
  its ancestor mask is the causal (lower-triangular) mask;
* a hand-worked dyadic example with exact ties (tests/golden/dyadic_tree.json);
* structural invariants on the workload-sized inputs.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

import synth
from oracle.logits import topk_logprobs
from oracle.tree import build_tree, expected_acceptance

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _random_table(rng, L, K, V=None):
    """Random sorted log-prob table with distinct token ids per row."""
    logp = np.stack([np.sort(np.log(rng.dirichlet(np.ones(K * 2))[:K]))[::-1]
                     for _ in range(L)]).astype(np.float32)
    V = V or 100
    ids = np.stack([rng.choice(V, size=K, replace=False) for _ in range(L)]).astype(np.int32)
    return logp, ids


def _universe(logp, k_tree):
    """Every rank tuple of depth 1..L with ranks < k_tree, with its float32
    score and a canonical sort key built recursively from the parent's key."""
    L = logp.shape[0]
    nodes = {(): ((), np.float32(0.0))}
    order = []
    for d in range(1, L + 1):
        for ranks in itertools.product(range(k_tree), repeat=d):
            par_key, par_score = nodes[ranks[:-1]]
            s = np.float32(par_score + logp[d - 1, ranks[-1]])
            key = (-float(s), d, par_key, ranks[-1])
            nodes[ranks] = (key, s)
            order.append(ranks)
    return nodes, order


@pytest.mark.parametrize("seed,L,K,k_tree,B", [
    (0, 3, 4, 4, 10), (1, 4, 3, 3, 30), (2, 2, 5, 5, 7), (3, 5, 2, 2, 20), (4, 3, 6, 3, 12),
    (5, 4, 4, 2, 15), (6, 1, 8, 8, 5), (7, 3, 3, 3, 39), (8, 3, 3, 3, 60)])
def test_heap_equals_sorted_universe(seed, L, K, k_tree, B):
    rng = np.random.default_rng(seed)
    logp, ids = _random_table(rng, L, K)
    if seed % 3 == 0:      # force exact score ties
        logp[:, 1] = logp[:, 0]
    t = build_tree(logp, ids, 7, k_tree, B)
    nodes, order = _universe(logp, k_tree)
    ranked = sorted(order, key=lambda rk: nodes[rk][0])[:B]
    assert t["n_nodes"] == len(ranked) + 1
    slot_of = {(): 0}
    for i, rk in enumerate(ranked, start=1):
        slot_of[rk] = i
        assert t["depth"][i] == len(rk)
        assert t["parent"][i] == slot_of[rk[:-1]]
        assert t["token"][i] == ids[len(rk) - 1, rk[-1]]
        assert t["score"][i] == nodes[rk][1]


def _prefix_prob(q, ranks):
    p = 1.0
    for d, r in enumerate(ranks):
        p *= q[d][r]
    return p


def _all_prefix_closed(L, k, size):
    """All prefix-closed sets of `size` non-empty rank tuples."""
    level = {frozenset()}
    for _ in range(size):
        nxt = set()
        for tree in level:
            frontier = [(r,) for r in range(k) if (r,) not in tree]
            for node in tree:
                if len(node) < L:
                    frontier += [node + (r,) for r in range(k) if node + (r,) not in tree]
            for f in frontier:
                nxt.add(tree | {f})
        level = nxt
    return level


@pytest.mark.parametrize("seed,L,V,B", [(0, 3, 3, 4), (1, 2, 4, 5), (2, 3, 2, 6), (3, 3, 3, 6)])
def test_top_b_is_optimal_over_all_trees(seed, L, V, B):
    rng = np.random.default_rng(100 + seed)
    q = [np.sort(rng.dirichlet(np.ones(V)))[::-1] for _ in range(L)]
    logp = np.array([np.log(qq) for qq in q], dtype=np.float32)
    ids = np.tile(np.arange(V, dtype=np.int32), (L, 1))
    t = build_tree(logp, ids, 0, V, B)
    ours = 0.0
    ranks_of = {0: ()}
    for s in range(1, t["n_nodes"]):
        rk = ranks_of[t["parent"][s]] + (int(t["token"][s]),)
        ranks_of[s] = rk
        ours += _prefix_prob(q, rk)
    best = max(sum(_prefix_prob(q, n) for n in tree) for tree in _all_prefix_closed(L, V, B))
    assert ours == pytest.approx(best, rel=1e-6, abs=1e-9)


def test_tree_knapsack_dp_matches_top_b_at_tiny_config():
    cfg = synth.CONFIGS[1]
    case = synth.make_case(cfg, with_drafter=False, with_verify=False)
    ids, logp, _ = topk_logprobs(case.logits, cfg.K)
    t = build_tree(logp, ids, int(case.root_token[0]), cfg.k_tree, cfg.B)
    L, k = cfg.L, cfg.k_tree
    w = np.exp(logp.astype(np.float64))

    # best[node][b]: largest value of a prefix-closed subtree hanging under
    # `node` (node itself excluded) that uses exactly b nodes.
    def best_under(ranks, p_node):
        d = len(ranks)
        NEG = -1.0
        table = [0.0] + [NEG] * cfg.B
        if d == L:
            return table
        for r in range(k):
            p_child = p_node * w[d, r]
            sub = best_under(ranks + (r,), p_child)
            child = [0.0] + [sub[b - 1] + p_child if sub[b - 1] >= 0 else NEG
                             for b in range(1, cfg.B + 1)]
            merged = [NEG] * (cfg.B + 1)
            for b1 in range(cfg.B + 1):
                if table[b1] < 0:
                    continue
                for b2 in range(cfg.B + 1 - b1):
                    if child[b2] >= 0:
                        merged[b1 + b2] = max(merged[b1 + b2], table[b1] + child[b2])
            table = merged
        return table

    dp = best_under((), 1.0)[cfg.B]
    ours = expected_acceptance(t["score"], t["n_nodes"])
    assert t["n_nodes"] == cfg.B + 1
    assert ours == pytest.approx(dp, rel=1e-6)


@pytest.mark.parametrize("seed,L,V,B", [(0, 3, 3, 5), (1, 3, 3, 13), (2, 4, 3, 20), (3, 2, 5, 9)])
def test_sum_of_prefix_probs_is_expected_acceptance(seed, L, V, B):
    rng = np.random.default_rng(200 + seed)
    q = [rng.dirichlet(np.ones(V)) for _ in range(L)]
    order = [np.argsort(-qq, kind="stable") for qq in q]
    logp = np.array([np.log(q[d][order[d]]) for d in range(L)], dtype=np.float32)
    ids = np.array(order, dtype=np.int32)
    t = build_tree(logp, ids, 0, V, B)
    n = t["n_nodes"]
    children = {}
    for s in range(1, n):
        children.setdefault(int(t["parent"][s]), {})[int(t["token"][s])] = s
    exact = 0.0
    for y in itertools.product(range(V), repeat=L):
        p = math.prod(q[d][y[d]] for d in range(L))
        cur, acc = 0, 0
        while acc < L and y[acc] in children.get(cur, {}):
            cur = children[cur][y[acc]]
            acc += 1
        exact += p * acc
    assert expected_acceptance(t["score"], n) == pytest.approx(exact, rel=2e-6)


def test_chain_tree_is_vanilla_dflash_path():
    cfg = synth.scaled(synth.CONFIGS[2], vocab=4000)
    case = synth.make_case(cfg, with_drafter=False, with_verify=False)
    ids, logp, _ = topk_logprobs(case.logits, cfg.K)
    t = build_tree(logp, ids, int(case.root_token[0]), 1, cfg.L)
    assert t["n_nodes"] == cfg.L + 1
    assert t["token"][1:].tolist() == [int(np.argmax(r)) for r in case.logits]
    assert t["parent"][1:].tolist() == list(range(cfg.L))
    assert t["depth"].tolist() == list(range(cfg.L + 1))
    N = cfg.L + 1
    dense = np.zeros((N, N), dtype=bool)
    for i in range(N):
        for j in range(N):
            dense[i, j] = (int(t["mask"][i, j // 64]) >> (j % 64)) & 1
    assert np.array_equal(dense, np.tril(np.ones((N, N), dtype=bool)))


def test_golden_dyadic_example():
    with open(os.path.join(GOLDEN, "dyadic_tree.json")) as f:
        g = json.load(f)
    inp, exp = g["inputs"], g["expected"]
    logp = np.array([[math.log(p) for p in row] for row in inp["probs"]], dtype=np.float32)
    ids = np.array(inp["ids"], dtype=np.int32)
    t = build_tree(logp, ids, inp["root_token"], inp["k_tree"], inp["budget"])
    assert t["n_nodes"] == exp["n_nodes"]
    assert t["token"].tolist() == exp["token"]
    assert t["parent"].tolist() == exp["parent"]
    assert t["depth"].tolist() == exp["depth"]
    assert [int(w) for w in t["mask"][:, 0]] == exp["mask_word0"]
    assert expected_acceptance(t["score"], t["n_nodes"]) == pytest.approx(
        exp["expected_acceptance"], rel=1e-6)


def test_short_tree_when_universe_smaller_than_budget():
    rng = np.random.default_rng(9)
    logp, ids = _random_table(rng, 2, 3)
    t = build_tree(logp, ids, 1, 2, 100)        # |U| = 2 + 4 = 6
    assert t["n_nodes"] == 7
    assert np.all(t["token"][7:] == -1) and np.all(t["parent"][7:] == -1)
    assert np.all(np.isneginf(t["score"][7:])) and np.all(t["mask"][7:] == 0)


def _check_structure(t, ids, k_tree):
    n = t["n_nodes"]
    tok, par, dep, sc, mask = t["token"], t["parent"], t["depth"], t["score"], t["mask"]
    assert par[0] == -1 and dep[0] == 0 and sc[0] == 0
    sib = {}
    for s in range(1, n):
        p = par[s]
        assert 0 <= p < s
        assert dep[s] == dep[p] + 1
        assert tok[s] in ids[dep[s] - 1, :k_tree]
        key = (int(p), int(tok[s]))
        assert key not in sib
        sib[key] = s
        assert sc[s] <= sc[p]
        assert sc[s] <= sc[s - 1]
        bits = sum(bin(int(w)).count("1") for w in mask[s])
        assert bits == dep[s] + 1
        for w in range(mask.shape[1]):
            assert int(mask[s, w]) & int(mask[p, w]) == int(mask[p, w])


@pytest.mark.parametrize("cfg", [synth.CONFIGS[3], synth.DEEP], ids=["c3", "deep"])
def test_structure_at_workload_size(cfg):
    case = synth.make_case(cfg, with_drafter=False, with_verify=False)
    ids, logp, _ = topk_logprobs(case.logits, cfg.K)
    t = build_tree(logp, ids, int(case.root_token[0]), cfg.k_tree, cfg.B)
    assert t["n_nodes"] == cfg.B + 1
    _check_structure(t, ids, cfg.k_tree)
    if cfg is synth.DEEP:
        assert t["depth"].max() == cfg.L
