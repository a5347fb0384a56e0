"""Oracle, step 2: the DDTree draft tree.

[DDTree] sections "핵심 아이디어" (core idea) and "방법론 자세히 보기" (method in
detail):
  * the per-position distributions are treated as independent (a factorized
    distribution over the block);
  * the value of a node is its prefix probability, the probability of the
    whole root-to-node path; expected acceptance length equals the sum of the
    prefix probabilities of all nodes in the tree, so the best tree of budget
    B is made of the B most probable prefixes;
  * those are found best-first with a max-heap (the OPT-Tree procedure
    extended to a single drafter call), B nodes in O(B log B);
  * the tree is flattened and verified in one target pass under an
    ancestor-only attention mask ("용어 정리" / glossary: each token sees only
    the tokens on its own ancestor path).

Readings where the page leaves a step open (each listed in the design notes):
  * the root (slot 0) is the bonus token, not counted in B;
  * position d (1-based depth) uses row d-1 of the top-K table, and the tree
    may branch only over ranks < k_tree of each row;
  * scores are float32 log-probabilities summed left to right:
    score(child) = fl32(score(parent) + logp[depth-1][rank]);
  * ties are broken by one total order, the canonical key
    (score desc, depth asc, parent slot asc, rank asc);
  * the flattened order is the pop order, so parents precede children;
  * "ancestor-only" includes the node itself and the root, so a chain tree
    gives ordinary causal attention.
"""
from __future__ import annotations

import heapq

import numpy as np


def build_tree(topk_logp: np.ndarray, topk_ids: np.ndarray, root_token: int,
               k_tree: int, budget: int):
    """Best-first top-B prefix tree for one request.

    topk_logp f32 [L, K] (non-increasing along K), topk_ids i32 [L, K].
    Returns a dict with n_nodes and arrays of length budget+1 (slot 0 = root,
    padding slots: token/parent/depth -1, score -inf) and the ancestor mask
    u64 [budget+1, ceil((budget+1)/64)].
    """
    y = np.asarray(topk_logp, dtype=np.float32)
    ids = np.asarray(topk_ids, dtype=np.int32)
    L, K = y.shape
    if not (1 <= k_tree <= K):
        raise ValueError("need 1 <= k_tree <= K")
    n_max = budget + 1

    token = [int(root_token)]
    parent = [-1]
    depth = [0]
    score = [np.float32(0.0)]

    # heap entries are the canonical key itself: (-score, depth, parent, rank)
    heap = []

    def push(par_slot: int, d: int, rank: int) -> None:
        s = np.float32(score[par_slot] + y[d - 1, rank])   # float32 addition
        heapq.heappush(heap, (-float(s), d, par_slot, rank))

    if budget > 0 and L > 0:
        push(0, 1, 0)
    while heap and len(token) - 1 < budget:
        neg_s, d, par, rank = heapq.heappop(heap)
        slot = len(token)
        token.append(int(ids[d - 1, rank]))
        parent.append(par)
        depth.append(d)
        score.append(np.float32(-neg_s))
        if rank + 1 < k_tree:          # next sibling under the same parent
            push(par, d, rank + 1)
        if d < L:                      # best child of the node just taken
            push(slot, d + 1, 0)

    n = len(token)
    out_token = np.full(n_max, -1, dtype=np.int32)
    out_parent = np.full(n_max, -1, dtype=np.int32)
    out_depth = np.full(n_max, -1, dtype=np.int32)
    out_score = np.full(n_max, -np.inf, dtype=np.float32)
    out_token[:n] = token
    out_parent[:n] = parent
    out_depth[:n] = depth
    out_score[:n] = score
    return {
        "n_nodes": n,
        "token": out_token,
        "parent": out_parent,
        "depth": out_depth,
        "score": out_score,
        "mask": ancestor_mask(out_parent, n, n_max),
    }


def ancestor_mask(parent: np.ndarray, n_nodes: int, n_max: int) -> np.ndarray:
    """mask[s] = mask[parent[s]] | {s}; mask[0] = {0}; padding rows are 0.
    Returned as little-endian u64 words [n_max, ceil(n_max/64)]."""
    W = (n_max + 63) // 64
    sets = [0] * n_max
    for s in range(n_nodes):
        p = int(parent[s])
        sets[s] = (sets[p] if s > 0 else 0) | (1 << s)
    out = np.zeros((n_max, W), dtype=np.uint64)
    for s in range(n_max):
        v = sets[s]
        for w in range(W):
            out[s, w] = (v >> (64 * w)) & 0xFFFFFFFFFFFFFFFF
    return out


def build_trees(topk_logp: np.ndarray, topk_ids: np.ndarray, root_token: np.ndarray,
                batch: int, L: int, k_tree: int, budget: int):
    """Batched wrapper: rows of request r are [r*L, (r+1)*L)."""
    res = [build_tree(topk_logp[r * L:(r + 1) * L], topk_ids[r * L:(r + 1) * L],
                      int(root_token[r]), k_tree, budget) for r in range(batch)]
    stack = {key: np.stack([t[key] for t in res]) for key in
             ("token", "parent", "depth", "score", "mask")}
    stack["n_nodes"] = np.array([t["n_nodes"] for t in res], dtype=np.int32)
    return stack


def expected_acceptance(score: np.ndarray, n_nodes: int) -> float:
    """Sum of prefix probabilities of the drafted nodes (root excluded), the
    quantity the DDTree page proves equal to the expected acceptance length
    under the factorized model."""
    s = np.asarray(score[1:n_nodes], dtype=np.float64)
    return float(np.exp(s).sum())
