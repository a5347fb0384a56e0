"""Oracle, step 4: greedy acceptance walk and KV-cache compaction.

[DDTree] "방법론 자세히 보기" (method in detail): the verifier compares the
target's outputs with the tree, accepts the longest path whose tokens the
target agrees with, and cleans the rejected branches out of the KV cache.
The general draft-then-verify rule (accept up to the first disagreement, the
target then supplies the next token) is the one both pages describe for
speculative decoding ([DFlash] "왜 기존 speculative decoding도 한계가
있었나", [DDTree] "이 논문을 고른 이유").

Definition (greedy verification; t[s] is the target's argmax after reading
tree slot s):
  cur = 0; path = [0]
  while some child c of cur has token[c] == t[cur]: append c, cur = c
  accept_len = len(path) - 1;  bonus = t[cur]
  for every layer: snapshot cache rows P + path[j] (j <= accept_len), then
  write them to rows P + j  (reads before writes: a destination row can be
  the source of a later path entry)
  new_len = P + accept_len + 1
"""
from __future__ import annotations

import numpy as np


def greedy_walk(node_token, node_parent, n_nodes: int, target, L: int):
    path = [0]
    cur = 0
    while len(path) <= L:
        nxt = -1
        for c in range(1, n_nodes):
            if node_parent[c] == cur and node_token[c] == target[cur]:
                nxt = c
                break
        if nxt < 0:
            break
        path.append(nxt)
        cur = nxt
    return path, int(target[cur])


def accept_compact(node_token, node_parent, n_nodes, target, L: int, k_cache, v_cache,
                   kv_base, prefix_len):
    """Batched.  node_token/node_parent/target [b, n_max]; n_nodes [b];
    k_cache/v_cache [n_layers, rows, hkv, D] (any dtype; rows are moved as
    raw values).  Returns (accept_len [b], accepted_nodes [b, L+1] padded
    with -1, bonus [b], new_len [b], k_out, v_out)."""
    b = len(n_nodes)
    k_out = np.array(k_cache, copy=True)
    v_out = np.array(v_cache, copy=True)
    accept_len = np.zeros(b, dtype=np.int32)
    accepted = np.full((b, L + 1), -1, dtype=np.int32)
    bonus = np.zeros(b, dtype=np.int32)
    new_len = np.zeros(b, dtype=np.int32)
    for r in range(b):
        path, bon = greedy_walk(node_token[r], node_parent[r], int(n_nodes[r]), target[r], L)
        n_acc = len(path) - 1
        accept_len[r] = n_acc
        accepted[r, :len(path)] = path
        bonus[r] = bon
        P = int(prefix_len[r])
        base = int(kv_base[r])
        new_len[r] = P + n_acc + 1
        src = [base + P + s for s in path]
        dst = [base + P + j for j in range(len(path))]
        for cache in (k_out, v_out):
            rows = cache[:, src].copy()      # snapshot every source row first
            cache[:, dst] = rows
    return accept_len, accepted, bonus, new_len, k_out, v_out
