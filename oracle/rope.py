"""Oracle: tree positions, rotary embedding, tree K/V scatter.

TEST INFRASTRUCTURE ONLY (see the package docstring).

[DDTree] "방법론 자세히 보기" (method in detail): the flattened tree is checked
by the target in one pass, each token continuing the sequence after its own
ancestors, so the token in slot i is at sequence position P + depth_i (the
root, the bonus token, at P).  A chain gives P, P+1, ...

The pages do not name the positional encoding.  Reading taken: the rotary
embedding in its split-half form, pairs (j, j + D/2) for j < D/2,
theta_j = base^(-2j/D), angle = position * theta_j, rotation
(x, y) -> (x cos a - y sin a, y cos a + x sin a), evaluated in float64 and
rounded to float32, then to bf16 (round to nearest even both times).
"""
from __future__ import annotations

import numpy as np


def _bf16_bits_to_f64(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(
        np.float64)


def _f64_to_bf16_bits(x):
    f = np.asarray(x, dtype=np.float64).astype(np.float32)          # RNE to float32
    u = f.view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)  # RNE to bf16


def tree_positions(node_depth, n_nodes, prefix_len):
    """i32 [batch, n_max]: P_b + depth for live slots, -1 after n_nodes."""
    node_depth = np.asarray(node_depth)
    b, n_max = node_depth.shape
    pos = np.full((b, n_max), -1, dtype=np.int32)
    for r in range(b):
        n = int(n_nodes[r])
        pos[r, :n] = int(prefix_len[r]) + node_depth[r, :n]
    return pos


def rope_f64(x, pos, base):
    """Rotary embedding of float64 vectors x [..., D] at positions pos [...]."""
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    j = np.arange(D // 2, dtype=np.float64)
    theta = float(base) ** (-2.0 * j / D)
    a = np.asarray(pos, dtype=np.float64)[..., None] * theta
    c, s = np.cos(a), np.sin(a)
    lo, hi = x[..., :D // 2], x[..., D // 2:]
    return np.concatenate([lo * c - hi * s, hi * c + lo * s], axis=-1)


def tree_rope_kv(node_depth, n_nodes, prefix_len, kv_base, q_bits, k_new_bits, v_new_bits,
                 k_cache_bits, v_cache_bits, base):
    """Return (positions, q_bits', k_cache_bits', v_cache_bits') as new arrays:
    q [b, n_max, hq, D] rotated for live slots, and the rotated k / copied v of
    slot i written to cache row kv_base + P + i."""
    pos = tree_positions(node_depth, n_nodes, prefix_len)
    q = np.array(q_bits, dtype=np.uint16, copy=True)
    kc = np.array(k_cache_bits, dtype=np.uint16, copy=True)
    vc = np.array(v_cache_bits, dtype=np.uint16, copy=True)
    for r in range(q.shape[0]):
        n = int(n_nodes[r])
        if n == 0:
            continue
        p = pos[r, :n]
        q[r, :n] = _f64_to_bf16_bits(rope_f64(_bf16_bits_to_f64(q_bits[r, :n]), p[:, None], base))
        rows = int(kv_base[r]) + int(prefix_len[r]) + np.arange(n)
        kc[rows] = _f64_to_bf16_bits(rope_f64(_bf16_bits_to_f64(k_new_bits[r, :n]), p[:, None],
                                              base))
        vc[rows] = v_new_bits[r, :n]
    return pos, q, kc, vc
