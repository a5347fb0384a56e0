"""Oracle, step 3: masked GQA attention over prefix KV plus the queries' own KV.

Two visibility rules share one definition:

* tree verification -- [DDTree] "방법론 자세히 보기" (method in detail) and
  "용어 정리" (glossary): the flattened tree is verified in one target pass
  where each tree token attends to the whole committed prefix and, inside the
  tree, only to its own ancestor path (itself included).  Bit j of row i of
  the ancestor mask says whether tree slot j is visible to tree slot i.
* drafter pass -- [DFlash] "DFlash의 핵심 아이디어" points 2-3 and
  [DFlash-news] "DFlash 핵심 기술 구조": context from the target is injected as
  key/value memory into every draft layer, and the block of masked positions
  is filled jointly, so block queries see all context rows and every row of
  their own block (no mask).
* packed drafter blocks -- [DFlash] "여러 블록을 한 번에 학습하되, 블록끼리 새지
  않게 막는다": several blocks share one sequence and the mask keeps them
  apart, so own row j is visible to query i only when both lie in the same
  block of block_len consecutive own rows (every prefix row stays visible).

Readings: softmax scale 1/sqrt(D) unless given; query head h reads KV head
floor(h / (hq/hkv)); no positional terms inside the kernel (inputs are taken as
already position-encoded).  Inputs are the bf16 values exactly as stored;
all arithmetic is float64.

For request r the cache rows are kv_base[r] + [0, P_r) for the prefix and
kv_base[r] + P_r + [0, n_q[r]) for the queries' own rows.
"""
from __future__ import annotations

import numpy as np


def _mask_bits(words: np.ndarray, n: int) -> np.ndarray:
    """Unpack the first n bits of a little-endian u64 word row into bools."""
    bits = np.zeros(n, dtype=bool)
    for j in range(n):
        bits[j] = (int(words[j // 64]) >> (j % 64)) & 1
    return bits


def masked_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, kv_base, prefix_len,
                     n_q, own_mask=None, scale=None, block_len=None):
    """q [b, nq_max, hq, D]; k, v [rows, hkv, D] (float values of bf16 data);
    own_mask u64 [b, nq_max, W] or None for the dense drafter block;
    block_len (no mask): packed blocks of that many own rows.
    Returns (out f64 [b, nq_max, hq, D], lse f64 [b, nq_max, hq]); rows
    i >= n_q[r] are left at zero."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    b, nq_max, hq, D = q.shape
    hkv = k.shape[1]
    if hq % hkv:
        raise ValueError("hq must be a multiple of hkv")
    g = hq // hkv
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    out = np.zeros((b, nq_max, hq, D))
    lse = np.zeros((b, nq_max, hq))
    for r in range(b):
        P = int(prefix_len[r])
        n = int(n_q[r])
        base = int(kv_base[r])
        if n == 0:
            continue
        Kr = k[base:base + P + n]          # [T, hkv, D]
        Vr = v[base:base + P + n]
        visible = np.ones((n, P + n), dtype=bool)
        if own_mask is not None:
            for i in range(n):
                visible[i, P:] = _mask_bits(own_mask[r, i], n)
        elif block_len is not None:
            for i in range(n):
                for j in range(n):
                    visible[i, P + j] = (i // block_len) == (j // block_len)
        for h in range(hq):
            kh = h // g
            s = (q[r, :n, h, :] @ Kr[:, kh, :].T) * scale        # [n, T]
            s = np.where(visible, s, -np.inf)
            m = s.max(axis=1, keepdims=True)
            w = np.exp(s - m)
            l = w.sum(axis=1, keepdims=True)
            out[r, :n, h, :] = (w @ Vr[:, kh, :]) / l
            lse[r, :n, h] = (m + np.log(l))[:, 0]
    return out, lse
