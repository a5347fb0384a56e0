"""Oracle, fused LM head + log-softmax / top-K.

TEST INFRASTRUCTURE ONLY (see the package docstring).

[DFlash] section "임베딩과 출력 헤드는 공유한다" (embedding and output head are
shared): the drafter uses the target's frozen LM head, so the logits of a
block position are the product of the drafter's hidden state at that
position with the head's weight, one row of the weight per vocabulary token.

Definition computed here, per row r:
  1. z64[v] = sum_h H[r, h] * W[v, h]   exactly: every bf16 product is exact
     in float64 and the hidden sizes used keep the sums exact to well below
     float32 resolution
  2. z = fl32(z64)                      (the float32 logit of an exact sum)
  3. the logit-pass definition (``logits.topk_logprobs``) on z with 1/T.
A GPU accumulates the products in float32 in its own order, so its logits
differ from z by at most ``accumulation_bound`` (hidden * 2^-24 * sum_h
|H W|, the textbook bound for n-term float32 summation); tests compare
decisions taken within that margin by validity, and exactly elsewhere.
"""
from __future__ import annotations

import numpy as np

from .logits import topk_logprobs

_BLOCK = 16384  # vocabulary rows per float64 product (memory only)


def _bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(
        np.float64)


def lmhead_logits(h_bits: np.ndarray, w_bits: np.ndarray) -> np.ndarray:
    """float64 logits [rows, vocab] of bf16 hidden states [rows, hidden] and a
    bf16 head [vocab, hidden] (bit patterns, uint16)."""
    h = _bf16_to_f64(h_bits)
    vocab = w_bits.shape[0]
    z = np.empty((h.shape[0], vocab), dtype=np.float64)
    for v0 in range(0, vocab, _BLOCK):
        z[:, v0:v0 + _BLOCK] = h @ _bf16_to_f64(w_bits[v0:v0 + _BLOCK]).T
    return z


def accumulation_bound(h_bits: np.ndarray, w_bits: np.ndarray) -> np.ndarray:
    """Per row: hidden * 2^-24 * max_v sum_h |H[r,h] W[v,h]|."""
    h = np.abs(_bf16_to_f64(h_bits))
    vocab, hidden = w_bits.shape
    m = np.zeros(h.shape[0])
    for v0 in range(0, vocab, _BLOCK):
        m = np.maximum(m, (h @ np.abs(_bf16_to_f64(w_bits[v0:v0 + _BLOCK])).T).max(axis=1))
    return hidden * 2.0 ** -24 * m


def lmhead_topk(h_bits: np.ndarray, w_bits: np.ndarray, k: int, inv_temperature: float = 1.0):
    """Return (ids i32 [rows, k], logp f32 [rows, k], lse f64 [rows],
    z64 [rows, vocab])."""
    z64 = lmhead_logits(h_bits, w_bits)
    ids, logp, lse = topk_logprobs(z64.astype(np.float32), k, inv_temperature)
    return ids, logp, lse, z64
