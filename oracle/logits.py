"""Oracle, step 1: per-position log-softmax and top-K over the vocabulary.

[DDTree] section "핵심 아이디어" (core idea): the block-diffusion drafter emits,
in one forward pass, one distribution over the vocabulary for every masked
position after the bonus token.  The tree builder consumes those per-position
distributions as log-probabilities.  The pages fix no top-K; the candidate
count K per position comes from the workload configuration.

``argmax_rows`` is the verifier's greedy token ([DDTree] "방법론 자세히 보기",
method in detail: the target's outputs at the tree slots are compared with the
tree; at temperature 0 the output is the most probable token):
  id = the smallest v with z_v = max_u z_u            (raw logits, no scaling)

Definition computed by ``topk_logprobs``, per row:
  1. x_v = fl32(z_v * fl32(1/T))          (T = 1 leaves z unchanged)
  2. lse = m + log(sum_v exp(x_v - m))      in float64, m = max_v x_v
  3. the K ids with largest x, ties broken by smaller id first
     (ranking uses the float32 x, the precision both sides share)
  4. logp_j = fl32(x_id_j - lse)            (difference in float64)
"""
from __future__ import annotations

import numpy as np


def topk_logprobs(logits: np.ndarray, k: int, inv_temperature: float = 1.0):
    """Return (ids i32 [rows, k], logp f32 [rows, k], lse f64 [rows])."""
    z = np.asarray(logits, dtype=np.float32)
    if z.ndim != 2:
        raise ValueError("logits must be [rows, vocab]")
    rows, vocab = z.shape
    if not (1 <= k <= vocab):
        raise ValueError("need 1 <= k <= vocab")
    x = (z * np.float32(inv_temperature)).astype(np.float32)
    ids = np.empty((rows, k), dtype=np.int32)
    logp = np.empty((rows, k), dtype=np.float32)
    lse = np.empty(rows, dtype=np.float64)
    token = np.arange(vocab)
    for r in range(rows):
        xr = x[r].astype(np.float64)
        m = xr.max()
        lse[r] = m + np.log(np.sum(np.exp(xr - m)))
        # sort key: primary x descending, secondary id ascending (lexsort
        # takes the last key as primary)
        order = np.lexsort((token, -xr))
        top = order[:k]
        ids[r] = top
        logp[r] = (xr[top] - lse[r]).astype(np.float32)
    return ids, logp, lse


def argmax_rows(logits: np.ndarray):
    """Return (ids i32 [rows], max f32 [rows]): per row the smallest index
    holding the row maximum (numpy's argmax returns the first occurrence)."""
    z = np.asarray(logits, dtype=np.float32)
    if z.ndim != 2 or z.shape[1] < 1:
        raise ValueError("logits must be [rows, vocab] with vocab >= 1")
    if np.isnan(z).any():
        raise ValueError("NaN logits have no arg-max")
    ids = np.argmax(z, axis=1).astype(np.int32)
    return ids, z[np.arange(z.shape[0]), ids]
