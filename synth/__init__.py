"""Seeded synthetic inputs for the draft-and-verify chain.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic (no log-softmax, no tree selection, no attention, no
acceptance walk).  Both the HIP path (tests, bench) and the CPU oracle consume
the arrays it returns, so the two sides always see identical inputs.

Workload shapes follow the DDTree summary page (block size 16, node budgets
16..1024, bf16; "Experiments" section) and the DFlash pages (16 masked block
positions after a bonus token, drafter conditioned on injected context KV).
Everything is synthetic: no dataset, checkpoint or benchmark item is used.

Random draws happen in one fixed order per case:
  logits -> planted ids -> (drafter Q, K, V) -> (verify Q, K, V)
  -> target-path uniforms -> off-path tokens
using ``numpy.random.Generator(PCG64(seed))``.  bf16 tensors are the
round-to-nearest-even rounding of float32 N(0,1) draws.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

QWEN3_VOCAB = 151936


# --------------------------------------------------------------------------
# bf16 helpers (storage only: round-to-nearest-even of float32, and back)
# --------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (RNE) and return the raw uint16 bits."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# --------------------------------------------------------------------------
# configurations
# --------------------------------------------------------------------------
@dataclass(frozen=True)
class Config:
    cid: int
    name: str
    batch: int
    L: int                 # masked block positions per request
    vocab: int
    K: int                 # top-K kept per position
    k_tree: int            # ranks per position the tree may branch over
    B: int                 # node budget (drafted nodes, root excluded)
    delta0: float          # planted-token raise at position 0
    delta_slope: float     # raise decreases by this per position
    hq: int
    hkv: int
    D: int
    prefix: tuple          # (lo, hi) inclusive prefix length range; lo == hi = fixed
    drafter_ctx: int       # injected context rows for the drafter pass (0 = none)
    flat: bool = False     # flat regime: 2*N(0,1) + delta/2 and temperature 1.0
    inv_temperature: float = 1.0


CONFIGS = {
    1: Config(1, "tiny", 1, 4, 1000, 4, 4, 8, 8.0, 1.5, 2, 1, 32, (64, 64), 64),
    2: Config(2, "dflash_chain", 1, 16, QWEN3_VOCAB, 8, 1, 16, 8.0, 0.3, 32, 8, 128,
              (2048, 2048), 2048),
    3: Config(3, "ddtree_b256", 1, 16, QWEN3_VOCAB, 32, 32, 256, 8.0, 0.3, 32, 8, 128,
              (2048, 2048), 2048),
    4: Config(4, "ddtree_b1024", 1, 16, QWEN3_VOCAB, 64, 64, 1024, 8.0, 0.3, 32, 8, 128,
              (4096, 4096), 2048),
    5: Config(5, "serving_b32", 32, 16, QWEN3_VOCAB, 16, 16, 64, 8.0, 0.3, 32, 4, 128,
              (512, 8192), 0),
}

# Test-only regimes (not workload configs): a deep planted chain gives deep trees.
DEEP = Config(103, "deep_b256", 1, 16, QWEN3_VOCAB, 32, 32, 256, 20.0, 0.3, 32, 8, 128,
              (2048, 2048), 2048)
FLAT4 = Config(104, "ddtree_b1024_flat", 1, 16, QWEN3_VOCAB, 64, 64, 1024, 8.0, 0.3,
               32, 8, 128, (4096, 4096), 2048, flat=True, inv_temperature=1.0)


def scaled(cfg: Config, **kw) -> Config:
    """A copy of ``cfg`` with some fields replaced (small parity cases)."""
    d = dict(cfg.__dict__)
    d.update(kw)
    return Config(**d)


# --------------------------------------------------------------------------
# one case = every array one chain step consumes
# --------------------------------------------------------------------------
@dataclass
class Case:
    cfg: Config
    seed: int
    logits: np.ndarray             # f32 [batch*L, V]
    planted: np.ndarray            # i64 [batch*L]
    # drafter pass: L block queries over ctx context rows + L own rows
    dq_bits: Optional[np.ndarray]  # u16 [batch, L, hq, D]
    dk_bits: Optional[np.ndarray]  # u16 [batch*(ctx+L), hkv, D]
    dv_bits: Optional[np.ndarray]
    # verify pass: N = B+1 tree queries over prefix rows + N own rows
    prefix_len: np.ndarray         # i32 [batch]
    kv_base: np.ndarray            # i64 [batch] first cache row of each request
    vq_bits: np.ndarray            # u16 [batch, N, hq, D]
    vk_bits: np.ndarray            # u16 [rows, hkv, D]
    vv_bits: np.ndarray
    path_uniforms: np.ndarray      # f64 [batch, L]
    off_path: np.ndarray           # i32 [batch, N]
    root_token: np.ndarray         # i32 [batch]
    extra: dict = field(default_factory=dict)

    @property
    def N(self) -> int:
        return self.cfg.B + 1


def _bf16_normal(rng, shape) -> np.ndarray:
    return f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32))


def make_logits(rng, cfg: Config):
    rows = cfg.batch * cfg.L
    z = (2.0 * rng.standard_normal((rows, cfg.vocab))).astype(np.float32)
    planted = rng.integers(0, cfg.vocab, size=rows, dtype=np.int64)
    pos = np.arange(rows) % cfg.L
    delta = (cfg.delta0 - cfg.delta_slope * pos).astype(np.float32)
    if cfg.flat:
        delta = (delta * np.float32(0.5)).astype(np.float32)
    z[np.arange(rows), planted] += delta
    return z, planted


def make_case(cfg: Config, seed: Optional[int] = None, with_drafter: bool = True,
              with_verify: bool = True) -> Case:
    seed = cfg.cid if seed is None else seed
    rng = np.random.Generator(np.random.PCG64(seed))
    logits, planted = make_logits(rng, cfg)
    b, L, hq, hkv, D = cfg.batch, cfg.L, cfg.hq, cfg.hkv, cfg.D
    N = cfg.B + 1
    dq = dk = dv = None
    if with_drafter and cfg.drafter_ctx > 0:
        rows_d = b * (cfg.drafter_ctx + L)
        dq = _bf16_normal(rng, (b, L, hq, D))
        dk = _bf16_normal(rng, (rows_d, hkv, D))
        dv = _bf16_normal(rng, (rows_d, hkv, D))
    lo, hi = cfg.prefix
    if lo == hi:
        prefix = np.full(b, lo, dtype=np.int32)
    else:
        prefix = rng.integers(lo, hi + 1, size=b).astype(np.int32)
    cap = prefix.astype(np.int64) + N
    kv_base = np.concatenate([[0], np.cumsum(cap)[:-1]]).astype(np.int64)
    rows_v = int(cap.sum())
    if with_verify:
        vq = _bf16_normal(rng, (b, N, hq, D))
        vk = _bf16_normal(rng, (rows_v, hkv, D))
        vv = _bf16_normal(rng, (rows_v, hkv, D))
    else:
        vq = vk = vv = None
    u = rng.random((b, L))
    off = rng.integers(0, cfg.vocab, size=(b, N)).astype(np.int32)
    root = rng.integers(0, cfg.vocab, size=b).astype(np.int32)
    return Case(cfg, seed, logits, planted, dq, dk, dv, prefix, kv_base, vq, vk, vv,
                u, off, root)


# --------------------------------------------------------------------------
# the synthetic target model
# --------------------------------------------------------------------------
def sample_target_path(case: Case) -> np.ndarray:
    """Tokens y[r, 0..L) drawn from each position's own softmax over the full
    vocab by inverse CDF on the stored float64 uniforms.  This is the synthetic
    target's continuation; it is input data, not part of the method."""
    cfg = case.cfg
    x = case.logits.astype(np.float64) * float(np.float32(cfg.inv_temperature))
    y = np.empty((cfg.batch, cfg.L), dtype=np.int32)
    for r in range(cfg.batch):
        for i in range(cfg.L):
            row = x[r * cfg.L + i]
            w = np.exp(row - row.max())
            cdf = np.cumsum(w)
            t = case.path_uniforms[r, i] * cdf[-1]
            y[r, i] = min(int(np.searchsorted(cdf, t, side="right")), cfg.vocab - 1)
    return y


def target_for_tree(node_token: np.ndarray, node_parent: np.ndarray,
                    node_depth: np.ndarray, n_nodes: int, y: np.ndarray,
                    off_path: np.ndarray) -> np.ndarray:
    """Target "argmax" per tree slot for one request.

    A slot whose root-to-node token path equals the target continuation
    y[0..depth) gets y[depth] (the target's next token); the root gets y[0];
    every other slot (off the target path, or at the last depth) gets the
    seeded uniform off-path token.  Padding slots keep their off-path token.
    """
    n_max = off_path.shape[0]
    L = y.shape[0]
    t = off_path.astype(np.int32).copy()
    on = np.zeros(n_max, dtype=bool)
    on[0] = True
    t[0] = y[0]
    for s in range(1, n_nodes):
        d = int(node_depth[s])
        p = int(node_parent[s])
        if on[p] and node_token[s] == y[d - 1]:
            on[s] = True
            if d < L:
                t[s] = y[d]
    return t


def force_path_target(node_token, node_parent, node_depth, n_nodes, stop_slot,
                      off_path, vocab) -> np.ndarray:
    """Target array that makes the greedy walk end exactly at ``stop_slot``:
    each ancestor's target is the token of the next node on the root->stop
    path, and stop_slot's target is a token none of its children carry."""
    t = off_path.astype(np.int32).copy()
    path = [int(stop_slot)]
    while path[-1] != 0:
        path.append(int(node_parent[path[-1]]))
    path.reverse()
    for a, c in zip(path[:-1], path[1:]):
        t[a] = node_token[c]
    kids = {int(node_token[c]) for c in range(1, n_nodes) if node_parent[c] == stop_slot}
    tok = int(off_path[stop_slot]) % vocab
    while tok in kids:
        tok = (tok + 1) % vocab
    t[stop_slot] = tok
    return t


def make_verify_logits(seed: int, rows: int, vocab: int = QWEN3_VOCAB,
                       peak: float = 12.0) -> tuple[np.ndarray, np.ndarray]:
    """Target logits at the tree slots (one row per flattened slot):
    float32 2*N(0,1) with +peak added at one seeded token per row, the shape
    of a confident target distribution.  Returns (logits [rows, vocab],
    planted ids [rows])."""
    rng = np.random.Generator(np.random.PCG64(seed))
    z = (2.0 * rng.standard_normal((rows, vocab), dtype=np.float32)).astype(np.float32)
    planted = rng.integers(0, vocab, size=rows, dtype=np.int64)
    z[np.arange(rows), planted] += np.float32(peak)
    return z, planted


def make_lmhead_case(seed: int, rows: int, hidden: int, vocab: int, delta: float = 6.0,
                     integer: bool = False):
    """Drafter hidden states and a shared LM head (bf16 bit patterns).

    Default: H ~ N(0,1) [rows, hidden], W ~ N(0,1) * 2/sqrt(hidden)
    [vocab, hidden] (logits of standard deviation about 2, like the logit
    configurations), and for each row one seeded token whose weight row gets
    delta * H[r] / |H[r]|^2 added, which raises that row's logit by about
    delta.  integer=True draws H and W from the integers -3..3 instead (every
    product and sum exact in float32).  Returns (h_bits [rows, hidden],
    w_bits [vocab, hidden], planted [rows])."""
    rng = np.random.Generator(np.random.PCG64(seed))
    if integer:
        h = rng.integers(-3, 4, size=(rows, hidden)).astype(np.float32)
        w = rng.integers(-3, 4, size=(vocab, hidden)).astype(np.float32)
        planted = rng.integers(0, vocab, size=rows, dtype=np.int64)
        return f32_to_bf16_bits(h), f32_to_bf16_bits(w), planted
    h = rng.standard_normal((rows, hidden), dtype=np.float32)
    w = rng.standard_normal((vocab, hidden), dtype=np.float32)
    w *= np.float32(2.0 / np.sqrt(hidden))
    planted = rng.integers(0, vocab, size=rows, dtype=np.int64)
    h_b = f32_to_bf16_bits(h)
    hr = bf16_bits_to_f32(h_b)
    for r in range(rows):
        w[planted[r]] += np.float32(delta) * hr[r] / np.float32(np.dot(hr[r], hr[r]))
    return h_b, f32_to_bf16_bits(w), planted
