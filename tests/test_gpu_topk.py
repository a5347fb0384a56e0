"""GPU parity: ddt_topk_logprobs vs the oracle's log-softmax + top-K.

Bar (workload tolerance): ids bit-exact (both rank on the same float32 x),
log-probs and lse within 1e-5 absolute.  Cases: every workload config at
full size (tiny V=1000 x 4, 16 x 151936 with K = 8/32/64 peaked and flat,
all 512 rows of 512 x 151936 with K=16) plus edge cases (ties, K = V, K = 128, strided rows,
vocab not a multiple of 4, temperature, one row)."""
import numpy as np
import pytest
import torch

import synth
from block_diffusion_draft_vocab_amd import ddt
from oracle.logits import topk_logprobs as oracle_topk
from tests import report

pytestmark = pytest.mark.gpu

TOL = 1e-5


def _run(gpu, logits: np.ndarray, k: int, inv_t: float = 1.0, ld: int = None):
    rows, V = logits.shape
    if ld is None or ld == V:
        dl = torch.from_numpy(logits).to(gpu)
    else:
        buf = np.full((rows, ld), 123.0, dtype=np.float32)   # junk beyond vocab
        buf[:, :V] = logits
        dl = torch.from_numpy(buf).to(gpu)
    ids, logp, lse = ddt.topk_logprobs(dl, k, inv_t, vocab=V)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), logp.cpu().numpy(), lse.cpu().numpy()


def _compare(gpu, logits, k, inv_t=1.0, ld=None, case=None):
    ids, logp, lse = _run(gpu, logits, k, inv_t, ld)
    oids, ologp, olse = oracle_topk(logits, k, inv_t)
    assert np.array_equal(ids, oids)
    assert np.abs(logp.astype(np.float64) - ologp).max() <= TOL
    assert np.abs(lse.astype(np.float64) - olse).max() <= TOL
    assert np.all(logp <= 0)
    if case is not None:
        report.record(case, "logp_max_abs", np.abs(logp.astype(np.float64) - ologp).max(), TOL)
        report.record(case, "lse_max_abs", np.abs(lse.astype(np.float64) - olse).max(), TOL)


@pytest.mark.parametrize("cfg", [synth.CONFIGS[1], synth.CONFIGS[2], synth.CONFIGS[3],
                                 synth.CONFIGS[4], synth.FLAT4, synth.DEEP],
                         ids=["c1", "c2", "c3", "c4", "c4flat", "deep"])
def test_topk_workloads(gpu, cfg):
    case = synth.make_case(cfg, with_drafter=False, with_verify=False)
    _compare(gpu, case.logits, cfg.K, cfg.inv_temperature, case=f"topk_{cfg.name}")


def test_topk_serving_batch(gpu):
    """All 512 rows of the serving batch (32 requests x 16 positions, K = 16)
    against the oracle."""
    cfg = synth.CONFIGS[5]
    case = synth.make_case(cfg, with_drafter=False, with_verify=False)
    ids, logp, lse = _run(gpu, case.logits, cfg.K)
    oids, ologp, olse = oracle_topk(case.logits, cfg.K)
    assert np.array_equal(ids, oids)
    assert np.abs(logp.astype(np.float64) - ologp).max() <= TOL
    assert np.abs(lse.astype(np.float64) - olse).max() <= TOL
    report.record("topk_serving_b32", "logp_max_abs",
                  np.abs(logp.astype(np.float64) - ologp).max(), TOL)


@pytest.mark.parametrize("rows,V,k,ld", [(3, 1001, 7, 1003), (1, 151936, 128, None),
                                         (5, 64, 64, None), (2, 5, 1, None),
                                         (7, 40000, 16, 40004), (1, 8193, 33, None)])
def test_topk_shapes(gpu, rows, V, k, ld):
    rng = np.random.default_rng(rows * 31 + V)
    logits = (2 * rng.standard_normal((rows, V))).astype(np.float32)
    _compare(gpu, logits, k, ld=ld)


def test_topk_ties(gpu):
    rng = np.random.default_rng(5)
    logits = np.round(rng.standard_normal((4, 30000)), 1).astype(np.float32)
    logits[1] = 0.5                                   # one value everywhere
    logits[2, ::7] = logits[2].max()                  # many copies of the max
    _compare(gpu, logits, 64)


@pytest.mark.parametrize("k", [32, 64])
def test_topk_ties_one_wave_merge(gpu, k):
    """16 x 151936 with K = 32 / 64: the merge runs one wave per row.  A
    constant row leaves about K lists' worth of keys at or above the
    threshold (the exact head-merge fallback), a row of many equal maxima and
    rows of coarse ties exercise the ranked path."""
    rng = np.random.default_rng(8)
    logits = np.round(rng.standard_normal((16, synth.QWEN3_VOCAB)), 1).astype(np.float32)
    logits[1] = -0.25
    logits[2, ::7] = logits[2].max()
    logits[3, ::8192] = 9.0                           # one equal max per chunk start
    logits[4, 8191::8192] = 9.0                       # ... and per chunk end
    _compare(gpu, logits, k)


def test_topk_temperature(gpu):
    rng = np.random.default_rng(6)
    logits = (3 * rng.standard_normal((8, 20000))).astype(np.float32)
    _compare(gpu, logits, 32, inv_t=1.0 / 0.7)


def test_topk_deterministic(gpu):
    case = synth.make_case(synth.CONFIGS[3], with_drafter=False, with_verify=False)
    a = _run(gpu, case.logits, 32)
    b = _run(gpu, case.logits, 32)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_topk_signed_zero_ties(gpu):
    """-0 and +0 are the same logit: they tie, and the smaller id ranks
    first whichever sign it carries (vocab 4, and a row long enough to span
    several chunks with zeros of both signs around the top)."""
    small = np.array([[0.0, -0.0, 2.0, 0.0]], np.float32)
    _compare(gpu, small, 4)
    rng = np.random.default_rng(21)
    big = np.round(rng.normal(0, 0.3, size=(3, 20000))).astype(np.float32) - 2.0
    big[:, ::7] = 0.0
    big[:, 3::7] = -0.0
    _compare(gpu, big, 64)
