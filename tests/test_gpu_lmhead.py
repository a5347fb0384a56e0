"""GPU parity: ddt_lmhead_topk (shared LM head GEMM fused with the logit
pass) vs the oracle.

Bars.  Integer inputs make every logit exact in float32 whatever the
summation order, so there ids must be bit-exact (ties included) and
log-probs / lse within 1e-5 plus three float32 half-ulps of the logit
magnitude (x, lse and x - lse are each rounded once; such logits reach
|x| ~ 1e3).  With real-valued inputs the kernel's float32
accumulation order differs from the oracle's exact sums by at most the
textbook bound b_r = hidden * 2^-24 * max_v sum |H W| per row; ranks whose
logits lie within that margin may legitimately swap, so the test checks
what is unique: every returned id is a valid top-k member up to 2 b_r,
ids are distinct and ordered, and log-probs / lse are within 1e-5 + b_r of
the oracle; where the oracle's top-k is separated by more than 2 b_r the
ids must be identical.  Cases: the drafter's 16 block rows with a
151936 x 4096 head (full size), partial and multiple 16-row blocks, a
vocabulary that is not a multiple of the 640-column chunk, hidden 256 and
1024, K 1 / 8 / 64, temperature, and massive integer ties."""
import numpy as np
import pytest
import torch

import synth
from block_diffusion_draft_vocab_amd import ddt
from oracle.lmhead import accumulation_bound, lmhead_topk as oracle_lmhead

pytestmark = pytest.mark.gpu


def _dev_bits(bits, gpu):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(gpu).view(
        torch.bfloat16)


def _run(gpu, hb, wb, k, inv_t=1.0):
    ids, logp, lse = ddt.lmhead_topk(_dev_bits(hb, gpu), _dev_bits(wb, gpu), k, inv_t)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), logp.cpu().numpy(), lse.cpu().numpy()


def _check_exact(gpu, hb, wb, k, inv_t=1.0):
    ids, logp, lse = _run(gpu, hb, wb, k, inv_t)
    oids, ologp, olse, _ = oracle_lmhead(hb, wb, k, inv_t)
    assert np.array_equal(ids, oids)
    # float32 logits of integer inputs reach |x| ~ 1e3: x, lse and x - lse
    # are each rounded once to float32 (half an ulp of the magnitude each)
    mag = np.maximum(np.abs(olse), np.abs(ologp.astype(np.float64) + olse[:, None]).max(axis=1))
    tol = 1e-5 + 3 * 2.0 ** -24 * mag
    assert np.all(np.abs(logp.astype(np.float64) - ologp).max(axis=1) <= tol)
    assert np.all(np.abs(lse.astype(np.float64) - olse) <= tol)


def _check_within_bound(gpu, hb, wb, k, inv_t=1.0):
    ids, logp, lse = _run(gpu, hb, wb, k, inv_t)
    oids, ologp, olse, z64 = oracle_lmhead(hb, wb, k, inv_t)
    b = accumulation_bound(hb, wb) * inv_t
    rows = ids.shape[0]
    for r in range(rows):
        x = z64[r] * inv_t
        order = np.sort(x)[::-1]
        xk = order[k - 1]
        assert len(set(ids[r].tolist())) == k
        assert np.all(x[ids[r]] >= xk - 2 * b[r])             # valid top-k members
        assert np.all(np.diff(logp[r]) <= 2 * b[r] + 1e-6)    # ordered up to the margin
        assert abs(lse[r] - olse[r]) <= 1e-5 + b[r]
        # log-probs of the returned ids against the oracle's exact values
        assert np.abs(logp[r].astype(np.float64) - (x[ids[r]] - olse[r])).max() <= 1e-5 + 2 * b[r]
        gaps = -np.diff(order[:k + 1])
        if np.all(gaps > 2 * b[r]):
            assert np.array_equal(ids[r], oids[r])


@pytest.fixture(scope="module")
def full_case():
    return synth.make_lmhead_case(61, 16, 4096, synth.QWEN3_VOCAB, delta=8.0)


def test_lmhead_drafter_rows_full_size(gpu, full_case):
    hb, wb, planted = full_case
    _check_within_bound(gpu, hb, wb, 32)


def test_lmhead_full_size_k64_temperature(gpu, full_case):
    hb, wb, _ = full_case
    _check_within_bound(gpu, hb, wb, 64, inv_t=1.0 / 0.7)


@pytest.mark.parametrize("rows,hidden,V,k", [(16, 4096, 20000, 32), (5, 1024, 7001, 8),
                                             (37, 256, 3333, 1), (16, 512, 641, 64),
                                             (1, 256, 64, 64)])
def test_lmhead_integer_exact(gpu, rows, hidden, V, k):
    hb, wb, _ = synth.make_lmhead_case(70 + rows, rows, hidden, V, integer=True)
    _check_exact(gpu, hb, wb, k)


def test_lmhead_integer_massive_ties(gpu):
    """Rows whose logits take a handful of values: hundreds of keys tie at
    each value, so chunk candidates overflow and the exact fallbacks run."""
    rows, hidden, V = 16, 256, 30000
    hb, wb, _ = synth.make_lmhead_case(80, rows, hidden, V, integer=True)
    w = synth.bf16_bits_to_f32(wb)
    w[:, 1:] = 0.0
    w[:, 0] = np.float32(np.random.default_rng(3).integers(0, 2, size=V))   # about 320 ties per chunk
    h = synth.bf16_bits_to_f32(hb)
    h[:, 0] = 1.0
    _check_exact(gpu, synth.f32_to_bf16_bits(h), synth.f32_to_bf16_bits(w), 64)


@pytest.mark.parametrize("rows,hidden,V,k", [(3, 1024, 40000, 16), (20, 2048, 9000, 32)])
def test_lmhead_random_shapes(gpu, rows, hidden, V, k):
    hb, wb, _ = synth.make_lmhead_case(90 + rows, rows, hidden, V)
    _check_within_bound(gpu, hb, wb, k)
