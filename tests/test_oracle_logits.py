"""Pins for the oracle's log-softmax + top-K (CPU only).

What fixes the answer without another implementation: log-sum-exp normalises
the distribution; closed forms for constant and two-valued rows; the top-K
order equals a stable library sort by (-x, id); brute force on tiny rows."""
import math

import numpy as np
import pytest

import synth
from oracle.logits import argmax_rows, topk_logprobs


def _rows(seed, rows, V):
    rng = np.random.default_rng(seed)
    return (2.0 * rng.standard_normal((rows, V))).astype(np.float32)


def test_distribution_normalises():
    z = _rows(0, 3, 1000)
    _, _, lse = topk_logprobs(z, 4)
    for r in range(3):
        x = z[r].astype(np.float64)
        assert abs(np.exp(x - lse[r]).sum() - 1.0) < 1e-12


def test_distribution_normalises_full_vocab():
    z = _rows(1, 1, synth.QWEN3_VOCAB)
    _, logp, lse = topk_logprobs(z, 8)
    x = z[0].astype(np.float64)
    assert abs(np.exp(x - lse[0]).sum() - 1.0) < 1e-12
    assert np.all(logp <= 0)


def test_lse_closed_forms():
    V = 777
    c = np.float32(3.25)
    z = np.full((1, V), c, dtype=np.float32)
    ids, logp, lse = topk_logprobs(z, 5)
    assert abs(lse[0] - (float(c) + math.log(V))) < 1e-12
    # all equal -> ties broken by id: the first five ids, each log(1/V)
    assert ids[0].tolist() == [0, 1, 2, 3, 4]
    assert np.allclose(logp[0], np.float32(-math.log(V)), atol=0)
    # two-valued row: closed form log(n_a e^a + n_b e^b)
    z2 = np.zeros((1, 10), dtype=np.float32)
    z2[0, 7] = 2.0
    _, logp2, lse2 = topk_logprobs(z2, 2)
    want = math.log(9 + math.exp(2.0))
    assert abs(lse2[0] - want) < 1e-12
    assert logp2[0, 0] == np.float32(2.0 - want)
    assert logp2[0, 1] == np.float32(0.0 - want)


def test_matches_stable_argsort_with_ties():
    z = _rows(2, 6, 5000)
    # plant exact ties inside the top region
    z[0, 10] = z[0, 20] = z[0, 30] = z[0].max() + 1
    z[1, 4999] = z[1, 3] = z[1].max()
    z[2, :] = np.round(z[2], 1)            # many equal values
    ids, logp, lse = topk_logprobs(z, 16)
    for r in range(z.shape[0]):
        want = np.argsort(-z[r].astype(np.float64), kind="stable")[:16]
        assert ids[r].tolist() == want.tolist()
        assert np.all(np.diff(logp[r]) <= 0)


def test_brute_force_tiny():
    z = _rows(3, 4, 37)
    z[1, 5] = z[1, 6]
    ids, logp, lse = topk_logprobs(z, 7)
    for r in range(4):
        order = sorted(range(37), key=lambda v: (-float(z[r, v]), v))[:7]
        assert ids[r].tolist() == order
        direct = math.log(sum(math.exp(float(a)) for a in z[r]))
        assert abs(lse[r] - direct) < 1e-12
        for j, v in enumerate(order):
            assert logp[r, j] == np.float32(float(z[r, v]) - lse[r])


def test_selection_invariants():
    z = _rows(4, 5, 3000)
    ids, _, _ = topk_logprobs(z, 32)
    for r in range(5):
        chosen = set(ids[r].tolist())
        rest = np.array([v for v in range(3000) if v not in chosen])
        kth = z[r, ids[r, -1]]
        assert z[r, rest].max() <= kth
        for v in rest[z[r, rest] == kth]:
            assert v > ids[r, -1]


def test_temperature_scaling_in_fp32():
    z = _rows(5, 2, 500)
    inv_t = 1.0 / 0.7
    ids, logp, lse = topk_logprobs(z, 3, inv_temperature=inv_t)
    x = (z * np.float32(inv_t)).astype(np.float32).astype(np.float64)
    for r in range(2):
        m = x[r].max()
        assert abs(lse[r] - (m + math.log(np.exp(x[r] - m).sum()))) < 1e-12
        assert ids[r, 0] == int(np.argmax(x[r]))


def test_planted_token_is_rank0_in_tiny_config():
    case = synth.make_case(synth.CONFIGS[1], with_drafter=False, with_verify=False)
    ids, _, _ = topk_logprobs(case.logits, 4)
    # raises of 8 and 6.5 clear the ~3 sigma tail of 999 draws of 2*N(0,1)
    assert ids[:2, 0].tolist() == case.planted[:2].tolist()


def test_rejects_bad_k():
    with pytest.raises(ValueError):
        topk_logprobs(np.zeros((1, 4), np.float32), 5)


# ---- argmax_rows: the target's greedy token -------------------------------
def test_argmax_planted_positions():
    """A value planted above every other entry is found wherever it sits,
    including the first and last columns."""
    rng = np.random.default_rng(11)
    V = 151936
    z = rng.uniform(-5, 5, size=(6, V)).astype(np.float32)
    where = [0, V - 1, 8191, 8192, 77777, 4]
    for r, j in enumerate(where):
        z[r, j] = 6.0
    ids, mx = argmax_rows(z)
    assert ids.tolist() == where
    assert np.all(mx == np.float32(6.0))


def test_argmax_ties_go_to_smaller_id():
    """Equal maxima: the smaller index wins, whatever their order of
    planting and distance apart."""
    z = np.zeros((4, 5000), dtype=np.float32)
    z[0, [4999, 17]] = 2.0
    z[1, [3, 4]] = 2.0
    z[2, :] = -1.5                      # constant row: index 0
    z[3, [4096, 4095, 9 * 4 + 1]] = 1e30
    ids, mx = argmax_rows(z)
    assert ids.tolist() == [17, 3, 0, 37]
    assert mx.tolist() == [2.0, 2.0, -1.5, np.float32(1e30)]


def test_argmax_infinities_and_signed_zero():
    """-inf rows still have an arg-max (index 0); +inf dominates; -0 == +0
    counts as a tie, so the earlier index wins."""
    z = np.full((3, 10), -np.inf, dtype=np.float32)
    z[1, 6] = np.inf
    z[2, :] = -1.0
    z[2, 5] = -0.0
    z[2, 2] = 0.0
    ids, _ = argmax_rows(z)
    assert ids.tolist() == [0, 6, 2]


def test_argmax_brute_force_tiny():
    """Exhaustive over small integer-valued rows (many ties): the index that
    maximises (value, -index), found by scanning every pair."""
    rng = np.random.default_rng(5)
    z = rng.integers(-3, 4, size=(300, 9)).astype(np.float32)
    ids, _ = argmax_rows(z)
    for r in range(z.shape[0]):
        best = 0
        for j in range(1, z.shape[1]):
            if z[r, j] > z[r, best]:
                best = j
        assert ids[r] == best


def test_argmax_is_rank0_of_topk():
    """Cross-check against the top-K ranking (lexsort path) at T = 1."""
    z = _rows(12, 16, 20000)
    z[3, 100] = z[3, 99] = z[3].max() + 1.0          # a tie at the top
    ids, _ = argmax_rows(z)
    tk, _, _ = topk_logprobs(z, 1)
    assert np.array_equal(ids, tk[:, 0])


def test_argmax_rejects_nan():
    z = np.zeros((1, 4), dtype=np.float32)
    z[0, 2] = np.nan
    with pytest.raises(ValueError):
        argmax_rows(z)


def test_signed_zeros_tie():
    """-0.0 and +0.0 are equal logits: ranked by id, as a plain sort on
    (-x, id) orders them."""
    from oracle.logits import topk_logprobs
    z = np.array([[0.0, -0.0, 2.0, 0.0, -0.0]], np.float32)
    ids, _, _ = topk_logprobs(z, 5)
    expect = sorted(range(5), key=lambda i: (-float(z[0, i]), i))
    assert ids[0].tolist() == expect == [2, 0, 1, 3, 4]
