"""Pins for the oracle's fused LM head (CPU only).

What fixes the answer without another implementation: one-hot hidden
states select a weight column exactly; an identity head returns the hidden
state; small integer inputs give exact logits that a plain Python loop
reproduces; the float32-summation bound holds for a float32 summation; the
planted token of the seeded recipe comes out on top."""
import numpy as np

import synth
from oracle.lmhead import accumulation_bound, lmhead_logits, lmhead_topk
from oracle.logits import topk_logprobs


def test_one_hot_rows_select_weight_columns():
    _, w, _ = synth.make_lmhead_case(1, 1, 256, 3000)
    h = np.zeros((3, 256), dtype=np.float32)
    cols = [0, 77, 255]
    for r, c in enumerate(cols):
        h[r, c] = 1.0
    z = lmhead_logits(synth.f32_to_bf16_bits(h), w)
    wf = synth.bf16_bits_to_f32(w).astype(np.float64)
    for r, c in enumerate(cols):
        assert np.array_equal(z[r], wf[:, c])


def test_identity_head_returns_hidden_state():
    hb, _, _ = synth.make_lmhead_case(2, 4, 512, 512)
    eye = synth.f32_to_bf16_bits(np.eye(512, dtype=np.float32))
    z = lmhead_logits(hb, eye)
    assert np.array_equal(z, synth.bf16_bits_to_f32(hb).astype(np.float64))


def test_integer_inputs_brute_force():
    hb, wb, _ = synth.make_lmhead_case(3, 3, 256, 50, integer=True)
    h = synth.bf16_bits_to_f32(hb)
    w = synth.bf16_bits_to_f32(wb)
    z = lmhead_logits(hb, wb)
    for r in range(3):
        for v in range(50):
            acc = 0
            for i in range(256):
                acc += int(h[r, i]) * int(w[v, i])
            assert z[r, v] == acc


def test_float32_summation_within_bound():
    hb, wb, _ = synth.make_lmhead_case(4, 2, 4096, 400)
    z64 = lmhead_logits(hb, wb)
    h = synth.bf16_bits_to_f32(hb)
    w = synth.bf16_bits_to_f32(wb)
    bound = accumulation_bound(hb, wb)
    for r in range(2):
        prod = (h[r][None, :] * w).astype(np.float32)        # exact products
        acc = np.zeros(w.shape[0], dtype=np.float32)
        for i in range(4096):                                 # left to right in float32
            acc += prod[:, i]
        assert np.abs(acc.astype(np.float64) - z64[r]).max() <= bound[r]
        assert bound[r] < 0.05                                # the margin is small


def test_planted_token_on_top_and_definition():
    hb, wb, planted = synth.make_lmhead_case(5, 6, 1024, 20000, delta=20.0)
    ids, logp, lse, z64 = lmhead_topk(hb, wb, 8)
    assert ids[:, 0].tolist() == planted.tolist()
    # the logit-pass definition on the float32 logits
    ids2, logp2, lse2 = topk_logprobs(z64.astype(np.float32), 8)
    assert np.array_equal(ids, ids2) and np.array_equal(logp, logp2)


def test_temperature_scales_integer_logit_gaps():
    """Integer inputs give exact integer logits; at inv_temperature 1/2 the
    scaled logits stay exact in float32, so the log-prob gaps are exactly
    half the logit gaps and the full-vocabulary distribution sums to 1."""
    hb, wb, _ = synth.make_lmhead_case(6, 3, 128, 64, integer=True)
    z = lmhead_logits(hb, wb)
    ids, logp, _, _ = lmhead_topk(hb, wb, 64, inv_temperature=0.5)
    for r in range(3):
        gaps = logp[r].astype(np.float64) - logp[r, 0]
        assert np.allclose(gaps, 0.5 * (z[r, ids[r]] - z[r, ids[r, 0]]), atol=2e-6)
        assert abs(np.exp(logp[r].astype(np.float64)).sum() - 1.0) < 1e-5
