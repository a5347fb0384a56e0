"""Pins for the oracle's tree positions + rotary embedding (CPU only).

What fixes the answer without another implementation: rotations compose
(rope at m then at n equals rope at m + n), preserve each pair's norm and
make q.k depend on the position difference only; position 0 is the
identity; theta at j = D/4 is base^(-1/2) exactly; a chain tree gets the
ordinary positions P, P+1, ...; cache rows outside the tree block stay."""
import numpy as np

import synth
from oracle.rope import rope_f64, tree_positions, tree_rope_kv


def _rng_vecs(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


def _bits(rng, *shape):
    return synth.f32_to_bf16_bits(rng.standard_normal(shape).astype(np.float32))


def test_position_zero_is_identity():
    x = _rng_vecs(0, 5, 128)
    assert np.array_equal(rope_f64(x, np.zeros(5), 1e6), x)


def test_rotations_compose():
    x = _rng_vecs(1, 7, 64)
    m = np.arange(7) * 37.0
    n = np.arange(7) * 11.0 + 3.0
    a = rope_f64(rope_f64(x, m, 1e4), n, 1e4)
    b = rope_f64(x, m + n, 1e4)
    assert np.abs(a - b).max() < 1e-9


def test_pair_norms_preserved():
    x = _rng_vecs(2, 9, 128)
    y = rope_f64(x, np.arange(9) * 1000.0 + 17.0, 1e6)
    nx = x[:, :64] ** 2 + x[:, 64:] ** 2
    ny = y[:, :64] ** 2 + y[:, 64:] ** 2
    assert np.abs(nx - ny).max() < 1e-12


def test_scores_depend_on_position_difference_only():
    q = _rng_vecs(3, 128)
    k = _rng_vecs(4, 128)
    for m, n, s in [(5, 2, 100), (2048, 2050, 7), (0, 300, 9000)]:
        d1 = rope_f64(q, m, 1e6) @ rope_f64(k, n, 1e6)
        d2 = rope_f64(q, m + s, 1e6) @ rope_f64(k, n + s, 1e6)
        assert abs(d1 - d2) < 1e-9


def test_theta_at_quarter_dimension():
    # j = D/4 turns (1, 0) by pos * base^(-1/2): base 1e4 -> 0.01 rad per position
    D = 128
    x = np.zeros(D)
    x[D // 4] = 1.0
    y = rope_f64(x, 100.0, 1e4)
    assert abs(y[D // 4] - np.cos(1.0)) < 1e-12 and abs(y[D // 4 + D // 2] - np.sin(1.0)) < 1e-12


def test_chain_gets_ordinary_positions_and_rows():
    n, P = 9, 2048
    depth = np.arange(n, dtype=np.int32)[None]
    pos = tree_positions(depth, [n], [P])
    assert pos[0].tolist() == list(range(P, P + n))
    rng = np.random.default_rng(5)
    q = _bits(rng, 1, n, 2, 32)
    kn = _bits(rng, 1, n, 1, 32)
    vn = _bits(rng, 1, n, 1, 32)
    kc = _bits(rng, P + 20, 1, 32)
    vc = kc.copy()
    _, q2, kc2, vc2 = tree_rope_kv(depth, [n], [P], [0], q, kn, vn, kc, vc, 1e6)
    assert np.array_equal(kc2[:P], kc[:P]) and np.array_equal(kc2[P + n:], kc[P + n:])
    assert np.array_equal(vc2[P:P + n], vn[0])
    # slot 3 of a chain sits at position P + 3: same as rotating by hand
    assert np.array_equal(q2[0, 3], tree_rope_kv(depth[:, 3:4] * 0 + 3, [1], [P], [0],
                                                 q[:, 3:4], kn[:, 3:4], vn[:, 3:4], kc, vc,
                                                 1e6)[1][0, 0])


def test_padding_slots_untouched():
    depth = np.array([[0, 1, 1, 2, -1, -1]], dtype=np.int32)
    rng = np.random.default_rng(6)
    q = _bits(rng, 1, 6, 2, 32)
    kn = _bits(rng, 1, 6, 1, 32)
    kc = np.zeros((40, 1, 32), dtype=np.uint16)
    pos, q2, kc2, _ = tree_rope_kv(depth, [4], [30], [0], q, kn, kn, kc, kc.copy(), 1e6)
    assert pos[0].tolist() == [30, 31, 31, 32, -1, -1]
    assert np.array_equal(q2[0, 4:], q[0, 4:])
    assert np.all(kc2[34:] == 0) and np.all(kc2[:30] == 0)


def _torch_bf16_bits(x64):
    import torch
    t = torch.from_numpy(np.asarray(x64, dtype=np.float64)).float().bfloat16()
    return t.view(torch.int16).numpy().view(np.uint16)


def test_bf16_rounding_matches_torch():
    """The oracle's final rounding (float64 -> float32 -> bf16, nearest-even
    both times) equals torch's CPU conversions on random values of every
    magnitude, on exact bf16 ties (float32 low half 0x8000, even and odd
    upper halves, both signs), just off the ties, on float64 values that
    only become a tie after the float32 step, on subnormals and signed
    zeros, and at the top of the float32 range (rounds to infinity)."""
    from oracle.rope import _f64_to_bf16_bits
    rng = np.random.default_rng(11)
    vals = [rng.standard_normal(4000) * 10.0 ** rng.integers(-30, 30, 4000)]
    hi = rng.integers(0, 0x7F7F, 2000, dtype=np.uint32) << 16
    for low in (0x8000, 0x7FFF, 0x8001, 0x0000, 0xFFFF):
        u = (hi | np.uint32(low)).astype(np.uint32)
        f = u.view(np.float32).astype(np.float64)
        vals += [f, -f]
    # float64 just above / below a float32 tie: the float32 step decides
    ties = ((hi | np.uint32(0x8000)).astype(np.uint32)).view(np.float32).astype(np.float64)
    vals += [np.nextafter(ties, np.inf), np.nextafter(ties, -np.inf)]
    vals += [np.array([0.0, -0.0, 1e-45, -1e-45, 1e-39, 3.4028234663852886e38,
                       -3.4028234663852886e38, 3.3961775292304e38, 1.0, -1.0])]
    x = np.concatenate(vals)
    assert np.array_equal(_f64_to_bf16_bits(x), _torch_bf16_bits(x))
    # the worked tie cases, by hand: 1 + 2^-8 is halfway between bf16 1 and
    # 1 + 2^-7 and goes to the even one (1.0); 1 + 3 * 2^-8 goes up to 1 + 2^-6
    assert _f64_to_bf16_bits(np.array([1 + 2.0 ** -8]))[0] == 0x3F80
    assert _f64_to_bf16_bits(np.array([1 + 3 * 2.0 ** -8]))[0] == 0x3F82


def test_bf16_input_generator_matches_torch():
    """The seeded generators' bf16 storage rounding (float32 -> bf16) equals
    torch's, so both sides of every parity test read the values torch would."""
    rng = np.random.default_rng(12)
    x = (rng.standard_normal(20000) * 10.0 ** rng.integers(-20, 20, 20000)).astype(np.float32)
    u = rng.integers(0, 0x7F7F, 2000, dtype=np.uint32) << 16 | np.uint32(0x8000)
    x = np.concatenate([x, u.astype(np.uint32).view(np.float32)])
    assert np.array_equal(synth.f32_to_bf16_bits(x), _torch_bf16_bits(x.astype(np.float64)))
