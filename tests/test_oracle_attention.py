"""Pins for the oracle's masked GQA attention (CPU only).

Independent library routine: torch's CPU scaled_dot_product_attention in
float64, with GQA expressed by repeat_interleave of the KV heads.
* a chain tree's ancestor mask is ordinary causal attention over [prefix; chain];
* the drafter block is unmasked attention;
* a general tree: SDPA with the boolean mask unpacked from the oracle's bits;
* a root row with no prefix returns its own value row exactly.
"""
import numpy as np
import pytest
import torch

import synth
from oracle.attention import masked_attention
from oracle.logits import topk_logprobs
from oracle.tree import build_tree


def _qkv(seed, b, n, P, hq, hkv, D):
    rng = np.random.default_rng(seed)
    q = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(rng.standard_normal((b, n, hq, D), dtype=np.float32)))
    rows = b * (P + n)
    k = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(rng.standard_normal((rows, hkv, D), dtype=np.float32)))
    v = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(rng.standard_normal((rows, hkv, D), dtype=np.float32)))
    base = np.arange(b, dtype=np.int64) * (P + n)
    return q, k, v, base


def _sdpa(q, k, v, allowed, g):
    """q [n, hq, D], k/v [T, hkv, D], allowed [n, T] bool -> [n, hq, D]"""
    qt = torch.from_numpy(q.astype(np.float64)).permute(1, 0, 2)            # hq n D
    kt = torch.from_numpy(k.astype(np.float64)).permute(1, 0, 2).repeat_interleave(g, 0)
    vt = torch.from_numpy(v.astype(np.float64)).permute(1, 0, 2).repeat_interleave(g, 0)
    m = torch.from_numpy(allowed)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=m)
    return o.permute(1, 0, 2).numpy()


def _pack(dense):
    n, T = dense.shape
    W = (T + 63) // 64
    out = np.zeros((n, W), dtype=np.uint64)
    for i in range(n):
        for j in range(T):
            if dense[i, j]:
                out[i, j // 64] |= np.uint64(1) << np.uint64(j % 64)
    return out


@pytest.mark.parametrize("P,n,hq,hkv,D", [(64, 9, 2, 1, 32), (100, 17, 8, 2, 64), (0, 5, 4, 4, 16)])
def test_chain_mask_is_causal_attention(P, n, hq, hkv, D):
    q, k, v, base = _qkv(P + n, 1, n, P, hq, hkv, D)
    causal = np.tril(np.ones((n, n), dtype=bool))
    mask = _pack(causal)[None]
    out, _ = masked_attention(q, k, v, base, [P], [n], mask)
    allowed = np.concatenate([np.ones((n, P), dtype=bool), causal], axis=1)
    want = _sdpa(q[0], k, v, allowed, hq // hkv)
    assert np.abs(out[0] - want).max() < 1e-12


def test_drafter_block_is_unmasked_attention():
    P, n, hq, hkv, D = 200, 16, 8, 2, 32
    q, k, v, base = _qkv(5, 2, n, P, hq, hkv, D)
    out, lse = masked_attention(q, k, v, base, [P, P], [n, n], None)
    for r in range(2):
        kr = k[base[r]:base[r] + P + n]
        vr = v[base[r]:base[r] + P + n]
        want = _sdpa(q[r], kr, vr, np.ones((n, P + n), dtype=bool), hq // hkv)
        assert np.abs(out[r] - want).max() < 1e-12
        s = np.einsum("nhd,thd->nht", q[r].astype(np.float64),
                      np.repeat(kr, hq // hkv, axis=1).astype(np.float64)) / np.sqrt(D)
        assert np.abs(lse[r] - torch.logsumexp(torch.from_numpy(s), dim=-1).numpy()).max() < 1e-12


def test_tree_mask_matches_sdpa_with_dense_mask():
    cfg = synth.CONFIGS[1]
    case = synth.make_case(cfg)
    ids, logp, _ = topk_logprobs(case.logits, cfg.K)
    t = build_tree(logp, ids, int(case.root_token[0]), cfg.k_tree, cfg.B)
    N = cfg.B + 1
    P = int(case.prefix_len[0])
    q = synth.bf16_bits_to_f32(case.vq_bits)
    k = synth.bf16_bits_to_f32(case.vk_bits)
    v = synth.bf16_bits_to_f32(case.vv_bits)
    out, _ = masked_attention(q, k, v, case.kv_base, case.prefix_len, [N], t["mask"][None])
    dense = np.zeros((N, N), dtype=bool)
    for i in range(N):
        a = i
        while a >= 0:
            dense[i, a] = True
            a = int(t["parent"][a]) if a > 0 else -1
    allowed = np.concatenate([np.ones((N, P), dtype=bool), dense], axis=1)
    want = _sdpa(q[0], k[:P + N], v[:P + N], allowed, cfg.hq // cfg.hkv)
    assert np.abs(out[0] - want).max() < 1e-12


def test_root_row_without_prefix_returns_its_value():
    q, k, v, base = _qkv(11, 1, 3, 0, 4, 2, 32)
    mask = _pack(np.tril(np.ones((3, 3), dtype=bool)))[None]
    out, lse = masked_attention(q, k, v, base, [0], [3], mask)
    g = 2
    for h in range(4):
        assert np.array_equal(out[0, 0, h], v[0, h // g].astype(np.float64))
        s = float(q[0, 0, h].astype(np.float64) @ k[0, h // g].astype(np.float64)) / np.sqrt(32)
        assert lse[0, 0, h] == pytest.approx(s, abs=1e-12)


def test_identical_visible_sets_give_identical_rows():
    P, n, hq, hkv, D = 40, 4, 2, 1, 32
    q, k, v, base = _qkv(12, 1, n, P, hq, hkv, D)
    q[0, 3] = q[0, 2]
    dense = np.eye(n, dtype=bool)
    dense[:, 0] = True
    dense[3, 2] = True            # row 3 sees {0, 2, 3}, row 2 sees {0, 2}
    dense[2, 3] = True            # row 2 sees {0, 2, 3} too
    out, _ = masked_attention(q, k, v, base, [P], [n], _pack(dense)[None])
    assert np.array_equal(out[0, 2], out[0, 3])


@pytest.mark.parametrize("n,bl", [(64, 16), (40, 16), (7, 3)])
def test_packed_blocks_match_sdpa_with_block_diagonal_mask(n, bl):
    """Packed drafter blocks: SDPA with every prefix row plus the block-diagonal
    own-row mask (the last block may be short)."""
    P, hq, hkv, D = 96, 8, 2, 32
    q, k, v, base = _qkv(13 + n, 1, n, P, hq, hkv, D)
    out, _ = masked_attention(q, k, v, base, [P], [n], None, block_len=bl)
    blk = np.arange(n) // bl
    allowed = np.concatenate([np.ones((n, P), dtype=bool), blk[:, None] == blk[None, :]], axis=1)
    want = _sdpa(q[0], k, v, allowed, hq // hkv)
    assert np.abs(out[0] - want).max() < 1e-12


def test_packed_block_at_least_n_is_the_dense_drafter_block():
    P, n, hq, hkv, D = 64, 16, 4, 2, 32
    q, k, v, base = _qkv(14, 1, n, P, hq, hkv, D)
    a, la = masked_attention(q, k, v, base, [P], [n], None, block_len=n)
    b, lb = masked_attention(q, k, v, base, [P], [n], None)
    assert np.array_equal(a, b) and np.array_equal(la, lb)


def test_packed_blocks_do_not_leak():
    """Changing the own rows of one block leaves every other block's output
    unchanged."""
    P, n, bl, hq, hkv, D = 50, 48, 16, 4, 1, 32
    q, k, v, base = _qkv(15, 1, n, P, hq, hkv, D)
    a, _ = masked_attention(q, k, v, base, [P], [n], None, block_len=bl)
    k2, v2 = k.copy(), v.copy()
    k2[P + 16:P + 32] += 1.0
    v2[P + 16:P + 32] -= 2.0
    b, _ = masked_attention(q, k2, v2, base, [P], [n], None, block_len=bl)
    assert np.array_equal(a[0, :16], b[0, :16]) and np.array_equal(a[0, 32:], b[0, 32:])
    assert not np.array_equal(a[0, 16:32], b[0, 16:32])
