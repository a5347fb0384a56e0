"""GPU parity: ddt_packed_block_attention (packed drafter blocks, block-
diagonal own rows) vs the oracle's float64 attention.

Bar: max |out - oracle| <= 2e-2 and lse within 2e-2 (the attention bar).
Cases: four packed 16-row drafter blocks over the 2048-row context at the
drafter's head shape (32/8/128), a short last block, block_len 1 (each query
sees the context and itself) and block_len >= n_q (the dense drafter block,
compared with ddt_masked_attention's drafter mode bit for bit), a ragged
two-request batch, head dims 32/64, and many blocks that span key tiles."""
import numpy as np
import pytest
import torch

import synth
from block_diffusion_draft_vocab_amd import ddt
from oracle.attention import masked_attention as oracle_attn
from tests.helpers import bf16_f32, dev_bf16

pytestmark = pytest.mark.gpu
TOL = 2e-2


def _case(seed, b, nq_max, prefix, hq, hkv, D):
    rng = np.random.default_rng(seed)
    q = synth.f32_to_bf16_bits(rng.standard_normal((b, nq_max, hq, D), dtype=np.float32))
    cap = np.asarray(prefix, np.int64) + nq_max
    base = np.concatenate([[0], np.cumsum(cap)[:-1]]).astype(np.int64)
    rows = int(cap.sum())
    k = synth.f32_to_bf16_bits(rng.standard_normal((rows, hkv, D), dtype=np.float32))
    v = synth.f32_to_bf16_bits(rng.standard_normal((rows, hkv, D), dtype=np.float32))
    return q, k, v, base


def _run(gpu, q, k, v, base, prefix, n_q, block_len):
    t = lambda a, dt: torch.from_numpy(np.asarray(a, dt)).to(gpu)
    out, lse = ddt.masked_attention(dev_bf16(q, gpu), dev_bf16(k, gpu), dev_bf16(v, gpu),
                                    t(base, np.int64), t(prefix, np.int32), t(n_q, np.int32),
                                    None, max_kv_len=int(max(p + n for p, n in zip(prefix, n_q))),
                                    want_lse=True, block_len=block_len)
    torch.cuda.synchronize()
    return out, lse


@pytest.mark.parametrize("b,nq,n_q,prefix,hq,hkv,D,bl", [
    (1, 64, [64], [2048], 32, 8, 128, 16),      # four packed drafter blocks
    (1, 40, [40], [2048], 32, 8, 128, 16),      # short last block
    (1, 64, [64], [300], 32, 8, 128, 1),        # each query: context + itself
    (2, 80, [80, 33], [130, 0], 8, 2, 64, 16),  # ragged batch, empty prefix
    (1, 200, [200], [64], 4, 1, 32, 24),        # blocks across key tiles
])
def test_packed_blocks(gpu, b, nq, n_q, prefix, hq, hkv, D, bl):
    q, k, v, base = _case(b * 100 + nq + bl, b, nq, prefix, hq, hkv, D)
    out, lse = _run(gpu, q, k, v, base, prefix, n_q, bl)
    oout, olse = oracle_attn(bf16_f32(q), bf16_f32(k), bf16_f32(v), base, prefix, n_q, None,
                             block_len=bl)
    out = out.float().cpu().numpy()
    lse = lse.cpu().numpy()
    for r in range(b):
        n = n_q[r]
        assert np.abs(out[r, :n] - oout[r, :n]).max() <= TOL
        assert np.abs(lse[r, :n] - olse[r, :n]).max() <= TOL


def test_block_at_least_n_q_is_the_drafter_block(gpu):
    q, k, v, base = _case(7, 1, 16, [2048], 32, 8, 128)
    a, la = _run(gpu, q, k, v, base, [2048], [16], 16)
    b, lb = _run(gpu, q, k, v, base, [2048], [16], 0)
    assert torch.equal(a, b) and torch.equal(la, lb)
