"""GPU: one workspace reused across calls and across HIP graph replays.

ddt_topk_logprobs and ddt_masked_attention keep chunk / split partials in
the caller's workspace.  These tests reuse a single workspace for several
different inputs in a row, then capture a call in a HIP graph and replay it
several times with new input contents copied in between (eager work and
synchronisation between replays), checking every result against the oracle
to the usual bars: ids exact and log-probs within 1e-5; attention within
2e-2."""
import numpy as np
import pytest
import torch

import synth
from block_diffusion_draft_vocab_amd import ddt
from oracle.attention import masked_attention as oracle_attn
from oracle.logits import topk_logprobs as oracle_topk
from oracle.tree import build_trees as oracle_trees
from tests.helpers import bf16_f32, dev_bf16, mask_to_dev

pytestmark = pytest.mark.gpu


def _check_topk(ids, logp, logits, k):
    oids, ologp, _ = oracle_topk(logits, k)
    assert np.array_equal(ids.cpu().numpy(), oids)
    assert np.abs(logp.cpu().numpy().astype(np.float64) - ologp).max() <= 1e-5


def test_topk_workspace_reuse_and_graph_replay(gpu):
    cfg = synth.CONFIGS[3]
    cases = [synth.make_case(cfg, seed=50 + i, with_drafter=False, with_verify=False)
             for i in range(4)]
    rows, V = cases[0].logits.shape
    ws = torch.zeros(ddt.topk_workspace_size(rows, V, cfg.K), dtype=torch.uint8, device=gpu)
    ids = torch.empty(rows, cfg.K, dtype=torch.int32, device=gpu)
    logp = torch.empty(rows, cfg.K, dtype=torch.float32, device=gpu)
    for c in cases:                                   # eager, one workspace
        lg = torch.from_numpy(c.logits).to(gpu)
        ddt.topk_logprobs(lg, cfg.K, ids=ids, logp=logp, workspace=ws)
        torch.cuda.synchronize()
        _check_topk(ids, logp, c.logits, cfg.K)
    buf = torch.from_numpy(cases[0].logits).to(gpu)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        ddt.topk_logprobs(buf, cfg.K, ids=ids, logp=logp, workspace=ws)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ddt.topk_logprobs(buf, cfg.K, ids=ids, logp=logp, workspace=ws)
    for c in cases[1:] + cases[:1]:                   # replays with new contents
        buf.copy_(torch.from_numpy(c.logits))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _check_topk(ids, logp, c.logits, cfg.K)


def _attn_case(seed, masked):
    cfg = synth.scaled(synth.CONFIGS[3], B=64, prefix=(1000, 1000), hq=8, hkv=2)
    case = synth.make_case(cfg, seed=seed, with_drafter=False)
    N = cfg.B + 1
    mask = None
    if masked:
        ids, logp, _ = oracle_topk(case.logits, cfg.K)
        mask = oracle_trees(logp, ids, case.root_token, 1, cfg.L, cfg.k_tree, cfg.B)["mask"]
    return cfg, case, N, mask


@pytest.mark.parametrize("masked", [True, False], ids=["verify", "drafter"])
def test_attention_workspace_reuse_and_graph_replay(gpu, masked):
    setups = [_attn_case(70 + i, masked) for i in range(4)]
    cfg, case0, N, _ = setups[0]
    P = int(case0.prefix_len[0])
    W = (N + 63) // 64
    desc = ddt.attn_desc(1, cfg.hq, cfg.hkv, cfg.D, N, P + N, W if masked else 0)
    need = ddt.attention_workspace_size(desc)
    assert need > 0                                   # this shape splits the keys
    ws = torch.zeros(need, dtype=torch.uint8, device=gpu)
    kvb = torch.zeros(1, dtype=torch.int64, device=gpu)
    pre = torch.full((1,), P, dtype=torch.int32, device=gpu)
    nq = torch.full((1,), N, dtype=torch.int32, device=gpu)

    def tensors(case, mask):
        return (dev_bf16(case.vq_bits, gpu), dev_bf16(case.vk_bits, gpu),
                dev_bf16(case.vv_bits, gpu), None if mask is None else mask_to_dev(mask, gpu))

    def check(out, lse, case, mask):
        oo, ol = oracle_attn(bf16_f32(case.vq_bits), bf16_f32(case.vk_bits),
                             bf16_f32(case.vv_bits), case.kv_base, case.prefix_len, [N], mask)
        assert np.abs(out.float().cpu().numpy()[0, :N] - oo[0, :N]).max() <= 2e-2
        assert np.abs(lse.cpu().numpy()[0, :N] - ol[0, :N]).max() <= 2e-2

    out = torch.empty(1, N, cfg.hq, cfg.D, dtype=torch.bfloat16, device=gpu)
    lse = torch.empty(1, N, cfg.hq, dtype=torch.float32, device=gpu)
    for _, case, _, mask in setups:                   # eager, one workspace
        q, k, v, m = tensors(case, mask)
        ddt.masked_attention(q, k, v, kvb, pre, nq, m, max_kv_len=P + N, out=out, lse=lse,
                             want_lse=True, workspace=ws)
        torch.cuda.synchronize()
        check(out, lse, case, mask)
    q, k, v, m = tensors(case0, setups[0][3])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        ddt.masked_attention(q, k, v, kvb, pre, nq, m, max_kv_len=P + N, out=out, lse=lse,
                             want_lse=True, workspace=ws)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ddt.masked_attention(q, k, v, kvb, pre, nq, m, max_kv_len=P + N, out=out, lse=lse,
                             want_lse=True, workspace=ws)
    for _, case, _, mask in setups[1:] + setups[:1]:  # replays with new contents
        q2, k2, v2, m2 = tensors(case, mask)
        q.copy_(q2)
        k.copy_(k2)
        v.copy_(v2)
        if m is not None:
            m.copy_(m2)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        check(out, lse, case, mask)


@pytest.mark.parametrize("masked", [True, False], ids=["verify", "drafter"])
def test_attention_empty_splits_ignore_stale_workspace(gpu, masked):
    """A launch planned for a long key range (max_kv_len 4096) on a request
    that only has 100 keys leaves most key splits empty; their workspace
    slots are never written.  Filled with 0xFF bytes (NaN partials), they
    must not reach the result."""
    rng = np.random.default_rng(91)
    n, P, hq, hkv, D = 20, 80, 8, 2, 128
    q = synth.f32_to_bf16_bits(rng.standard_normal((1, n, hq, D), dtype=np.float32))
    k = synth.f32_to_bf16_bits(rng.standard_normal((P + n, hkv, D), dtype=np.float32))
    v = synth.f32_to_bf16_bits(rng.standard_normal((P + n, hkv, D), dtype=np.float32))
    mask = None
    if masked:
        from oracle.tree import ancestor_mask
        parent = np.array([-1] + [int(rng.integers(0, i)) for i in range(1, n)], np.int32)
        mask = ancestor_mask(parent, n, n)[None]
    desc = ddt.attn_desc(1, hq, hkv, D, n, 4096, 1 if masked else 0)
    ws = torch.full((ddt.attention_workspace_size(desc),), 0xFF, dtype=torch.uint8, device=gpu)
    out, lse = ddt.masked_attention(
        dev_bf16(q, gpu), dev_bf16(k, gpu), dev_bf16(v, gpu),
        torch.zeros(1, dtype=torch.int64, device=gpu), torch.full((1,), P, dtype=torch.int32,
                                                                   device=gpu),
        torch.full((1,), n, dtype=torch.int32, device=gpu),
        None if mask is None else mask_to_dev(mask, gpu), max_kv_len=4096, want_lse=True,
        workspace=ws)
    torch.cuda.synchronize()
    oo, ol = oracle_attn(bf16_f32(q), bf16_f32(k), bf16_f32(v), [0], [P], [n], mask)
    assert np.abs(out.float().cpu().numpy()[0] - oo[0]).max() <= 2e-2
    assert np.abs(lse.cpu().numpy()[0] - ol[0]).max() <= 2e-2
