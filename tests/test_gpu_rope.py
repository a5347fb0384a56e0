"""GPU parity: ddt_tree_rope_kv (tree positions, rotary embedding, tree K/V
scatter) vs the oracle.

Bar: positions exact; every bf16 output bit-exact (both sides evaluate the
rotation in double and round to float, then to bf16); rows outside the tree
block and padding slots untouched.  Cases: the C3 tree (B=256, P=2048,
32/8/128), a serving batch of 32 trees with ragged P and n_nodes (32/4/128),
a chain (ordinary positions), head dims 32/64/256, and a non-zero kv_base."""
import numpy as np
import pytest
import torch

import synth
from block_diffusion_draft_vocab_amd import ddt
from oracle.logits import topk_logprobs
from oracle.rope import tree_rope_kv as oracle_rope
from oracle.tree import build_trees

pytestmark = pytest.mark.gpu


def _bits(rng, *shape):
    return synth.f32_to_bf16_bits(rng.standard_normal(shape).astype(np.float32))


def _dev(bits, gpu):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(gpu).view(torch.bfloat16)


def _host(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _run_and_check(gpu, depth, n_nodes, prefix, kv_base, hq, hkv, D, rows, base, seed):
    rng = np.random.default_rng(seed)
    b, n_max = depth.shape
    q = _bits(rng, b, n_max, hq, D)
    kn = _bits(rng, b, n_max, hkv, D)
    vn = _bits(rng, b, n_max, hkv, D)
    kc = _bits(rng, rows, hkv, D)
    vc = _bits(rng, rows, hkv, D)
    opos, oq, okc, ovc = oracle_rope(depth, n_nodes, prefix, kv_base, q, kn, vn, kc, vc, base)
    tq, tkc, tvc = _dev(q, gpu), _dev(kc, gpu), _dev(vc, gpu)
    pos = ddt.tree_rope_kv(torch.from_numpy(depth).to(gpu), torch.from_numpy(n_nodes).to(gpu),
                           torch.from_numpy(prefix).to(gpu), torch.from_numpy(kv_base).to(gpu),
                           tq, _dev(kn, gpu), _dev(vn, gpu), tkc, tvc, base)
    torch.cuda.synchronize()
    assert np.array_equal(pos.cpu().numpy(), opos)
    assert np.array_equal(_host(tq), oq)
    assert np.array_equal(_host(tkc), okc)
    assert np.array_equal(_host(tvc), ovc)
    return opos


def test_rope_c3_tree(gpu):
    cfg = synth.CONFIGS[3]
    case = synth.make_case(cfg, with_drafter=False, with_verify=False)
    ids, logp, _ = topk_logprobs(case.logits, cfg.K)
    t = build_trees(logp, ids, case.root_token, 1, cfg.L, cfg.k_tree, cfg.B)
    depth = t["depth"].astype(np.int32)
    n_nodes = t["n_nodes"].astype(np.int32)
    P = 2048
    _run_and_check(gpu, depth, n_nodes, np.array([P], np.int32), np.zeros(1, np.int64),
                   32, 8, 128, P + cfg.B + 1 + 5, 1.0e6, 1)


def test_rope_serving_batch_ragged(gpu):
    rng = np.random.default_rng(7)
    b, n_max = 32, 65
    n_nodes = rng.integers(1, n_max + 1, size=b).astype(np.int32)
    depth = np.full((b, n_max), -1, np.int32)
    for r in range(b):
        # any parent-before-child tree: depth of slot i = depth(parent) + 1
        d = [0]
        for i in range(1, n_nodes[r]):
            d.append(d[int(rng.integers(0, i))] + 1)
        depth[r, :n_nodes[r]] = d
    prefix = rng.integers(512, 8193, size=b).astype(np.int32)
    kv_base = np.zeros(b, np.int64)
    kv_base[1:] = np.cumsum(prefix[:-1].astype(np.int64) + n_max)
    rows = int(kv_base[-1] + prefix[-1] + n_max)
    _run_and_check(gpu, depth, n_nodes, prefix, kv_base, 32, 4, 128, rows, 1.0e6, 2)


def test_rope_chain_positions(gpu):
    n = 17
    depth = np.arange(n, dtype=np.int32)[None]
    pos = _run_and_check(gpu, depth, np.array([n], np.int32), np.array([100], np.int32),
                         np.array([3], np.int64), 4, 2, 64, 200, 1.0e4, 3)
    assert pos[0].tolist() == list(range(100, 100 + n))


@pytest.mark.parametrize("D,hq,hkv", [(32, 2, 1), (64, 8, 8), (256, 16, 2)])
def test_rope_head_dims(gpu, D, hq, hkv):
    depth = np.array([[0, 1, 1, 2, 3, 2, -1, -1]], np.int32)
    _run_and_check(gpu, depth, np.array([6], np.int32), np.array([9000], np.int32),
                   np.array([5], np.int64), hq, hkv, D, 9100, 5.0e5, 4 + D)
