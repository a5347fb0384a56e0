"""GPU parity: ddt_accept_compact vs the oracle's walk + compaction.

Bar: accept_len, the accepted path, the bonus token, new_len and every KV
row [0, new_len) of every layer are bit-identical given the same tree and
target.  Trees come from the oracle; targets from the synthetic target
model (sampled path) and forced paths that end at chosen nodes (every node
of the tiny tree; deep nodes of the deep regime).  Also: the ragged serving
batch, an overlapping-rows path, n_layers = 0, and determinism."""
import numpy as np
import pytest
import torch

import synth
from block_diffusion_draft_vocab_amd import ddt
from oracle.accept import accept_compact as oracle_accept
from oracle.logits import topk_logprobs as oracle_topk
from oracle.tree import build_trees as oracle_trees
from tests.helpers import dev_bf16, host_bf16_bits

pytestmark = pytest.mark.gpu


def _caches(seed, n_layers, rows, hkv, D):
    rng = np.random.default_rng(seed)
    k = rng.integers(0, 65536, (n_layers, rows, hkv, D), dtype=np.uint16)
    v = rng.integers(0, 65536, (n_layers, rows, hkv, D), dtype=np.uint16)
    return k, v


def _gpu_accept(gpu, tok, par, n_nodes, tgt, L, k, v, kv_base, prefix):
    kd = dev_bf16(k, gpu) if k is not None else None
    vd = dev_bf16(v, gpu) if v is not None else None
    out = ddt.accept_compact(
        torch.from_numpy(np.ascontiguousarray(tok, np.int32)).to(gpu),
        torch.from_numpy(np.ascontiguousarray(par, np.int32)).to(gpu),
        torch.from_numpy(np.asarray(n_nodes, np.int32)).to(gpu),
        torch.from_numpy(np.ascontiguousarray(tgt, np.int32)).to(gpu), L, kd, vd,
        torch.from_numpy(np.asarray(kv_base, np.int64)).to(gpu),
        torch.from_numpy(np.asarray(prefix, np.int32)).to(gpu))
    torch.cuda.synchronize()
    res = {kk: vv.cpu().numpy() for kk, vv in out.items()}
    if kd is not None:
        res["k"] = host_bf16_bits(kd)
        res["v"] = host_bf16_bits(vd)
    return res


def _check(gpu, tok, par, n_nodes, tgt, L, k, v, kv_base, prefix):
    g = _gpu_accept(gpu, tok, par, n_nodes, tgt, L, k, v, kv_base, prefix)
    acc, path, bonus, new_len, ko, vo = oracle_accept(tok, par, n_nodes, tgt, L, k, v, kv_base,
                                                      prefix)
    assert np.array_equal(g["accept_len"], acc)
    assert np.array_equal(g["accepted"], path)
    assert np.array_equal(g["bonus"], bonus)
    assert np.array_equal(g["new_len"], new_len)
    for r in range(len(n_nodes)):
        lo = int(kv_base[r])
        hi = lo + int(new_len[r])
        assert np.array_equal(g["k"][:, lo:hi], ko[:, lo:hi]), r
        assert np.array_equal(g["v"][:, lo:hi], vo[:, lo:hi]), r
    return g


def _tree(cfg):
    case = synth.make_case(cfg, with_drafter=False, with_verify=False)
    ids, logp, _ = oracle_topk(case.logits, cfg.K, cfg.inv_temperature)
    return case, oracle_trees(logp, ids, case.root_token, cfg.batch, cfg.L, cfg.k_tree, cfg.B)


def test_every_forced_stop_tiny(gpu):
    cfg = synth.CONFIGS[1]
    case, t = _tree(cfg)
    n = int(t["n_nodes"][0])
    P = 20
    for stop in range(n):
        tgt = synth.force_path_target(t["token"][0], t["parent"][0], t["depth"][0], n, stop,
                                      case.off_path[0], cfg.vocab)
        k, v = _caches(stop, 3, P + cfg.B + 1, 1, 32)
        g = _check(gpu, t["token"], t["parent"], t["n_nodes"], tgt[None], cfg.L, k, v, [0], [P])
        assert g["accept_len"][0] == t["depth"][0][stop]


@pytest.mark.parametrize("cfg", [synth.CONFIGS[3], synth.DEEP], ids=["c3", "deep"])
def test_sampled_and_forced_paths(gpu, cfg):
    case, t = _tree(cfg)
    n = int(t["n_nodes"][0])
    y = synth.sample_target_path(case)
    P = int(case.prefix_len[0])
    rows = P + cfg.B + 1
    k, v = _caches(1, 2, rows, cfg.hkv, cfg.D)
    tgt = synth.target_for_tree(t["token"][0], t["parent"][0], t["depth"][0], n, y[0],
                                case.off_path[0])
    _check(gpu, t["token"], t["parent"], t["n_nodes"], tgt[None], cfg.L, k, v, [0], [P])
    deepest = np.argsort(-t["depth"][0][:n], kind="stable")[:5]
    for stop in deepest:
        tgt = synth.force_path_target(t["token"][0], t["parent"][0], t["depth"][0], n,
                                      int(stop), case.off_path[0], cfg.vocab)
        g = _check(gpu, t["token"], t["parent"], t["n_nodes"], tgt[None], cfg.L, k, v, [0], [P])
        assert g["accept_len"][0] == t["depth"][0][stop]


def test_serving_batch(gpu):
    cfg = synth.CONFIGS[5]
    case, t = _tree(cfg)
    y = synth.sample_target_path(case)
    N = cfg.B + 1
    tgt = np.stack([synth.target_for_tree(t["token"][r], t["parent"][r], t["depth"][r],
                                          int(t["n_nodes"][r]), y[r], case.off_path[r])
                    for r in range(cfg.batch)])
    # force longer walks on every other request
    for r in range(0, cfg.batch, 2):
        n = int(t["n_nodes"][r])
        stop = int(np.argmax(t["depth"][r][:n]))
        tgt[r] = synth.force_path_target(t["token"][r], t["parent"][r], t["depth"][r], n, stop,
                                         case.off_path[r], cfg.vocab)
    # small per-request prefixes keep the host copies light; bases are ragged
    prefix = (case.prefix_len // 64).astype(np.int32)
    cap = prefix.astype(np.int64) + N
    base = np.concatenate([[0], np.cumsum(cap)[:-1]]).astype(np.int64)
    k, v = _caches(5, 2, int(cap.sum()), cfg.hkv, cfg.D)
    _check(gpu, t["token"], t["parent"], t["n_nodes"], tgt, cfg.L, k, v, base, prefix)


def test_overlapping_rows(gpu):
    tok = np.array([[0, 10, 11, 12, 13, 14]], np.int32)
    par = np.array([[-1, 0, 0, 1, 1, 2]], np.int32)
    tgt = np.array([[11, 0, 14, 0, 0, 77]], np.int32)
    k, v = _caches(9, 4, 3 + 6, 2, 64)
    g = _check(gpu, tok, par, [6], tgt, 4, k, v, [0], [3])
    assert g["accepted"][0, :3].tolist() == [0, 2, 5]


def test_no_layers(gpu):
    tok = np.array([[5, 1, 2]], np.int32)
    par = np.array([[-1, 0, 1]], np.int32)
    tgt = np.array([[1, 2, 9]], np.int32)
    out = ddt.accept_compact(torch.from_numpy(tok).to(gpu), torch.from_numpy(par).to(gpu),
                             torch.tensor([3], dtype=torch.int32, device=gpu),
                             torch.from_numpy(tgt).to(gpu), 4, None, None, None,
                             torch.tensor([100], dtype=torch.int32, device=gpu))
    torch.cuda.synchronize()
    assert out["accept_len"].item() == 2 and out["bonus"].item() == 9
    assert out["new_len"].item() == 103
    assert out["accepted"].cpu().tolist() == [[0, 1, 2, -1, -1]]


def test_wide_slot_arrays(gpu):
    """n_max = 20000 (the walk's slot table is 80 KB of on-chip memory): a
    five-node tree in wide arrays walks and compacts as the oracle does."""
    n_max, L = 20000, 4
    tok = np.full((1, n_max), -1, np.int32)
    par = np.full((1, n_max), -1, np.int32)
    tgt = np.full((1, n_max), 7, np.int32)
    tok[0, :5] = [5, 1, 3, 8, 2]
    par[0, :5] = [-1, 0, 0, 1, 2]
    tgt[0, :5] = [3, 4, 2, 4, 9]          # root -> slot 2 -> slot 4, bonus 9
    rows, hkv, D, P = 64, 2, 16, 40
    rng = np.random.default_rng(5)
    kbits = rng.integers(0, 2 ** 15, size=(1, rows, hkv, D), dtype=np.int64).astype(np.uint16)
    vbits = rng.integers(0, 2 ** 15, size=(1, rows, hkv, D), dtype=np.int64).astype(np.uint16)
    kc = torch.from_numpy(kbits.view(np.int16)).to(gpu).view(torch.bfloat16)
    vc = torch.from_numpy(vbits.view(np.int16)).to(gpu).view(torch.bfloat16)
    base = np.zeros(1, np.int64)
    prefix = np.array([P], np.int32)
    nn = np.array([5], np.int32)
    out = ddt.accept_compact(torch.from_numpy(tok).to(gpu), torch.from_numpy(par).to(gpu),
                             torch.from_numpy(nn).to(gpu), torch.from_numpy(tgt).to(gpu), L,
                             kc, vc, torch.from_numpy(base).to(gpu),
                             torch.from_numpy(prefix).to(gpu))
    torch.cuda.synchronize()
    oacc, opath, obonus, onew, okc, ovc = oracle_accept(tok, par, nn, tgt, L, kbits, vbits, base,
                                                        prefix)
    assert out["accept_len"].item() == int(oacc[0]) == 2
    assert out["bonus"].item() == int(obonus[0]) == 9
    assert out["new_len"].item() == int(onew[0]) == P + 3
    assert out["accepted"].cpu().tolist() == [[0, 2, 4, -1, -1]]
    assert np.array_equal(host_bf16_bits(kc), okc)
    assert np.array_equal(host_bf16_bits(vc), ovc)


def test_long_path_several_rounds(gpu):
    """An accepted path of 1100 nodes (more rows than one register round of
    the compaction holds: 1024 per tensor) whose nodes sit at every other
    slot, so rows of the first round's sources are the second round's
    destinations."""
    plen = 1100
    n = 2 * plen + 1
    tok = np.zeros((1, n), np.int32)
    par = np.full((1, n), -1, np.int32)
    tgt = np.full((1, n), 3, np.int32)
    for j in range(1, plen + 1):
        on, off = 2 * j, 2 * j - 1                     # path node, and a leaf beside it
        prev = 2 * (j - 1)
        par[0, on] = prev
        par[0, off] = prev
        tok[0, on] = 1000 + j
        tok[0, off] = 5000 + j
        tgt[0, prev] = 1000 + j
    tgt[0, 2 * plen] = 42                              # bonus
    P = 5
    k, v = _caches(21, 2, P + n, 1, 64)
    g = _check(gpu, tok, par, [n], tgt, plen, k, v, [0], [P])
    assert g["accept_len"][0] == plen and g["bonus"][0] == 42


def test_deterministic(gpu):
    """Two runs on the same inputs give identical outputs and caches."""
    cfg = synth.CONFIGS[5]
    case, t = _tree(cfg)
    y = synth.sample_target_path(case)
    tgt = np.stack([synth.target_for_tree(t["token"][r], t["parent"][r], t["depth"][r],
                                          int(t["n_nodes"][r]), y[r], case.off_path[r])
                    for r in range(cfg.batch)])
    for r in range(0, cfg.batch, 3):
        n = int(t["n_nodes"][r])
        stop = int(np.argmax(t["depth"][r][:n]))
        tgt[r] = synth.force_path_target(t["token"][r], t["parent"][r], t["depth"][r], n, stop,
                                         case.off_path[r], cfg.vocab)
    N = cfg.B + 1
    prefix = np.full(cfg.batch, 7, np.int32)
    base = np.arange(cfg.batch, dtype=np.int64) * (7 + N)
    k, v = _caches(23, 3, int(base[-1]) + 7 + N, cfg.hkv, cfg.D)
    a = _gpu_accept(gpu, t["token"], t["parent"], t["n_nodes"], tgt, cfg.L, k, v, base, prefix)
    b = _gpu_accept(gpu, t["token"], t["parent"], t["n_nodes"], tgt, cfg.L, k, v, base, prefix)
    for key in a:
        assert np.array_equal(a[key], b[key]), key
