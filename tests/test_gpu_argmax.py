"""GPU parity: ddt_argmax (the target's greedy token per tree slot) vs the
oracle's arg-max.

Bar: ids bit-exact and maxima equal as floats (an arg-max is an index
decision on float32 values both sides read unchanged; a -0 maximum is
reported as +0).  Cases: the verify-logit shape at full
size (257 slots x 151936), a serving batch (32 x 65 slots), ragged vocab
sizes around the 8192-float chunk and the 4-float load group, strided rows
with larger junk past the vocab, a misaligned base (scalar loads), planted
ties inside one thread, across waves and across chunks, -inf / +inf / -0
rows, workspace reuse with graph replay, and agreement with the K = 1
top-K pass."""
import numpy as np
import pytest
import torch

import synth
from block_diffusion_draft_vocab_amd import ddt
from oracle.logits import argmax_rows as oracle_argmax
from oracle.logits import topk_logprobs as oracle_topk

pytestmark = pytest.mark.gpu


def _dev(gpu, z, ld=None, junk=3.0e38):
    rows, V = z.shape
    if ld is None or ld == V:
        return torch.from_numpy(np.ascontiguousarray(z)).to(gpu)
    buf = np.full((rows, ld), junk, dtype=np.float32)   # larger than any logit
    buf[:, :V] = z
    return torch.from_numpy(buf).to(gpu)


def _check(gpu, z, ld=None, offset=0):
    rows, V = z.shape
    if offset:
        # view that starts `offset` floats into its allocation: scalar loads
        flat = np.full(rows * V + offset, 3.0e38, dtype=np.float32)
        flat[offset:] = z.ravel()
        base = torch.from_numpy(flat).to(gpu)
        dl = base[offset:].view(rows, V)
    else:
        dl = _dev(gpu, z, ld)
    ids, mx = ddt.argmax(dl, vocab=V, want_max=True)
    torch.cuda.synchronize()
    oids, omx = oracle_argmax(z)
    assert np.array_equal(ids.cpu().numpy(), oids)
    # values compare as floats: a -0 maximum comes back as +0 (equal)
    assert np.array_equal(mx.cpu().numpy(), omx)


def test_argmax_verify_logits_full_size(gpu):
    z, planted = synth.make_verify_logits(31, 257)
    _check(gpu, z)


def test_argmax_serving_batch(gpu):
    z, _ = synth.make_verify_logits(32, 32 * 65)
    _check(gpu, z)


@pytest.mark.parametrize("rows,V", [(1, 1), (2, 5), (3, 1000), (5, 8192), (5, 8193),
                                    (4, 8195), (7, 16387), (3, 24577), (2, 151937)])
def test_argmax_ragged_vocab(gpu, rows, V):
    z, _ = synth.make_verify_logits(40 + V % 97, rows, V, peak=0.0)
    _check(gpu, z)


def test_argmax_strided_rows_with_junk(gpu):
    z, _ = synth.make_verify_logits(41, 6, 151936)
    _check(gpu, z, ld=151936 + 40)
    z2, _ = synth.make_verify_logits(42, 3, 9001, peak=0.0)
    _check(gpu, z2, ld=9005)


def test_argmax_misaligned_scalar_path(gpu):
    z, _ = synth.make_verify_logits(43, 5, 20001)
    _check(gpu, z, offset=1)


def test_argmax_planted_ties(gpu):
    V = 151936
    z, _ = synth.make_verify_logits(44, 10, V, peak=0.0)
    top = np.float32(50.0)
    # thread t of a 256-thread chunk holds floats 4t..4t+3, then 1024+4t..
    cases = [
        [5, 6],                 # same 4-float group
        [1024 * 3 + 4, 4],      # same thread, different groups (later planted first)
        [64 * 4 + 1, 3],        # different waves of one chunk
        [8192 * 7 + 5, 8192 * 2 + 100],   # different chunks
        [V - 1, V - 2],         # the last two columns
        [0, V - 1],
        [8191, 8192],           # both sides of a chunk boundary
    ]
    for r, cols in enumerate(cases):
        z[r, cols] = top
    z[7, :] = np.float32(-2.5)  # constant row
    z[8, :] = np.float32(-np.inf)
    z[9, :] = np.float32(-1.0)
    z[9, 9000] = np.float32(-0.0)
    z[9, 12000] = np.float32(0.0)
    _check(gpu, z)
    z[0, :] = np.float32(np.inf)   # all +inf: index 0
    _check(gpu, z)


def test_argmax_matches_topk_k1(gpu):
    z, _ = synth.make_verify_logits(45, 64)
    dl = _dev(gpu, z)
    ids, _ = ddt.argmax(dl)
    tk, _, _ = ddt.topk_logprobs(dl, 1)
    torch.cuda.synchronize()
    assert np.array_equal(ids.cpu().numpy(), tk.cpu().numpy()[:, 0])
    oids, _, _ = oracle_topk(z[:8], 1)
    assert np.array_equal(tk.cpu().numpy()[:8, 0], oids[:, 0])


def test_argmax_workspace_reuse_and_graph_replay(gpu):
    sets = [synth.make_verify_logits(50 + i, 257)[0] for i in range(3)]
    rows, V = sets[0].shape
    ws = torch.zeros(ddt.argmax_workspace_size(rows, V), dtype=torch.uint8, device=gpu)
    ids = torch.empty(rows, dtype=torch.int32, device=gpu)
    for z in sets:                                    # eager, one workspace
        ddt.argmax(_dev(gpu, z), ids=ids, workspace=ws)
        torch.cuda.synchronize()
        assert np.array_equal(ids.cpu().numpy(), oracle_argmax(z)[0])
    buf = _dev(gpu, sets[0])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        ddt.argmax(buf, ids=ids, workspace=ws)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ddt.argmax(buf, ids=ids, workspace=ws)
    for z in sets[1:] + sets[:1]:                     # replays with new contents
        buf.copy_(torch.from_numpy(z))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(ids.cpu().numpy(), oracle_argmax(z)[0])
