"""The allocation-free top-K entry point (ddt_topk_logprobs_noalloc) against
the workspace one (ddt_topk_logprobs), called through the C ABI.

Bar: the logit pass's (ids bit-exact, log-probs and lse within 1e-5); the two
share their kernels, so the outputs are in fact compared bit for bit.  Two
calls in a row on the library's one scratch array, the second with a smaller
input (512 x 151936, K = 16, then 16 x 151936, K = 32), and a third that
reuses the first shape after the smaller call."""
import ctypes

import numpy as np
import pytest
import torch

import synth
from block_diffusion_draft_vocab_amd import ddt

pytestmark = pytest.mark.gpu


def _call(lib, fn, logits, k, ws=None):
    rows, V = logits.shape
    ids = torch.full((rows, k), -7, dtype=torch.int32, device=logits.device)
    logp = torch.full((rows, k), 7.0, dtype=torch.float32, device=logits.device)
    lse = torch.full((rows,), 7.0, dtype=torch.float32, device=logits.device)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    p = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    if fn == "noalloc":
        st = lib.ddt_topk_logprobs_noalloc(p(logits), V, rows, V, k, 1.0, p(ids), p(logp),
                                           p(lse), stream)
    else:
        st = lib.ddt_topk_logprobs(p(logits), V, rows, V, k, 1.0, p(ids), p(logp), p(lse),
                                   p(ws), ws.numel(), stream)
    assert st == ddt.DDT_OK, st
    torch.cuda.synchronize()
    return ids.cpu().numpy(), logp.cpu().numpy(), lse.cpu().numpy()


def _same(a, b):
    assert np.array_equal(a[0], b[0])
    assert np.array_equal(a[1].view(np.uint32), b[1].view(np.uint32))
    assert np.array_equal(a[2].view(np.uint32), b[2].view(np.uint32))


def test_noalloc_matches_workspace_entry_point(gpu):
    lib = ddt.load()
    big_cfg, small_cfg = synth.CONFIGS[5], synth.CONFIGS[3]
    big = torch.from_numpy(
        synth.make_case(big_cfg, with_drafter=False, with_verify=False).logits).to(gpu)
    small = torch.from_numpy(
        synth.make_case(small_cfg, with_drafter=False, with_verify=False).logits).to(gpu)
    cases = [(big, big_cfg.K), (small, small_cfg.K), (big, big_cfg.K)]
    for logits, k in cases:
        rows, V = logits.shape
        ws = torch.empty(lib.ddt_topk_logprobs_workspace_size(rows, V, k), dtype=torch.uint8,
                         device=gpu)
        ref = _call(lib, "workspace", logits, k, ws)
        got = _call(lib, "noalloc", logits, k)
        _same(ref, got)
        assert np.all(got[0] >= 0) and np.all(got[1] <= 0)
