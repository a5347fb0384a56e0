"""Entry points launched on a caller-supplied stream (``stream=``).

The binding makes the given stream torch's current stream for the call, so
the workspace and outputs it allocates belong to the stream the kernels run
on.  Bar: results on a side stream, with allocations churning on the default
stream meanwhile, are bit-identical to the same calls on the default stream."""
import numpy as np
import pytest
import torch

import synth
from block_diffusion_draft_vocab_amd import ddt
from tests.helpers import dev_bf16

pytestmark = pytest.mark.gpu


def _inputs(gpu, case):
    d = {
        "logits": torch.from_numpy(case.logits).to(gpu),
        "root": torch.from_numpy(case.root_token).to(gpu),
        "q": dev_bf16(case.vq_bits, gpu), "k": dev_bf16(case.vk_bits, gpu),
        "v": dev_bf16(case.vv_bits, gpu), "base": torch.from_numpy(case.kv_base).to(gpu),
        "prefix": torch.from_numpy(case.prefix_len).to(gpu),
    }
    torch.cuda.synchronize()
    return d


def _step(d, case, cfg, stream=None):
    N = cfg.B + 1
    kw = {} if stream is None else {"stream": stream}
    ids, logp, lse = ddt.topk_logprobs(d["logits"], cfg.K, **kw)
    tree = ddt.build_tree(logp, ids, d["root"], cfg.batch, cfg.L, cfg.k_tree, cfg.B, **kw)
    out = ddt.masked_attention(d["q"], d["k"], d["v"], d["base"], d["prefix"], tree["n_nodes"],
                               tree["mask"], max_kv_len=int(case.prefix_len.max()) + N, **kw)
    am, _ = ddt.argmax(d["logits"], **kw)
    return [ids, logp, lse, tree["token"], tree["mask"], out, am]


def test_side_stream_matches_default(gpu):
    cfg = synth.CONFIGS[3]
    case = synth.make_case(cfg, with_drafter=False)
    d = _inputs(gpu, case)
    ref = [t.cpu() for t in _step(d, case, cfg)]
    side = torch.cuda.Stream()
    torch.cuda.synchronize()
    for rep in range(3):
        res = _step(d, case, cfg, stream=side)
        # churn the default stream's pool while the side stream works
        junk = [torch.empty(1 << 20, dtype=torch.uint8, device=gpu).fill_(rep) for _ in range(8)]
        del junk
        side.synchronize()
        for a, b in zip(ref, res):
            assert torch.equal(a, b.cpu()), rep
        del res
