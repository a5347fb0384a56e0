"""A whole draft-and-verify step captured in one HIP graph and replayed.

The step at full size (drafter attention over 2048 + 16 rows, top-32 over
16 x 151936, tree of budget 256, verify attention of 257 rows, acceptance
and compaction of one layer) is captured once on fixed buffers.  Each
replay follows new contents copied into those buffers (eager work between
replays) and must reproduce the eager calls on the same inputs bit for bit:
every kernel of the chain is deterministic, and none may depend on state a
previous call left behind (counters, flags, memsets inside the graph)."""
import numpy as np
import pytest
import torch

import synth
from block_diffusion_draft_vocab_amd import ddt
from tests.helpers import dev_bf16

pytestmark = pytest.mark.gpu


class _Buffers:
    def __init__(self, gpu, cfg, case):
        L, N, ctx = cfg.L, cfg.B + 1, cfg.drafter_ctx
        self.logits = torch.from_numpy(case.logits).to(gpu)
        self.root = torch.from_numpy(case.root_token).to(gpu)
        self.dq, self.dk, self.dv = (dev_bf16(case.dq_bits, gpu), dev_bf16(case.dk_bits, gpu),
                                     dev_bf16(case.dv_bits, gpu))
        self.vq, self.vk, self.vv = (dev_bf16(case.vq_bits, gpu), dev_bf16(case.vk_bits, gpu),
                                     dev_bf16(case.vv_bits, gpu))
        self.kv_base = torch.from_numpy(case.kv_base).to(gpu)
        self.prefix = torch.from_numpy(case.prefix_len).to(gpu)
        self.d_base = torch.zeros(1, dtype=torch.int64, device=gpu)
        self.d_prefix = torch.full((1,), ctx, dtype=torch.int32, device=gpu)
        self.d_nq = torch.full((1,), L, dtype=torch.int32, device=gpu)
        self.target = torch.zeros(1, N, dtype=torch.int32, device=gpu)
        self.d_out = torch.empty_like(self.dq)
        self.v_out = torch.empty_like(self.vq)
        self.ids = torch.empty(L, cfg.K, dtype=torch.int32, device=gpu)
        self.logp = torch.empty(L, cfg.K, dtype=torch.float32, device=gpu)
        self.lse = torch.empty(L, dtype=torch.float32, device=gpu)
        W = (N + 63) // 64
        self.tree = {k: torch.empty(shape, dtype=dt, device=gpu) for k, shape, dt in (
            ("n_nodes", (1,), torch.int32), ("token", (1, N), torch.int32),
            ("parent", (1, N), torch.int32), ("depth", (1, N), torch.int32),
            ("score", (1, N), torch.float32), ("mask", (1, N, W), torch.int64))}
        self.acc = {k: torch.empty(shape, dtype=torch.int32, device=gpu) for k, shape in (
            ("accept_len", (1,)), ("accepted", (1, L + 1)), ("bonus", (1,)), ("new_len", (1,)))}

    def load(self, case, target):
        self.logits.copy_(torch.from_numpy(case.logits))
        self.root.copy_(torch.from_numpy(case.root_token))
        for dst, bits in ((self.dq, case.dq_bits), (self.dk, case.dk_bits),
                          (self.dv, case.dv_bits), (self.vq, case.vq_bits),
                          (self.vk, case.vk_bits), (self.vv, case.vv_bits)):
            dst.view(torch.int16).copy_(
                torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)))
        self.target.copy_(torch.from_numpy(target))

    def snapshot(self):
        out = {"d_out": self.d_out, "ids": self.ids, "logp": self.logp, "lse": self.lse,
               "v_out": self.v_out, "k_after": self.vk, "v_after": self.vv}
        out.update({"tree_" + k: v for k, v in self.tree.items()})
        out.update({"acc_" + k: v for k, v in self.acc.items()})
        return {k: v.view(torch.int16).cpu().numpy() if v.dtype == torch.bfloat16
                else v.cpu().numpy() for k, v in out.items()}


def _step_calls(cfg, bufs, ws):
    L, N, B, ctx, P = cfg.L, cfg.B + 1, cfg.B, cfg.drafter_ctx, cfg.prefix[0]
    s = bufs
    return [
        lambda: ddt.masked_attention(s.dq, s.dk, s.dv, s.d_base, s.d_prefix, s.d_nq, None,
                                     max_kv_len=ctx + L, out=s.d_out, workspace=ws["d"]),
        lambda: ddt.topk_logprobs(s.logits, cfg.K, 1.0, ids=s.ids, logp=s.logp, lse=s.lse,
                                  workspace=ws["topk"]),
        lambda: ddt.build_tree(s.logp, s.ids, s.root, 1, L, cfg.k_tree, B, out=s.tree),
        lambda: ddt.masked_attention(s.vq, s.vk, s.vv, s.kv_base, s.prefix, s.tree["n_nodes"],
                                     s.tree["mask"], max_kv_len=P + N, out=s.v_out,
                                     workspace=ws["v"]),
        lambda: ddt.accept_compact(s.tree["token"], s.tree["parent"], s.tree["n_nodes"],
                                   s.target, L, s.vk[None], s.vv[None], s.kv_base, s.prefix,
                                   out=s.acc),
    ]


def test_step_graph_replays_match_eager(gpu):
    cfg = synth.CONFIGS[3]
    L, N, ctx, P = cfg.L, cfg.B + 1, cfg.drafter_ctx, cfg.prefix[0]
    cases = [synth.make_case(cfg, seed=90 + i) for i in range(3)]
    bufs = _Buffers(gpu, cfg, cases[0])
    d_desc = ddt.attn_desc(1, cfg.hq, cfg.hkv, cfg.D, L, ctx + L)
    v_desc = ddt.attn_desc(1, cfg.hq, cfg.hkv, cfg.D, N, P + N, (N + 63) // 64)
    ws = {"d": torch.empty(max(1, ddt.attention_workspace_size(d_desc)), dtype=torch.uint8,
                           device=gpu),
          "v": torch.empty(max(1, ddt.attention_workspace_size(v_desc)), dtype=torch.uint8,
                           device=gpu),
          "topk": torch.empty(ddt.topk_workspace_size(L, cfg.vocab, cfg.K), dtype=torch.uint8,
                              device=gpu)}
    calls = _step_calls(cfg, bufs, ws)

    # eager reference per input set.  The target accepts the set's deepest
    # tree path (a sampled target token at this vocabulary size almost never
    # lands in the tree, and compaction would then move nothing).
    eager, targets = [], []
    for c in cases:
        bufs.load(c, np.zeros((1, N), np.int32))
        for f in calls[:3]:
            f()
        torch.cuda.synchronize()
        t = bufs.tree
        tok, par, dep = (t["token"].cpu().numpy()[0], t["parent"].cpu().numpy()[0],
                         t["depth"].cpu().numpy()[0])
        n = int(t["n_nodes"].item())
        deepest = int(np.argmax(dep[:n]))
        tgt = synth.force_path_target(tok, par, dep, n, deepest, c.off_path[0],
                                      cfg.vocab)[None].astype(np.int32)
        targets.append(tgt)
        bufs.load(c, tgt)
        for f in calls:
            f()
        torch.cuda.synchronize()
        eager.append(bufs.snapshot())
    assert all(int(e["acc_accept_len"][0]) > 0 for e in eager)   # compaction is exercised

    # capture once (after a warm-up on a side stream), replay per set, twice over
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for f in calls:
            f()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for f in calls:
            f()
    for rnd in range(2):
        for i, c in enumerate(cases):
            bufs.load(c, targets[i])
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            got = bufs.snapshot()
            for k, v in eager[i].items():
                assert np.array_equal(got[k], v), (rnd, i, k)
