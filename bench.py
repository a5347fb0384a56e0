"""Benchmark: draft-tree steps/s of the DFlash + DDTree kernel chain on one GPU.

One step = one pass of the whole chain over one batch of synthetic input:
  1. drafter-mode attention  (16 block queries over 2048 context + 16 own
     rows, 32 q-heads / 8 KV heads, head_dim 128, bf16)
  2. log-softmax + top-32    (16 positions x 151936 vocab, fp32)
  3. tree build              (budget 256, 32 ranks per position)
  4. verify-mode attention   (257 tree rows over 2048 prefix rows + own
     rows under the ancestor mask, 32/8/128, bf16)
  5. acceptance walk + KV compaction (1 layer)
Inputs: R seeded synthetic sets (the workload's shapes and distributions),
rotated so that the timed steps read cold HBM rather than the 256 MB
last-level cache.  All inputs are resident in device memory before timing.

Prints ONE JSON line.  The step rate comes from replaying one HIP graph per
input set (every stage of a step in one graph).  Per-stage device times come
from a second timed region: one graph per stage holding that stage for every
input set, replayed between HIP events recorded on the launch stream.  A third
region times the same steps with plain launches (no graph).  Side legs time
the compaction of a 36-layer cache, the tree RoPE/scatter step, packed drafter
blocks, the ragged serving-batch verify pass and the large logit streams.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s
METRIC = "draft-tree steps/s at L=16,B=256,ctx 2048; logit GB/s + attn % MFMA peak"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--sets", type=int, default=20, help="rotated input sets (>= 512 MB total)")
    ap.add_argument("--seed", type=int, default=3)
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="time budget of the oracle CPU baseline (0 disables it)")
    ap.add_argument("--graph-sets", type=int, default=20,
                    help="consecutive steps (one per input set) captured in one HIP graph")
    ap.add_argument("--eager", action="store_true",
                    help="launch every stage from Python instead of replaying one HIP graph "
                         "per input set")
    ap.add_argument("--quiet", action="store_true")
    ap.add_argument("--no-streams", action="store_true",
                    help="skip the extra logit-stream measurements (target argmax over the "
                         "verify logits, the 512-row top-K pass, the fused LM head)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run device-to-device copies of MIB MiB (a plain copy kernel of "
                         "known size, to scale HBM byte counters) and exit")
    return ap.parse_args()


def calibrate_copy(mib: int) -> None:
    import torch
    n = mib * 1024 * 1024 // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_mib": mib, "launches": 5, "bytes_read_per_launch": n * 4,
                      "bytes_written_per_launch": n * 4}))


def time_graph(torch, fns, reps):
    """Average device time of one call: a HIP graph holds every call of fns
    back to back and is replayed reps times between HIP events recorded on
    the launch stream."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for f in fns:
            f()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for f in fns:
            f()
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(reps):
        g.replay()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e-3 / (reps * len(fns))


def stream_passes(args, torch, ddt, synth, dev):
    """HBM-bound logit passes beside the step: the target's greedy tokens over
    the verify logits (257 tree slots x 151936, ddt_argmax), the 512-row
    top-16 pass of the serving batch, and the fused LM head -> top-32 of the
    16 drafter rows (ddt_lmhead_topk, a 151936 x 4096 bf16 head).  Cold: the calls rotate over input sets
    larger together than the 256 MB last-level cache; warm: one set again."""
    out = {}
    V = synth.QWEN3_VOCAB
    n_slots = synth.CONFIGS[3].B + 1
    log(args, "target argmax: generating 4 x 257-row verify logit sets")
    sets = [torch.from_numpy(synth.make_verify_logits(args.seed + 77 + i, n_slots)[0]).to(dev)
            for i in range(4)]
    ids = torch.empty(n_slots, dtype=torch.int32, device=dev)
    ws = torch.empty(max(1, ddt.argmax_workspace_size(n_slots, V)), dtype=torch.uint8,
                     device=dev)
    nbytes = n_slots * V * 4 + n_slots * 4
    for mode, bufs in (("cold", sets), ("warm", [sets[0]] * 4)):
        t = time_graph(torch, [lambda b=b: ddt.argmax(b, ids=ids, workspace=ws) for b in bufs],
                       50)
        out[mode] = t
    out = {
        "rows": n_slots, "vocab": V, "algorithmic_bytes": nbytes,
        "bound": "hbm", "peak": HBM_PEAK_GBS, "unit": "GB/s",
        "achieved": round(nbytes / out["cold"] / 1e9, 1),
        "frac": round(nbytes / out["cold"] / 1e9 / HBM_PEAK_GBS, 4),
        "us_cold": round(out["cold"] * 1e6, 3), "us_warm": round(out["warm"] * 1e6, 3),
        "achieved_warm": round(nbytes / out["warm"] / 1e9, 1),
    }
    del sets
    c5 = synth.CONFIGS[5]
    rows, K = c5.batch * c5.L, c5.K
    log(args, f"top-{K} pass: generating 2 x {rows}-row logit sets")
    big = []
    for i in range(2):
        z, _ = synth.make_logits(np.random.Generator(np.random.PCG64(args.seed + 99 + i)), c5)
        big.append(torch.from_numpy(z).to(dev))
    tids = torch.empty(rows, K, dtype=torch.int32, device=dev)
    tlogp = torch.empty(rows, K, dtype=torch.float32, device=dev)
    tws = torch.empty(ddt.topk_workspace_size(rows, V, K), dtype=torch.uint8, device=dev)
    tb = rows * V * 4 + rows * K * 8
    t = time_graph(torch, [lambda b=b: ddt.topk_logprobs(b, K, 1.0, ids=tids, logp=tlogp,
                                                        want_lse=False, workspace=tws)
                           for b in big * 2], 25)
    del big
    c5out = {"rows": rows, "vocab": V, "K": K, "algorithmic_bytes": tb, "bound": "hbm",
             "peak": HBM_PEAK_GBS, "unit": "GB/s", "us_cold": round(t * 1e6, 3),
             "achieved": round(tb / t / 1e9, 1), "frac": round(tb / t / 1e9 / HBM_PEAK_GBS, 4)}
    # fused shared LM head -> top-32 for the 16 drafter rows (hidden 4096):
    # the bf16 head is streamed once per call; two heads rotate (2.5 GB)
    c3 = synth.CONFIGS[3]
    L, hidden, K3 = c3.L, 4096, c3.K
    log(args, "LM head: generating 2 x 151936 x 4096 bf16 heads on the device")
    gen = torch.Generator(device=dev)
    gen.manual_seed(args.seed + 123)
    hs = torch.randn(L, hidden, device=dev, generator=gen).to(torch.bfloat16)
    heads = [(torch.randn(V, hidden, device=dev, generator=gen) * (2.0 / 64.0)).to(torch.bfloat16)
             for _ in range(2)]
    lids = torch.empty(L, K3, dtype=torch.int32, device=dev)
    llogp = torch.empty(L, K3, dtype=torch.float32, device=dev)
    lws = torch.empty(ddt.lmhead_topk_workspace_size(L, hidden, V, K3), dtype=torch.uint8,
                      device=dev)
    t = time_graph(torch, [lambda w=w: ddt.lmhead_topk(hs, w, K3, ids=lids, logp=llogp,
                                                       want_lse=False, workspace=lws)
                           for w in heads * 2], 10)
    del heads
    lb = V * hidden * 2 + L * hidden * 2 + L * K3 * 8
    lmout = {"rows": L, "hidden": hidden, "vocab": V, "K": K3, "algorithmic_bytes": lb,
             "bound": "hbm", "peak": HBM_PEAK_GBS, "unit": "GB/s", "us_cold": round(t * 1e6, 3),
             "achieved": round(lb / t / 1e9, 1), "frac": round(lb / t / 1e9 / HBM_PEAK_GBS, 4)}
    return out, c5out, lmout


def tree_rope_leg(torch, ddt, steps, cfg, dev):
    """Tree positions + rotary embedding + tree K/V scatter (the step between
    the tree build and verify attention) on each input set's own tree: q, k
    and v of the verify rows, written to a separate cache, 20 sets per graph."""
    P, N = cfg.prefix[0], cfg.B + 1
    calls = []
    for s in steps:
        q = s.vq.clone()
        kn = s.vk[P:P + N].clone().view(1, N, cfg.hkv, cfg.D)
        vn = s.vv[P:P + N].clone().view(1, N, cfg.hkv, cfg.D)
        kc = torch.zeros(P + N, cfg.hkv, cfg.D, dtype=torch.bfloat16, device=dev)
        vc = torch.zeros_like(kc)
        pos = torch.empty(1, N, dtype=torch.int32, device=dev)
        calls.append(lambda s=s, q=q, kn=kn, vn=vn, kc=kc, vc=vc, pos=pos: ddt.tree_rope_kv(
            s.tree["depth"], s.tree["n_nodes"], s.prefix, s.kv_base, q, kn, vn, kc, vc, 1.0e6,
            positions=pos))
    t = time_graph(torch, calls, 50)
    nb = (N * cfg.hq * cfg.D * 2 * 2 + 2 * N * cfg.hkv * cfg.D * 2 * 2 + N * 4 * 2)
    return {"rows": N, "hq": cfg.hq, "hkv": cfg.hkv, "D": cfg.D, "algorithmic_bytes": nb,
            "bound": "hbm", "peak": HBM_PEAK_GBS, "unit": "GB/s", "us": round(t * 1e6, 3),
            "achieved": round(nb / t / 1e9, 1), "frac": round(nb / t / 1e9 / HBM_PEAK_GBS, 4)}


def packed_blocks_leg(torch, ddt, steps, cfg, dev):
    """Packed drafter blocks: 4 blocks of 16 query rows over the 2048-row
    context plus their own rows (block-diagonal), drafter head shape 32/8/128,
    from each set's verify tensors (the first 64 query rows and cache rows);
    20 calls per graph."""
    P, nb, L = cfg.drafter_ctx, 4, cfg.L
    n = nb * L
    desc = ddt.attn_desc(1, cfg.hq, cfg.hkv, cfg.D, n, P + n)
    ws = torch.empty(max(1, ddt.attention_workspace_size(desc)), dtype=torch.uint8, device=dev)
    base = torch.zeros(1, dtype=torch.int64, device=dev)
    pre = torch.full((1,), P, dtype=torch.int32, device=dev)
    nq = torch.full((1,), n, dtype=torch.int32, device=dev)
    calls = []
    for s in steps:
        q = s.vq[:, :n].contiguous()
        out = torch.empty_like(q)
        calls.append(lambda s=s, q=q, out=out: ddt.masked_attention(
            q, s.vk, s.vv, base, pre, nq, None, max_kv_len=P + n, out=out, workspace=ws,
            block_len=L))
    t = time_graph(torch, calls, 50)
    nb_bytes = (P + n) * cfg.hkv * cfg.D * 2 * 2 + 2 * n * cfg.hq * cfg.D * 2
    return {"blocks": nb, "block_len": L, "context": P, "algorithmic_bytes": nb_bytes,
            "bound": "hbm", "peak": HBM_PEAK_GBS, "unit": "GB/s", "us": round(t * 1e6, 3),
            "achieved": round(nb_bytes / t / 1e9, 1),
            "frac": round(nb_bytes / t / 1e9 / HBM_PEAK_GBS, 4)}


def accept_layers_leg(torch, ddt, synth, steps, cases, cfg, dev, n_layers=36):
    """Acceptance walk + KV compaction over a 36-layer cache (the target
    model's depth; the step itself compacts one layer) on each input set's own
    tree, 20 calls per graph, one workgroup per layer.  The target accepts the
    tree's deepest path (the most rows a tree can move), not the sampled path
    of the step."""
    P, N, L = cfg.prefix[0], cfg.B + 1, cfg.L
    kc = torch.zeros(n_layers, P + N, cfg.hkv, cfg.D, dtype=torch.bfloat16, device=dev)
    vc = torch.zeros_like(kc)
    base = torch.zeros(1, dtype=torch.int64, device=dev)
    calls, outs = [], []
    for s, c in zip(steps, cases):
        tok = s.tree["token"].cpu().numpy()[0]
        par = s.tree["parent"].cpu().numpy()[0]
        dep = s.tree["depth"].cpu().numpy()[0]
        n = int(s.tree["n_nodes"].item())
        deepest = int(np.argmax(dep[:n]))
        tgt = torch.from_numpy(synth.force_path_target(
            tok, par, dep, n, deepest, c.off_path[0], cfg.vocab)[None]).to(dev)
        out = {k: torch.empty_like(v) for k, v in s.acc.items()}
        outs.append(out)
        calls.append(lambda s=s, out=out, tgt=tgt: ddt.accept_compact(
            s.tree["token"], s.tree["parent"], s.tree["n_nodes"], tgt, L, kc, vc, base,
            s.prefix, out=out))
    t = time_graph(torch, calls, 50)
    acc = float(np.mean([int(o["accept_len"].item()) for o in outs]))
    nb = n_layers * acc * cfg.hkv * cfg.D * 2 * 2 * 2   # K and V rows, read + written
    return {"layers": n_layers, "mean_accept_len": round(acc, 3), "algorithmic_bytes": nb,
            "bound": "latency", "us": round(t * 1e6, 3),
            "achieved_gbs": round(nb / t / 1e9, 1)}


def serving_verify_leg(args, torch, ddt, synth, dev):
    """Verify attention of the ragged serving batch: 32 requests, 65 tree rows
    each, prefixes U{512..8192}, 32/4/128.  The trees come from this library's
    own top-K and tree kernels on the batch's synthetic logits; FLOPs count
    the keys each tree row can see."""
    c5 = synth.CONFIGS[5]
    N = c5.B + 1
    sets = []
    for i in range(2):
        case = synth.make_case(c5, seed=args.seed + 500 + i, with_drafter=False)
        lg = torch.from_numpy(case.logits).to(dev)
        ids, logp, _ = ddt.topk_logprobs(lg, c5.K)
        tree = ddt.build_tree(logp, ids, torch.from_numpy(case.root_token).to(dev), c5.batch,
                              c5.L, c5.k_tree, c5.B)
        torch.cuda.synchronize()
        depth = tree["depth"].cpu().numpy()
        nn = tree["n_nodes"].cpu().numpy()
        vis = sum(int(nn[r]) * int(case.prefix_len[r]) + int((depth[r, :nn[r]] + 1).sum())
                  for r in range(c5.batch))

        def bf16(bits):
            return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(
                torch.bfloat16)
        sets.append(dict(q=bf16(case.vq_bits), k=bf16(case.vk_bits), v=bf16(case.vv_bits),
                         base=torch.from_numpy(case.kv_base).to(dev),
                         pre=torch.from_numpy(case.prefix_len).to(dev), nq=tree["n_nodes"],
                         mask=tree["mask"], maxkv=int(case.prefix_len.max()) + N,
                         flops=4.0 * c5.D * c5.hq * vis))
        del lg
    maxkv = max(st["maxkv"] for st in sets)
    desc = ddt.attn_desc(c5.batch, c5.hq, c5.hkv, c5.D, N, maxkv, (N + 63) // 64)
    ws = torch.empty(max(1, ddt.attention_workspace_size(desc)), dtype=torch.uint8, device=dev)
    outs = [torch.empty_like(st["q"]) for st in sets]
    t = time_graph(torch, [lambda st=st, o=o: ddt.masked_attention(
        st["q"], st["k"], st["v"], st["base"], st["pre"], st["nq"], st["mask"],
        max_kv_len=maxkv, out=o, workspace=ws) for st, o in zip(sets, outs)] * 2, 10)
    fl = float(np.mean([st["flops"] for st in sets]))
    return {"requests": c5.batch, "rows_per_request": N, "prefix": "U{512..8192}",
            "hq": c5.hq, "hkv": c5.hkv, "D": c5.D, "algorithmic_flops": fl, "bound": "mfma",
            "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "us": round(t * 1e6, 2),
            "achieved": round(fl / t / 1e12, 1), "frac": round(fl / t / 1e12 / BF16_PEAK_TFLOPS, 4)}


def log(args, msg):
    if not args.quiet:
        print(msg, file=sys.stderr, flush=True)


class Step:
    """Device buffers for one input set plus the preallocated outputs."""

    def __init__(self, case, dev, torch, ddt):
        cfg = case.cfg
        self.cfg = cfg
        L, N, ctx = cfg.L, cfg.B + 1, cfg.drafter_ctx

        def bf16(bits):
            return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(
                torch.bfloat16)

        self.logits = torch.from_numpy(case.logits).to(dev)
        self.root = torch.from_numpy(case.root_token).to(dev)
        self.dq, self.dk, self.dv = bf16(case.dq_bits), bf16(case.dk_bits), bf16(case.dv_bits)
        self.d_base = torch.zeros(1, dtype=torch.int64, device=dev)
        self.d_prefix = torch.full((1,), ctx, dtype=torch.int32, device=dev)
        self.d_nq = torch.full((1,), L, dtype=torch.int32, device=dev)
        self.vq, self.vk, self.vv = bf16(case.vq_bits), bf16(case.vk_bits), bf16(case.vv_bits)
        self.kv_base = torch.from_numpy(case.kv_base).to(dev)
        self.prefix = torch.from_numpy(case.prefix_len).to(dev)
        self.kc = self.vk[None]          # one layer, compacted in place
        self.vc = self.vv[None]
        self.d_out = torch.empty_like(self.dq)
        self.v_out = torch.empty_like(self.vq)
        self.ids = torch.empty(L, cfg.K, dtype=torch.int32, device=dev)
        self.logp = torch.empty(L, cfg.K, dtype=torch.float32, device=dev)
        self.lse = torch.empty(L, dtype=torch.float32, device=dev)
        W = (N + 63) // 64
        self.tree = {
            "n_nodes": torch.empty(1, dtype=torch.int32, device=dev),
            "token": torch.empty(1, N, dtype=torch.int32, device=dev),
            "parent": torch.empty(1, N, dtype=torch.int32, device=dev),
            "depth": torch.empty(1, N, dtype=torch.int32, device=dev),
            "score": torch.empty(1, N, dtype=torch.float32, device=dev),
            "mask": torch.empty(1, N, W, dtype=torch.int64, device=dev),
        }
        self.acc = {
            "accept_len": torch.empty(1, dtype=torch.int32, device=dev),
            "accepted": torch.empty(1, L + 1, dtype=torch.int32, device=dev),
            "bonus": torch.empty(1, dtype=torch.int32, device=dev),
            "new_len": torch.empty(1, dtype=torch.int32, device=dev),
        }
        self.target = None


def main():
    args = parse()
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the chain's "
              "multi-GPU sharding is a design note, not a runnable path.", file=sys.stderr)
        sys.exit(2)

    import torch

    import synth
    from block_diffusion_draft_vocab_amd import ddt

    ddt.load()
    dev = torch.device("cuda:0")
    cfg = synth.CONFIGS[3]
    L, N, K, B = cfg.L, cfg.B + 1, cfg.K, cfg.B
    ctx, P = cfg.drafter_ctx, cfg.prefix[0]
    log(args, f"generating {args.sets} input sets")
    cases = [synth.make_case(cfg, seed=args.seed + 1000 * i) for i in range(args.sets)]
    steps = [Step(c, dev, torch, ddt) for c in cases]

    d_desc = ddt.attn_desc(1, cfg.hq, cfg.hkv, cfg.D, L, ctx + L)
    v_desc = ddt.attn_desc(1, cfg.hq, cfg.hkv, cfg.D, N, P + N, (N + 63) // 64)
    ws_attn_d = torch.empty(max(1, ddt.attention_workspace_size(d_desc)), dtype=torch.uint8,
                            device=dev)
    ws_attn_v = torch.empty(max(1, ddt.attention_workspace_size(v_desc)), dtype=torch.uint8,
                            device=dev)
    ws_topk = torch.empty(ddt.topk_workspace_size(L, cfg.vocab, K), dtype=torch.uint8,
                          device=dev)

    def stage_calls(s: Step):
        return [
            lambda: ddt.masked_attention(s.dq, s.dk, s.dv, s.d_base, s.d_prefix, s.d_nq, None,
                                         max_kv_len=ctx + L, out=s.d_out, workspace=ws_attn_d),
            lambda: ddt.topk_logprobs(s.logits, K, 1.0, ids=s.ids, logp=s.logp, lse=s.lse,
                                      workspace=ws_topk),
            lambda: ddt.build_tree(s.logp, s.ids, s.root, 1, L, cfg.k_tree, B, out=s.tree),
            lambda: ddt.masked_attention(s.vq, s.vk, s.vv, s.kv_base, s.prefix,
                                         s.tree["n_nodes"], s.tree["mask"], max_kv_len=P + N,
                                         out=s.v_out, workspace=ws_attn_v),
            lambda: ddt.accept_compact(s.tree["token"], s.tree["parent"], s.tree["n_nodes"],
                                       s.target, L, s.kc, s.vc, s.kv_base, s.prefix,
                                       out=s.acc),
        ]

    # synthetic target "argmax" per set, along the tree this chain builds
    depths = []
    for s, c in zip(steps, cases):
        for f in stage_calls(s)[:3]:
            f()
        torch.cuda.synchronize()
        tok = s.tree["token"].cpu().numpy()[0]
        par = s.tree["parent"].cpu().numpy()[0]
        dep = s.tree["depth"].cpu().numpy()[0]
        n = int(s.tree["n_nodes"].item())
        y = synth.sample_target_path(c)[0]
        s.target = torch.from_numpy(
            synth.target_for_tree(tok, par, dep, n, y, c.off_path[0])[None]).to(dev)
        depths.append(dep[:n].astype(np.int64))
    calls = [stage_calls(s) for s in steps]
    names = ["drafter_attn", "topk", "tree", "verify_attn", "accept"]

    stream = torch.cuda.current_stream()
    G = 1
    if args.eager:
        log(args, f"warmup {args.warmup}")
        for i in range(args.warmup):
            for f in calls[i % len(calls)]:
                f()
        torch.cuda.synchronize()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
              for _ in range(args.steps)]
        log(args, f"timing {args.steps} eager steps")
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            e = ev[i]
            e[0].record(stream)
            for j, f in enumerate(calls[i % len(calls)]):
                f()
                e[j + 1].record(stream)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    else:
        # region A: one HIP graph per input set holds the whole step
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            for c in calls:
                for f in c:
                    f()
        torch.cuda.synchronize()

        def capture(fns):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for f in fns:
                    f()
            return g

        # G consecutive steps (input sets i..i+G-1) per graph; single-step
        # graphs cover a remainder, so exactly --steps steps run
        G = max(1, min(args.graph_sets, len(calls)))
        multi = [capture([f for c in calls[i:i + G] for f in c])
                 for i in range(0, len(calls) - G + 1, G)]
        single = [capture(c) for c in calls]
        log(args, f"warmup {args.warmup}")
        for i in range(args.warmup):
            single[i % len(single)].replay()
        torch.cuda.synchronize()
        log(args, f"timing {args.steps} graph steps, {G} per graph")
        t0 = time.perf_counter()
        for i in range(args.steps // G):
            multi[i % len(multi)].replay()
        for i in range(args.steps % G):
            single[i % len(single)].replay()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        # region B: per-stage device time.  One graph per stage holds that
        # stage for every input set back to back; HIP events on the launch
        # stream bracket each replay (events cannot be timed inside a
        # captured graph here), so a launch's average duration includes the
        # small gap between kernels of one graph.
        stage_graphs = [capture([c[j] for c in calls]) for j in range(len(names))]
        reps = max(1, min(args.steps, 1000) // len(calls))
        ev = []
        for j, g in enumerate(stage_graphs):
            for _ in range(3):
                g.replay()
            torch.cuda.synchronize()
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(reps):
                g.replay()
            b.record(stream)
            ev.append((a, b))
        torch.cuda.synchronize()
        log(args, f"timed {reps} replays of {len(calls)} launches per stage")
        # region C: the same step with plain launches (one ctypes call per
        # stage from Python, no graph), for comparison with region A
        n_eager = min(args.steps, 500)
        for i in range(5):
            for f in calls[i % len(calls)]:
                f()
        torch.cuda.synchronize()
        te0 = time.perf_counter()
        for i in range(n_eager):
            for f in calls[i % len(calls)]:
                f()
        torch.cuda.synchronize()
        eager_ms = (time.perf_counter() - te0) * 1e3 / n_eager
        log(args, f"timed {n_eager} plain-launch steps")
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    stage_ms = np.zeros(len(names))
    if args.eager:
        for e in ev:
            for j in range(len(names)):
                stage_ms[j] += e[j].elapsed_time(e[j + 1])
        stage_ms /= len(ev)
    else:
        for j, (a, b) in enumerate(ev):
            stage_ms[j] = a.elapsed_time(b) / (reps * len(calls))
    steps_per_s = 1e3 / ms_per_step

    # algorithmic work
    logit_bytes = L * cfg.vocab * 4 + L * K * 8 + L * 4
    flops = []
    for dep in depths:
        vis = P + (dep + 1)                       # prefix + ancestors incl. self
        flops.append(4.0 * cfg.D * cfg.hq * float(vis.sum()))
    verify_flops = float(np.mean(flops))
    drafter_bytes = ((ctx + L) * cfg.hkv * cfg.D * 2 * 2) + 2 * (L * cfg.hq * cfg.D * 2)
    t_logit = stage_ms[1] * 1e-3
    t_verify = stage_ms[3] * 1e-3
    t_draft = stage_ms[0] * 1e-3
    logit_gbs = logit_bytes / t_logit / 1e9
    verify_tflops = verify_flops / t_verify / 1e12

    # HBM bytes and MFMA counters of the verify launch, from the rocprofv3
    # counter passes summarised under profiles/ (only while attention.hip
    # is the source they were taken from)
    traffic = issued_mfma = mfma_busy = None
    tfile = os.path.join(ROOT, "profiles", "verify_attn_traffic.json")
    if os.path.exists(tfile):
        with open(tfile) as f:
            tr = json.load(f)
        src = os.path.join(ROOT, "block_diffusion_draft_vocab_amd", "csrc", "attention.hip")
        sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
        if tr.get("source_sha256") == sha:
            traffic = tr.get("hbm_bytes_per_launch")
            issued_mfma = tr.get("issued_mfma_bf16_flops_per_launch")
            mfma_busy = tr.get("mfma_busy_pct_main_kernel")

    # HBM bytes per launch of the logit pass and the drafter pass, likewise
    stage_traffic = {}
    sfile = os.path.join(ROOT, "profiles", "step_stage_traffic.json")
    if os.path.exists(sfile):
        with open(sfile) as f:
            for name, tr in json.load(f).items():
                src = os.path.join(ROOT, tr["source"])
                if hashlib.sha256(open(src, "rb").read()).hexdigest() == tr.get("source_sha256"):
                    stage_traffic[name] = tr.get("hbm_bytes_per_launch")

    result = {
        "metric": METRIC,
        "value": round(steps_per_s, 2),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "launch": "eager" if args.eager else f"hip_graph ({G} steps per graph)",
        "config": {
            "workload": "ddtree_step_c3: L=16 V=151936 K=32 B=256 k_tree=32; drafter 16q over "
                        "2048+16 rows; verify 257q over 2048+257 rows; hq=32 hkv=8 D=128; "
                        "1 layer compaction",
            "batch": 1, "input_sets": args.sets,
        },
        "roofline": {
            "bound": "mfma",
            "kernel": "verify attention (attn_kernel<128,split> + attn_combine_kernel<128>)",
            "achieved": round(verify_tflops, 3),
            "peak": BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(verify_tflops / BF16_PEAK_TFLOPS, 5),
            "traffic": traffic,
            "algorithmic_flops_per_launch": verify_flops,
            "issued_mfma_flops_per_launch": issued_mfma,
            "mfma_busy_pct_main_kernel": mfma_busy,
        },
        "stages_us": {n: round(float(m) * 1e3, 3) for n, m in zip(names, stage_ms)},
        "logit_pass": {
            "bound": "hbm", "achieved": round(logit_gbs, 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(logit_gbs / HBM_PEAK_GBS, 4),
            "algorithmic_bytes": logit_bytes, "traffic": stage_traffic.get("logit_pass"),
        },
        "drafter_attn": {
            "bound": "hbm", "achieved": round(drafter_bytes / t_draft / 1e9, 1),
            "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(drafter_bytes / t_draft / 1e9 / HBM_PEAK_GBS, 4),
            "algorithmic_bytes": drafter_bytes, "traffic": stage_traffic.get("drafter_attn"),
        },
    }

    if not args.eager:
        result["plain_launches"] = {"steps": n_eager, "ms_per_step": round(eager_ms, 5),
                                    "steps_per_s": round(1e3 / eager_ms, 2)}
    result["accept_36_layers"] = accept_layers_leg(torch, ddt, synth, steps, cases, cfg, dev)
    result["tree_rope_kv"] = tree_rope_leg(torch, ddt, steps, cfg, dev)
    result["packed_blocks_attn"] = packed_blocks_leg(torch, ddt, steps, cfg, dev)
    if not args.no_streams:
        result["verify_attn_serving"] = serving_verify_leg(args, torch, ddt, synth, dev)
    if not args.no_streams:
        (result["target_argmax"], result["logit_pass_512rows"],
         result["lmhead_topk"]) = stream_passes(args, torch, ddt, synth, dev)
    if args.cpu_seconds > 0:
        result["cpu_baseline"] = cpu_baseline(cases[0], args.cpu_seconds, args)
    print(json.dumps(result), flush=True)


def cpu_baseline(case, budget_s, args):
    """The oracle, as it stands, running the same chain step on the host."""
    import synth
    from oracle.accept import accept_compact
    from oracle.attention import masked_attention
    from oracle.logits import topk_logprobs
    from oracle.tree import build_trees
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:
        cores = 1
    cfg = case.cfg
    L, N, ctx = cfg.L, cfg.B + 1, cfg.drafter_ctx
    dq = synth.bf16_bits_to_f32(case.dq_bits)
    dk = synth.bf16_bits_to_f32(case.dk_bits)
    dv = synth.bf16_bits_to_f32(case.dv_bits)
    vq = synth.bf16_bits_to_f32(case.vq_bits)
    vk = synth.bf16_bits_to_f32(case.vk_bits)
    vv = synth.bf16_bits_to_f32(case.vv_bits)
    y = synth.sample_target_path(case)
    n_steps = 0
    t0 = time.perf_counter()
    while True:
        masked_attention(dq, dk, dv, [0], [ctx], [L], None)
        ids, logp, _ = topk_logprobs(case.logits, cfg.K)
        t = build_trees(logp, ids, case.root_token, 1, L, cfg.k_tree, cfg.B)
        masked_attention(vq, vk, vv, case.kv_base, case.prefix_len, t["n_nodes"], t["mask"])
        tgt = synth.target_for_tree(t["token"][0], t["parent"][0], t["depth"][0],
                                    int(t["n_nodes"][0]), y[0], case.off_path[0])[None]
        accept_compact(t["token"], t["parent"], t["n_nodes"], tgt, L, case.vk_bits[None],
                       case.vv_bits[None], case.kv_base, case.prefix_len)
        n_steps += 1
        el = time.perf_counter() - t0
        log(args, f"cpu baseline step {n_steps}: {el:.1f}s")
        if el >= budget_s:
            break
    return {"value": round(n_steps / el, 4), "unit": "steps/s", "cores": int(cores),
            "kind": "oracle",
            "sample": f"{n_steps} full oracle chain steps on input set 0 ({el:.1f} s of host "
                      f"time; float64 numpy, BLAS threads={cores})"}


if __name__ == "__main__":
    main()
