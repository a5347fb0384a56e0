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
    ap.add_argument("--stage-replays", type=int, default=50,
                    help="replays of each per-stage graph (and of the step graph) timed one "
                         "by one for the per-stage times and their spread")
    ap.add_argument("--no-workloads", action="store_true",
                    help="skip the budget-1024 and serving-batch chain steps")
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


def time_graph(torch, fns, reps, min_calls=20):
    """Average device time of one call: a HIP graph holds the calls of fns
    back to back, repeated until it holds at least min_calls calls (so the
    graph's own launch cost is spread thin), and is replayed reps times
    between HIP events recorded on the launch stream."""
    fns = list(fns) * max(1, -(-min_calls // len(fns)))
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


def replay_times(torch, g, reps):
    """Device time of each of reps replays of graph g (ms): HIP events on the
    launch stream between consecutive replays."""
    stream = torch.cuda.current_stream()
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    ev[0].record(stream)
    for i in range(reps):
        g.replay()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    return np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(reps)])


def capture(torch, fns):
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for f in fns:
            f()
    return g


def warm_on_side_stream(torch, fns):
    """Run fns once on a side stream (allocator warm-up before capture)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for f in fns:
            f()
    torch.cuda.synchronize()


def spread(per_launch_ms):
    """(mean, median, min) in microseconds."""
    a = np.asarray(per_launch_ms) * 1e3
    return float(a.mean()), float(np.median(a)), float(a.min())


class Chain:
    """Device buffers and the stage calls of one input set of a workload:
    drafter attention (when the workload has a drafter pass), top-K, tree,
    verify attention, acceptance + compaction of one layer.  Workspaces are
    shared by all sets of the workload (ws dict)."""

    NAMES = ["drafter_attn", "topk", "tree", "verify_attn", "accept"]

    def __init__(self, case, dev, torch, ddt, ws, max_kv):
        cfg = case.cfg
        self.cfg, self.case, self.ddt, self.ws, self.max_kv = cfg, case, ddt, ws, max_kv
        b, L, N, ctx = cfg.batch, cfg.L, cfg.B + 1, cfg.drafter_ctx

        def bf16(bits):
            return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(
                torch.bfloat16)

        self.logits = torch.from_numpy(case.logits).to(dev)
        self.root = torch.from_numpy(case.root_token).to(dev)
        self.has_drafter = ctx > 0 and case.dq_bits is not None
        if self.has_drafter:
            self.dq, self.dk, self.dv = (bf16(case.dq_bits), bf16(case.dk_bits),
                                         bf16(case.dv_bits))
            self.d_base = torch.arange(b, dtype=torch.int64, device=dev) * (ctx + L)
            self.d_prefix = torch.full((b,), ctx, dtype=torch.int32, device=dev)
            self.d_nq = torch.full((b,), L, dtype=torch.int32, device=dev)
            self.d_out = torch.empty_like(self.dq)
        self.vq, self.vk, self.vv = bf16(case.vq_bits), bf16(case.vk_bits), bf16(case.vv_bits)
        self.kv_base = torch.from_numpy(case.kv_base).to(dev)
        self.prefix = torch.from_numpy(case.prefix_len).to(dev)
        self.kc = self.vk[None]          # one layer, compacted in place
        self.vc = self.vv[None]
        self.v_out = torch.empty_like(self.vq)
        self.ids = torch.empty(b * L, cfg.K, dtype=torch.int32, device=dev)
        self.logp = torch.empty(b * L, cfg.K, dtype=torch.float32, device=dev)
        self.lse = torch.empty(b * L, dtype=torch.float32, device=dev)
        W = (N + 63) // 64
        self.tree = {
            "n_nodes": torch.empty(b, dtype=torch.int32, device=dev),
            "token": torch.empty(b, N, dtype=torch.int32, device=dev),
            "parent": torch.empty(b, N, dtype=torch.int32, device=dev),
            "depth": torch.empty(b, N, dtype=torch.int32, device=dev),
            "score": torch.empty(b, N, dtype=torch.float32, device=dev),
            "mask": torch.empty(b, N, W, dtype=torch.int64, device=dev),
        }
        self.acc = {
            "accept_len": torch.empty(b, dtype=torch.int32, device=dev),
            "accepted": torch.empty(b, L + 1, dtype=torch.int32, device=dev),
            "bonus": torch.empty(b, dtype=torch.int32, device=dev),
            "new_len": torch.empty(b, dtype=torch.int32, device=dev),
        }
        self.target = None
        self.verify_flops = None

    def stage_calls(self):
        """[(name, fn)] of one step, in chain order."""
        ddt, cfg, ws = self.ddt, self.cfg, self.ws
        L, ctx = cfg.L, cfg.drafter_ctx
        out = []
        if self.has_drafter:
            out.append(("drafter_attn", lambda: ddt.masked_attention(
                self.dq, self.dk, self.dv, self.d_base, self.d_prefix, self.d_nq, None,
                max_kv_len=ctx + L, out=self.d_out, workspace=ws["attn_d"])))
        out += [
            ("topk", lambda: ddt.topk_logprobs(self.logits, cfg.K, cfg.inv_temperature,
                                               ids=self.ids, logp=self.logp, lse=self.lse,
                                               workspace=ws["topk"])),
            ("tree", lambda: ddt.build_tree(self.logp, self.ids, self.root, cfg.batch, L,
                                            cfg.k_tree, cfg.B, out=self.tree)),
            ("verify_attn", lambda: ddt.masked_attention(
                self.vq, self.vk, self.vv, self.kv_base, self.prefix, self.tree["n_nodes"],
                self.tree["mask"], max_kv_len=self.max_kv, out=self.v_out,
                workspace=ws["attn_v"])),
            ("accept", lambda: ddt.accept_compact(
                self.tree["token"], self.tree["parent"], self.tree["n_nodes"], self.target, L,
                self.kc, self.vc, self.kv_base, self.prefix, out=self.acc)),
        ]
        return out

    def prepare(self, torch, synth, dev):
        """Run the stages up to the tree once, then draw the synthetic
        target's greedy tokens along the tree they built (host-side input
        generation, outside every timed region), and count the verify FLOPs
        (keys each tree row can see)."""
        for name, f in self.stage_calls():
            if name in ("drafter_attn", "topk", "tree"):
                f()
        torch.cuda.synchronize()
        cfg, case = self.cfg, self.case
        tok = self.tree["token"].cpu().numpy()
        par = self.tree["parent"].cpu().numpy()
        dep = self.tree["depth"].cpu().numpy()
        nn = self.tree["n_nodes"].cpu().numpy()
        y = synth.sample_target_path(case)
        self.target = torch.from_numpy(np.stack([
            synth.target_for_tree(tok[r], par[r], dep[r], int(nn[r]), y[r], case.off_path[r])
            for r in range(cfg.batch)])).to(dev)
        vis = sum(int(nn[r]) * int(case.prefix_len[r]) + int((dep[r, :nn[r]] + 1).sum())
                  for r in range(cfg.batch))
        self.verify_flops = 4.0 * cfg.D * cfg.hq * vis
        self.depths = [dep[r, :nn[r]].astype(np.int64) for r in range(cfg.batch)]


def chain_workspaces(torch, ddt, cfg, max_kv, dev):
    L, N, ctx, b = cfg.L, cfg.B + 1, cfg.drafter_ctx, cfg.batch
    ws = {}
    if ctx > 0:
        d = ddt.attn_desc(b, cfg.hq, cfg.hkv, cfg.D, L, ctx + L)
        ws["attn_d"] = torch.empty(max(1, ddt.attention_workspace_size(d)), dtype=torch.uint8,
                                   device=dev)
    v = ddt.attn_desc(b, cfg.hq, cfg.hkv, cfg.D, N, max_kv, (N + 63) // 64)
    ws["attn_v"] = torch.empty(max(1, ddt.attention_workspace_size(v)), dtype=torch.uint8,
                               device=dev)
    ws["topk"] = torch.empty(ddt.topk_workspace_size(b * L, cfg.vocab, cfg.K),
                             dtype=torch.uint8, device=dev)
    return ws


def make_chains(args, torch, ddt, synth, cfg, n_sets, seed0, dev):
    cases = [synth.make_case(cfg, seed=seed0 + 1000 * i) for i in range(n_sets)]
    max_kv = max(int(c.prefix_len.max()) for c in cases) + cfg.B + 1
    ws = chain_workspaces(torch, ddt, cfg, max_kv, dev)
    chains = [Chain(c, dev, torch, ddt, ws, max_kv) for c in cases]
    for ch in chains:
        ch.prepare(torch, synth, dev)
    return cases, chains


def time_stages(torch, chains, reps, min_launches=20):
    """Per-stage device time: one graph per stage holds that stage for the
    input sets back to back, cycling through them until the graph holds at
    least min_launches launches (so the graph's own launch cost is spread
    thin), and is replayed reps times, a HIP event between replays.
    Returns {stage: per-launch ms of each replay}."""
    names = [n for n, _ in chains[0].stage_calls()]
    cyc = max(1, -(-min_launches // len(chains)))
    order = [ch for _ in range(cyc) for ch in chains]
    per = {}
    for j, name in enumerate(names):
        g = capture(torch, [ch.stage_calls()[j][1] for ch in order])
        per[name] = replay_times(torch, g, reps) / len(order)
        del g
    return per


def stage_summary(per):
    out = {}
    for name, a in per.items():
        mean, med, mn = spread(a)
        out[name] = {"mean": round(mean, 3), "median": round(med, 3), "min": round(mn, 3)}
    return out


def workload_leg(args, torch, ddt, synth, cfg, n_sets, seed0, dev, label, reps):
    """A whole chain step of one more workload (budget 1024 peaked / flat, the
    32-request serving batch): steps/s from graphs of n_sets steps replayed
    reps times, per-stage times, verify attention and tree against their
    bounds."""
    log(args, f"{label}: generating {n_sets} input sets")
    cases, chains = make_chains(args, torch, ddt, synth, cfg, n_sets, seed0, dev)
    # one graph of at least 8 steps, cycling through the input sets
    cyc = max(1, -(-8 // n_sets))
    fns = [f for _ in range(cyc) for ch in chains for _, f in ch.stage_calls()]
    warm_on_side_stream(torch, fns)
    g = capture(torch, fns)
    step_ms = replay_times(torch, g, reps) / (n_sets * cyc)
    del g
    per = time_stages(torch, chains, reps)
    st = stage_summary(per)
    fl = float(np.mean([ch.verify_flops for ch in chains]))
    tv = st["verify_attn"]["mean"] * 1e-6
    b, L = cfg.batch, cfg.L
    lb = b * L * cfg.vocab * 4 + b * L * cfg.K * 8 + b * L * 4
    tl = st["topk"]["mean"] * 1e-6
    mean, med, mn = spread(step_ms)
    res = {
        "workload": label, "steps_per_s": round(1e3 / (mean * 1e-3), 2),
        "us_per_step": {"mean": round(mean, 3), "median": round(med, 3), "min": round(mn, 3)},
        "replays": reps, "input_sets": n_sets, "stages_us": st,
        "verify_attn": {"bound": "mfma", "algorithmic_flops": fl, "peak": BF16_PEAK_TFLOPS,
                        "unit": "TFLOP/s", "achieved": round(fl / tv / 1e12, 1),
                        "frac": round(fl / tv / 1e12 / BF16_PEAK_TFLOPS, 4)},
        "logit_pass": {"bound": "hbm", "algorithmic_bytes": lb, "peak": HBM_PEAK_GBS,
                       "unit": "GB/s", "achieved": round(lb / tl / 1e9, 1),
                       "frac": round(lb / tl / 1e9 / HBM_PEAK_GBS, 4)},
        "mean_tree_depth_max": round(float(np.mean([max(int(d.max()) for d in ch.depths)
                                                    for ch in chains])), 2),
        "mean_accept_len": None,
    }
    torch.cuda.synchronize()
    res["mean_accept_len"] = round(float(np.mean([ch.acc["accept_len"].float().mean().item()
                                                  for ch in chains])), 3)
    del chains, cases
    torch.cuda.empty_cache()
    return res


def floor_leg(torch, ddt, dev, reps):
    """What one launch costs on this GPU, with this library's simplest kernel
    (ddt_argmax over rows of at most one 8192-float chunk: a single launch,
    one read of the input, no merge): 20 dependent launches of a 1 x 64 row
    in one graph (the per-launch floor of back-to-back kernels), and 20
    launches that each read 9.73 MB, the logit pass's byte count, in two grid
    shapes (297 x 8192 and 1188 x 2048 floats)."""
    out = {}
    tiny = torch.zeros(1, 64, dtype=torch.float32, device=dev)
    ids = torch.empty(1, dtype=torch.int32, device=dev)
    fns = [lambda: ddt.argmax(tiny, ids=ids) for _ in range(20)]
    warm_on_side_stream(torch, fns)
    g = capture(torch, fns)
    out["dependent_launch_us"] = round(spread(replay_times(torch, g, reps) / 20)[0], 3)
    best = None
    for rows, V in ((297, 8192), (1188, 2048)):
        bufs = [torch.randn(rows, V, device=dev) for _ in range(4)]
        oid = torch.empty(rows, dtype=torch.int32, device=dev)
        fns = [lambda b=b: ddt.argmax(b, ids=oid) for b in bufs] * 5
        warm_on_side_stream(torch, fns)
        g = capture(torch, fns)
        t = spread(replay_times(torch, g, reps) / 20)[0]
        out[f"one_launch_read_us_{rows}x{V}"] = round(t, 3)
        best = t if best is None else min(best, t)
        del bufs, g
    out["one_launch_read_us"] = round(best, 3)
    out["read_bytes"] = 297 * 8192 * 4
    return out


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
    cases, chains = make_chains(args, torch, ddt, synth, cfg, args.sets, args.seed, dev)
    calls = [[f for _, f in ch.stage_calls()] for ch in chains]
    names = Chain.NAMES
    stream = torch.cuda.current_stream()
    G = 1
    reps_b = max(args.stage_replays, 1)
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
        per = {n: np.array([e[j].elapsed_time(e[j + 1]) for e in ev])
               for j, n in enumerate(names)}
    else:
        # region A: HIP graphs of G consecutive steps (one per input set);
        # single-step graphs cover a remainder, so exactly --steps steps run
        warm_on_side_stream(torch, [f for c in calls for f in c])
        G = max(1, min(args.graph_sets, len(calls)))
        multi = [capture(torch, [f for c in calls[i:i + G] for f in c])
                 for i in range(0, len(calls) - G + 1, G)]
        single = [capture(torch, c) for c in calls]
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
        # the same graphs replayed reps_b times with an event between
        # replays: the spread of the step time
        step_ms = replay_times(torch, multi[0], reps_b) / G
        del multi, single
        # region B: per-stage device time, each stage's graph replayed
        # reps_b times (independent of --steps)
        per = time_stages(torch, chains, reps_b)
        log(args, f"timed {reps_b} replays of {len(calls)} launches per stage")
        # region C: plain launches (one ctypes call per stage, no graph)
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
    stages = stage_summary(per)
    steps_per_s = 1e3 / ms_per_step

    # algorithmic work
    logit_bytes = L * cfg.vocab * 4 + L * K * 8 + L * 4
    verify_flops = float(np.mean([ch.verify_flops for ch in chains]))
    drafter_bytes = ((ctx + L) * cfg.hkv * cfg.D * 2 * 2) + 2 * (L * cfg.hq * cfg.D * 2)
    t_logit = stages["topk"]["mean"] * 1e-6
    t_verify = stages["verify_attn"]["mean"] * 1e-6
    t_draft = stages["drafter_attn"]["mean"] * 1e-6
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
            "kernel": "verify attention (attn_kernel<128,split> + attn_combine_kernel<128,8,spec>)",
            "achieved": round(verify_tflops, 3),
            "peak": BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(verify_tflops / BF16_PEAK_TFLOPS, 5),
            "traffic": traffic,
            "launch_us": stages["verify_attn"],
            "replays": reps_b,
            "algorithmic_flops_per_launch": verify_flops,
            "issued_mfma_flops_per_launch": issued_mfma,
            "mfma_busy_pct_main_kernel": mfma_busy,
        },
        "stages_us": {n: stages[n]["mean"] for n in names},
        "stages_us_spread": stages,
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
        mean, med, mn = spread(step_ms)
        result["step_us_spread"] = {"mean": round(mean, 3), "median": round(med, 3),
                                    "min": round(mn, 3), "replays": reps_b}
        result["plain_launches"] = {"steps": n_eager, "ms_per_step": round(eager_ms, 5),
                                    "steps_per_s": round(1e3 / eager_ms, 2)}
        fl = floor_leg(torch, ddt, dev, reps_b)
        two = fl["one_launch_read_us"] + fl["dependent_launch_us"]
        fl["two_launch_floor_us"] = round(two, 3)
        fl["logit_pass_us"] = stages["topk"]["mean"]
        fl["logit_pass_frac_of_floor"] = round(two / stages["topk"]["mean"], 4)
        result["logit_pass"]["floor"] = fl
    result["accept_36_layers"] = accept_layers_leg(torch, ddt, synth, chains, cases, cfg, dev)
    result["tree_rope_kv"] = tree_rope_leg(torch, ddt, chains, cfg, dev)
    result["packed_blocks_attn"] = packed_blocks_leg(torch, ddt, chains, cfg, dev)
    if not args.no_workloads and not args.eager:
        del calls
        result["workloads"] = {
            "c4_peaked": workload_leg(args, torch, ddt, synth, synth.CONFIGS[4], 4,
                                      args.seed + 40, dev,
                                      "ddtree_b1024_peaked: L=16 K=64 B=1024 P=4096", reps_b),
            "c4_flat": workload_leg(args, torch, ddt, synth, synth.FLAT4, 4, args.seed + 41,
                                    dev, "ddtree_b1024_flat: L=16 K=64 B=1024 P=4096, delta/2",
                                    reps_b),
            "c5_serving": workload_leg(args, torch, ddt, synth, synth.CONFIGS[5], 2,
                                       args.seed + 50, dev,
                                       "serving_b32: 32 requests x (L=16 K=16 B=64), "
                                       "P~U{512..8192}, hq=32 hkv=4", max(10, reps_b // 5)),
        }
    if not args.no_streams:
        result["verify_attn_serving"] = serving_verify_leg(args, torch, ddt, synth, dev)
    if not args.no_streams:
        (result["target_argmax"], result["logit_pass_512rows"],
         result["lmhead_topk"]) = stream_passes(args, torch, ddt, synth, dev)
    if args.cpu_seconds > 0:
        result["cpu_baseline"] = cpu_baseline(cases[0], args.cpu_seconds, args)
    print(json.dumps(result), flush=True)


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(case, budget_s, args):
    """The oracle, as it stands, running the same chain step on the host:
    first with every core its numerical libraries use, then limited to one
    thread; per-stage times in both modes.  About budget_s seconds of host
    time per mode (at least one step each)."""
    import synth
    from oracle.accept import accept_compact
    from oracle.attention import masked_attention
    from oracle.logits import topk_logprobs
    from oracle.tree import build_trees
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:  # pragma: no cover - threadpoolctl is in the image
        threadpool_info = threadpool_limits = None
        threads = 1
    cfg = case.cfg
    L, ctx = cfg.L, cfg.drafter_ctx
    dq = synth.bf16_bits_to_f32(case.dq_bits)
    dk = synth.bf16_bits_to_f32(case.dk_bits)
    dv = synth.bf16_bits_to_f32(case.dv_bits)
    vq = synth.bf16_bits_to_f32(case.vq_bits)
    vk = synth.bf16_bits_to_f32(case.vk_bits)
    vv = synth.bf16_bits_to_f32(case.vv_bits)
    y = synth.sample_target_path(case)
    names = ["drafter_attn", "topk", "tree", "verify_attn", "accept"]

    def one_step(acc):
        t = [time.perf_counter()]
        masked_attention(dq, dk, dv, [0], [ctx], [L], None)
        t.append(time.perf_counter())
        ids, logp, _ = topk_logprobs(case.logits, cfg.K)
        t.append(time.perf_counter())
        tr = build_trees(logp, ids, case.root_token, 1, L, cfg.k_tree, cfg.B)
        t.append(time.perf_counter())
        masked_attention(vq, vk, vv, case.kv_base, case.prefix_len, tr["n_nodes"], tr["mask"])
        t.append(time.perf_counter())
        tgt = synth.target_for_tree(tr["token"][0], tr["parent"][0], tr["depth"][0],
                                    int(tr["n_nodes"][0]), y[0], case.off_path[0])[None]
        t0 = time.perf_counter()
        accept_compact(tr["token"], tr["parent"], tr["n_nodes"], tgt, L, case.vk_bits[None],
                       case.vv_bits[None], case.kv_base, case.prefix_len)
        t.append(time.perf_counter() - (t0 - t[-1]))     # target drawing excluded
        for j in range(len(names)):
            acc[j] += t[j + 1] - t[j]

    def run(mode):
        acc = np.zeros(len(names))
        n, t0 = 0, time.perf_counter()
        while True:
            one_step(acc)
            n += 1
            el = time.perf_counter() - t0
            log(args, f"cpu baseline ({mode}) step {n}: {el:.1f}s")
            if el >= budget_s:
                break
        return n, float(acc.sum()), {nm: round(a / n * 1e3, 2) for nm, a in zip(names, acc)}

    n_all, t_all, st_all = run("all cores")
    if threadpool_limits is not None:
        with threadpool_limits(limits=1):
            n_one, t_one, st_one = run("one thread")
    else:
        n_one, t_one, st_one = run("one thread")
    try:
        affinity = len(os.sched_getaffinity(0))
    except Exception:
        affinity = os.cpu_count()
    return {"value": round(n_all / t_all, 4), "unit": "steps/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{n_all} full oracle chain steps on input set 0 of the same workload "
                      f"({t_all:.1f} s of host time; float64 numpy, numerical-library threads="
                      f"{threads})",
            "stage_ms": st_all,
            "single_thread": {"value": round(n_one / t_one, 4), "unit": "steps/s", "cores": 1,
                              "steps": n_one, "stage_ms": st_one},
            "nproc": os.cpu_count(), "affinity_cpus": affinity, "cpu_model": _cpu_model()}


if __name__ == "__main__":
    main()
