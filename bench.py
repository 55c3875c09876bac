"""Benchmark: one rank's share of context-parallel Pass-KV ring attention on one MI355X.

A step is one pass of the whole hot path for one rank: the zigzag partition and
block classes (host), then every ring step's forward kernel with the merge of
its partial output, with each visiting KV block staged through a receive
buffer on a side stream.  Default workload: Llama-3-8B attention shape
(Hq=32, Hkv=8, D=128, bf16) on rank 0's share of S=128K at CP=8 (local 16K
tokens as two zigzag 8K chunks, 8 ring steps).  Inputs are seeded synthetic
N(0,1) values rounded to bf16, resident in HBM before timing starts.

Prints one JSON line.  FLOPs are causal-counted: 4*D per visible (query, key)
pair and query head for the forward.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

BF16_PEAK_TFLOPS = 2516.6   # MI355X dense bf16 MFMA (256 CU x 2.4 GHz x 4096 FLOP/clk)


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def _dev_bf16(torch, x):
    from context_long_attention_amd import inputs
    return torch.from_numpy(inputs.bf16_bits(x).view(np.int16)).cuda().view(torch.bfloat16)


def make_rank_inputs(torch, w, rank):
    from context_long_attention_amd import cpattn, inputs
    c, R = w.chunk, w.cp
    pos = cpattn.cp_partition_zigzag(w.seq_len, R, rank)
    qa, qb = int(pos[0]) // c, int(pos[c]) // c
    q = _dev_bf16(torch, inputs.chunks_normal(inputs.SEED_Q, [qa, qb], c, w.hq, w.dim))
    kv = {}
    for s in range(R):
        ps = cpattn.cp_partition_zigzag(w.seq_len, R, s)
        ka, kb = int(ps[0]) // c, int(ps[c]) // c
        kv[s] = (_dev_bf16(torch, inputs.chunks_normal(inputs.SEED_K, [ka, kb], c, w.hkv, w.dim)),
                 _dev_bf16(torch, inputs.chunks_normal(inputs.SEED_V, [ka, kb], c, w.hkv, w.dim)))
    return q, kv


class KernelTimer:
    """HIP events around each launch of one kernel, on the stream it runs on."""

    def __init__(self, torch, kind):
        self.torch = torch
        self.kind = kind
        self.pairs = []
        self.enabled = False

    def __call__(self, step, what, stream):
        if not self.enabled or not what.startswith(self.kind):
            return
        ev = self.torch.cuda.Event(enable_timing=True)
        ev.record(stream)
        if what.endswith("begin"):
            self.pairs.append([ev, None])
        else:
            self.pairs[-1][1] = ev

    def total_ms(self):
        return sum(a.elapsed_time(b) for a, b in self.pairs)


def cpu_baseline(w, rank, heads):
    """The float64 oracle on a bounded sample: ``heads`` query heads of the GQA group
    of KV head 0, every ring step of the rank, every local row."""
    import oracle
    from context_long_attention_amd import inputs
    try:
        from threadpoolctl import threadpool_info
        threads = max([int(i.get("num_threads", 1)) for i in threadpool_info() if i.get("user_api") == "blas"]
                      or [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    c, R = w.chunk, w.cp
    qa, qb = oracle.zigzag_chunks(R, rank)
    qpos = oracle.zigzag_positions(w.seq_len, R, rank)
    q = inputs.round_bf16(inputs.chunks_normal(inputs.SEED_Q, [qa, qb], c, w.hq, w.dim))[:, :heads]
    blocks = []
    for t in range(R):
        s = oracle.ring_source(rank, t, R)
        ka, kb = oracle.zigzag_chunks(R, s)
        k = inputs.round_bf16(inputs.chunks_normal(inputs.SEED_K, [ka, kb], c, w.hkv, w.dim))[:, :1]
        v = inputs.round_bf16(inputs.chunks_normal(inputs.SEED_V, [ka, kb], c, w.hkv, w.dim))[:, :1]
        blocks.append((k, v, oracle.zigzag_positions(w.seq_len, R, s)))
    flops = 0
    for k, v, kpos in blocks:
        flops += oracle.causal_flops(qpos, kpos, heads, w.dim)
    t0 = time.perf_counter()
    oracle.rank_forward(q, qpos, blocks, None, w.scale)
    dt = time.perf_counter() - t0
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{w.name} rank {rank}: forward of {heads} of {w.hq} query heads (KV head 0), "
                      f"all {R} ring steps, all {2 * c} local rows, float64 NumPy; {dt:.1f} s",
            "seconds": dt, "flops": flops}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="llama3_8b_fwd")
    ap.add_argument("--rank", type=int, default=0)
    ap.add_argument("--cpu-heads", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU (one rank's share of the ring); --gpus {args.gpus} "
              "is not supported: nothing here uses a second GPU.", file=sys.stderr)
        sys.exit(2)

    import torch
    from context_long_attention_amd import cpattn, inputs
    from context_long_attention_amd.ring import RankRing

    w = inputs.WORKLOADS[args.workload]
    cpattn.lib()
    torch.cuda.set_device(0)
    log(f"workload {w.name}: S={w.seq_len} CP={w.cp} Hq={w.hq} Hkv={w.hkv} D={w.dim} rank={args.rank}")
    t0 = time.perf_counter()
    q, kv = make_rank_inputs(torch, w, args.rank)
    torch.cuda.synchronize()
    log(f"inputs resident in HBM ({time.perf_counter() - t0:.1f} s)")

    ring = RankRing(w, args.rank)
    pairs = [ring.step_pairs(t) for t in range(w.cp)]
    flops_fwd = sum(pairs) * w.hq * w.dim * 4
    timer = KernelTimer(torch, "fwd")
    kv_of = kv.__getitem__

    def one_step():
        # host part of the path: partition and per-step classes are recomputed each step
        r = RankRing(w, args.rank)
        return r.forward(q, kv_of, stage=True, timer=timer)

    for i in range(args.warmup):
        one_step()
        torch.cuda.synchronize()
        log(f"warmup {i + 1}/{args.warmup} done")
    timer.enabled = True
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(args.steps):
        one_step()
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    kern_ms = timer.total_ms() / args.steps
    log(f"timed {args.steps} steps: {ms:.3f} ms/step, fwd kernels {kern_ms:.3f} ms/step")

    value = flops_fwd / (ms * 1e-3) / 1e12
    achieved = flops_fwd / (kern_ms * 1e-3) / 1e12
    n_launch = w.cp
    record = {
        "metric": "causal attention TFLOP/s per ring-step share (fwd, fwd+bwd); % bf16 MFMA peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "seq_len": w.seq_len, "cp": w.cp, "rank": args.rank,
                   "local_tokens": w.local, "hq": w.hq, "hkv": w.hkv, "head_dim": w.dim,
                   "ring_steps": w.cp, "pass": "fwd"},
        "pct_bf16_peak": round(100 * value / BF16_PEAK_TFLOPS, 2),
        "kernel_only": {"tflops": round(achieved, 2), "pct_bf16_peak": round(100 * achieved / BF16_PEAK_TFLOPS, 2),
                        "ms_per_step": round(kern_ms, 4)},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / BF16_PEAK_TFLOPS, 4), "traffic": None,
                     "kernel": "fwd_step_kernel<128,4>",
                     "flops_per_launch": flops_fwd / n_launch,
                     "avg_launch_ms": round(kern_ms / n_launch, 4)},
    }
    if not args.no_cpu_baseline:
        log("timing the float64 oracle on the host (cpu_baseline)")
        record["cpu_baseline"] = cpu_baseline(w, args.rank, args.cpu_heads)
    print(json.dumps(record), flush=True)


if __name__ == "__main__":
    main()
