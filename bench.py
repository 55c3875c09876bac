"""Benchmark: one rank's share of context-parallel Pass-KV ring attention on one MI355X.

A step is one pass of the whole hot path for one rank: the zigzag partition and
block classes (host), then every ring step's forward kernel with the merge of
its partial output (step 0 writes the accumulator, later steps merge into it
inside the kernel), with each visiting KV block staged through a receive buffer
on a side stream.  Default workload: Llama-3-8B attention shape
(Hq=32, Hkv=8, D=128, bf16) on rank 0's share of S=128K at CP=8 (local 16K
tokens as two zigzag 8K chunks, 8 ring steps).  Inputs are seeded synthetic
N(0,1) values rounded to bf16, resident in HBM before timing starts.

Prints one JSON line.  FLOPs are causal-counted: 4*D per visible (query, key)
pair and query head for the forward.  The roofline object describes the
merging step kernel (ring steps 1..R-1); its ``traffic`` is that kernel's HBM
traffic per launch from the committed FETCH_SIZE / WRITE_SIZE summary under
profiles/, when that summary was taken on the current kernel sources (else
null); ``--calibrate-copy-mib`` makes the known-size copies that summary is
scaled by.
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

    def launch_ms(self):
        return [a.elapsed_time(b) for a, b in self.pairs]


class ClockSampler:
    """GFX clock (MHz) and socket power (W) as reported by amd-smi, sampled every
    `period` seconds in a background thread while a measured leg runs (warm-up
    and timed steps; the driver's own sampling window may be coarser).  Reads
    only; reports None where amd-smi is unavailable."""

    def __init__(self, period=0.02):
        import threading
        self.period = period
        self.clk, self.power = [], []
        self._stop = threading.Event()
        self._thread = None
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            self.smi = amdsmi
            self.handle = amdsmi.amdsmi_get_processor_handles()[0]  # the box's one GPU
        except Exception:  # noqa: BLE001 -- any failure just disables the readings
            self.smi = self.handle = None

    def _sample(self):
        a = self.smi
        while not self._stop.is_set():
            try:
                c = a.amdsmi_get_clock_info(self.handle, a.AmdSmiClkType.GFX)
                v = c.get("clk", c.get("cur_clk"))
                if isinstance(v, (int, float)) and v > 0:
                    self.clk.append(float(v))
                pw = a.amdsmi_get_power_info(self.handle)
                v = pw.get("current_socket_power", pw.get("average_socket_power"))
                if isinstance(v, (int, float)) and v > 0:
                    self.power.append(float(v))
            except Exception:  # noqa: BLE001
                pass
            self._stop.wait(self.period)

    def start(self):
        import threading
        if self.handle is not None:
            self._thread = threading.Thread(target=self._sample, daemon=True)
            self._thread.start()
        return self

    def stop(self):
        if self._thread is None:
            return None
        self._stop.set()
        self._thread.join()
        if not self.clk:
            return None
        med = lambda x: float(np.median(x)) if x else None
        return {"sclk_mhz_median": med(self.clk), "sclk_mhz_min": min(self.clk), "sclk_mhz_max": max(self.clk),
                "socket_power_w_median": med(self.power), "samples": len(self.clk),
                "source": "amd-smi GFX clock / socket power, sampled every 20 ms over warm-up and timed steps"}


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


def fwd_algorithmic_bytes(w, live_rows, merge):
    """Bytes one forward step launch must move at least: Q, K and V read once
    (bf16); then for the rows that see a key in the step, O and LSE (fp32)
    written once, or, when the launch merges into the accumulator, read and
    written once."""
    q = w.local * w.hq * w.dim * 2
    kv = 2 * w.local * w.hkv * w.dim * 2
    out = live_rows * w.hq * (w.dim + 1) * 4
    return q + kv + out * (2 if merge else 1)


def live_rows(w, rank, step):
    """Local rows with a visible key at this step of a causal ring: every row of
    a query chunk whose chunk pairs are not all SKIP (a causal DIAG or FULL
    pair gives each of its rows at least one key)."""
    from context_long_attention_amd import cpattn
    m = cpattn.cp_step_masks(w.cp, rank, step, False)
    return w.chunk * sum(any(c != cpattn.CP_MASK_SKIP for c in row) for row in m)


def calibration_copies(torch, mib, count=3):
    """Plain device-to-device copies of a known size, made before any other GPU
    work so that they are the first copy dispatches a counter run records."""
    src = torch.empty(mib << 20, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(count):
        dst.copy_(src)
    torch.zeros(1, device="cuda")  # a non-copy dispatch marks the end of the calibration
    torch.cuda.synchronize()
    log(f"calibration: {count} copies of {mib} MiB")
    del src, dst


def measure(torch, w, rank, steps, warmup, backward):
    """Time `steps` whole-rank passes (forward ring, plus the backward ring if asked)."""
    from context_long_attention_amd.ring import RankRing
    t0 = time.perf_counter()
    q, kv = make_rank_inputs(torch, w, rank)
    d_o = None
    if backward:
        from context_long_attention_amd import cpattn, inputs
        c = w.chunk
        pos = cpattn.cp_partition_zigzag(w.seq_len, w.cp, rank)
        d_o = _dev_bf16(torch, inputs.chunks_normal(inputs.SEED_DO, [int(pos[0]) // c, int(pos[c]) // c], c,
                                                    w.hq, w.dim))
    torch.cuda.synchronize()
    log(f"{w.name}: inputs resident in HBM ({time.perf_counter() - t0:.1f} s)")
    ring = RankRing(w, rank)
    pairs = sum(ring.step_pairs(t) for t in range(w.cp))
    flops_fwd = pairs * w.hq * w.dim * 4
    flops_bwd = pairs * w.hq * w.dim * 10
    fwd_timer = KernelTimer(torch, "fwd")
    bwd_timer = KernelTimer(torch, "bwd")
    kv_of = kv.__getitem__

    def timer(step, what, stream):
        fwd_timer(step, what, stream)
        bwd_timer(step, what, stream)

    def one_step():
        # the host part of the path (partition, per-step classes) is redone every step
        r = RankRing(w, rank)
        o, lse, _ = r.forward(q, kv_of, stage=True, timer=timer)
        if backward:
            r.backward(q, d_o, o, lse, kv_of, stage=True, keep_steps=False, timer=timer)

    sampler = ClockSampler().start()
    for i in range(warmup):
        one_step()
        torch.cuda.synchronize()
        log(f"{w.name}: warmup {i + 1}/{warmup} done")
    fwd_timer.enabled = bwd_timer.enabled = True
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(steps):
        one_step()
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    clocks = sampler.stop()
    per_step = [ring.step_pairs(t) * w.hq * w.dim * 4 for t in range(w.cp)]
    launch = fwd_timer.launch_ms()
    merge_ms = [x for i, x in enumerate(launch) if i % w.cp > 0]
    out = {"ms": ms, "fwd_kernel_ms": fwd_timer.total_ms() / steps, "flops_fwd": flops_fwd,
           "flops_bwd": flops_bwd if backward else 0, "launches": w.cp, "clocks": clocks,
           # the launches that merge into the accumulator (ring steps 1..R-1)
           "merge_flops_per_launch": sum(per_step[1:]) / max(1, w.cp - 1),
           "merge_avg_launch_ms": sum(merge_ms) / max(1, len(merge_ms)),
           "merge_bytes_per_launch": sum(fwd_algorithmic_bytes(w, live_rows(w, rank, t), True)
                                         for t in range(1, w.cp)) / max(1, w.cp - 1)}
    if backward:
        out["bwd_kernel_ms"] = bwd_timer.total_ms() / steps
    log(f"{w.name}: {steps} steps, {ms:.3f} ms/step, fwd kernels {out['fwd_kernel_ms']:.3f} ms"
        + (f", bwd kernels {out['bwd_kernel_ms']:.3f} ms" if backward else ""))
    return out


def _hpw(w):
    """Query heads per forward workgroup (the kernel's second template argument)."""
    from context_long_attention_amd import cpattn
    bm, _ = cpattn.cp_tile_shape(w.hq, w.hkv, w.dim)
    return 256 // bm


def tflops(flops, ms):
    return flops / (ms * 1e-3) / 1e12


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="llama3_8b_fwd")
    ap.add_argument("--bwd-workload", default="llama3_8b_fwdbwd")
    ap.add_argument("--rank", type=int, default=0)
    ap.add_argument("--cpu-heads", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-bwd", action="store_true")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="first make 3 device-to-device copies of this many MiB (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU (one rank's share of the ring); --gpus {args.gpus} "
              "is not supported: nothing here uses a second GPU.", file=sys.stderr)
        sys.exit(2)

    import torch
    from context_long_attention_amd import cpattn, inputs, profsum

    cpattn.lib()
    torch.cuda.set_device(0)
    if args.calibrate_copy_mib > 0:
        calibration_copies(torch, args.calibrate_copy_mib)
    w = inputs.WORKLOADS[args.workload]
    log(f"workload {w.name}: S={w.seq_len} CP={w.cp} Hq={w.hq} Hkv={w.hkv} D={w.dim} rank={args.rank}")
    fwd = measure(torch, w, args.rank, args.steps, args.warmup, backward=False)
    value = tflops(fwd["flops_fwd"], fwd["ms"])
    kernel_tflops = tflops(fwd["flops_fwd"], fwd["fwd_kernel_ms"])
    # roofline of the dominant kernel: the step kernel that merges into the
    # accumulator (ring steps 1..R-1; step 0 writes the accumulator directly)
    achieved = tflops(fwd["merge_flops_per_launch"], fwd["merge_avg_launch_ms"])
    kernel = f"fwd_step_kernel<{w.dim}, {_hpw(w)}, true>"
    prof = os.path.join(ROOT, "profiles", f"fwd_step_kernel_{w.name}_traffic.md")
    measured = profsum.read_traffic(prof, kernel, w.name)
    record = {
        "metric": "causal attention TFLOP/s per ring-step share (fwd, fwd+bwd); % bf16 MFMA peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(fwd["ms"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "seq_len": w.seq_len, "cp": w.cp, "rank": args.rank,
                   "local_tokens": w.local, "hq": w.hq, "hkv": w.hkv, "head_dim": w.dim,
                   "ring_steps": w.cp, "pass": "fwd"},
        "pct_bf16_peak": round(100 * value / BF16_PEAK_TFLOPS, 2),
        "clocks": fwd["clocks"],
        "kernel_only": {"tflops": round(kernel_tflops, 2),
                        "pct_bf16_peak": round(100 * kernel_tflops / BF16_PEAK_TFLOPS, 2),
                        "ms_per_step": round(fwd["fwd_kernel_ms"], 4)},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / BF16_PEAK_TFLOPS, 4),
                     "traffic": measured["traffic_bytes_per_launch"] if measured else None,
                     "kernel": kernel,
                     "flops_per_launch": fwd["merge_flops_per_launch"],
                     "algorithmic_bytes_per_launch": round(fwd["merge_bytes_per_launch"]),
                     "traffic_source": os.path.relpath(prof, ROOT) if measured else None,
                     "avg_launch_ms": round(fwd["merge_avg_launch_ms"], 4)},
    }
    if not args.no_bwd:
        wb = inputs.WORKLOADS[args.bwd_workload]
        fb = measure(torch, wb, args.rank, max(1, args.steps // 2), 1, backward=True)
        total = fb["flops_fwd"] + fb["flops_bwd"]
        record["fwd_bwd"] = {
            "workload": wb.name, "seq_len": wb.seq_len, "cp": wb.cp, "ring_steps": wb.cp,
            "tflops": round(tflops(total, fb["ms"]), 2),
            "pct_bf16_peak": round(100 * tflops(total, fb["ms"]) / BF16_PEAK_TFLOPS, 2),
            "ms_per_step": round(fb["ms"], 4),
            "fwd_kernel_tflops": round(tflops(fb["flops_fwd"], fb["fwd_kernel_ms"]), 2),
            "bwd_kernel_tflops": round(tflops(fb["flops_bwd"], fb["bwd_kernel_ms"]), 2),
            "bwd_kernel_ms_per_step": round(fb["bwd_kernel_ms"], 4),
            "clocks": fb["clocks"],
        }
    if not args.no_cpu_baseline:
        log("timing the float64 oracle on the host (cpu_baseline)")
        record["cpu_baseline"] = cpu_baseline(w, args.rank, args.cpu_heads)
    print(json.dumps(record), flush=True)


if __name__ == "__main__":
    main()
