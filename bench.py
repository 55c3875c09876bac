"""Benchmark: one rank's share of context-parallel Pass-KV ring attention on one MI355X.

A step is one pass of the whole hot path for one rank: the zigzag partition and
block classes (host), then every ring step's forward kernel with the merge of
its partial output (step 0 writes the accumulator, later steps merge into it
inside the kernel); step 0 reads the rank's own KV block in place and every
later visiting block is staged through a receive buffer on a side stream.  Default workload: Llama-3-8B attention shape
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

Timing protocol: every timed pass of a leg is bracketed by its own pair of HIP
events, so each leg reports the median (and min / max) over its repetitions --
the K headline steps, 10 passes of the Llama-3-8B training and packed-document
legs, 3 of the Llama-3-405B leg -- and the headline and training legs also give
the median launch time of every ring step.  ``value`` itself is the whole-job
rate over the K bracketed headline steps.  The float64 oracle is timed on the
host on a bounded sample of the headline workload (``cpu_baseline``) and, with
its rate extrapolated to the whole share, of the Llama-3-405B one; on the
headline sample its result is also compared with the final O and LSE of the
last measured ring (``cpu_baseline.parity``: max-abs error of O, max relative
error of LSE, against the 2e-2 and 1e-3 bars).
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


def probe_clock(torch, one_step):
    """Shader clock the forward step kernel runs at, from its own counters: two
    extra (untimed) passes with cp_debug_clock_probe on (launches after an idle
    GPU start up to 25% slower and settle within about ten milliseconds, so the
    first pass only warms up); per workgroup of the last launch, clock =
    cycle-counter difference / 100 MHz tick difference.
    Workgroups shorter than 10 us (steps where their tile sees no key) are left
    out.  Returns the median over workgroups and per XCD (workgroup id mod 8)."""
    from context_long_attention_amd import cpattn
    buf = torch.zeros(4 * 65536, dtype=torch.int64, device="cuda")
    cpattn.cp_debug_clock_probe(buf)
    try:
        one_step()
        one_step()
        torch.cuda.synchronize()
    finally:
        cpattn.cp_debug_clock_probe(None)
    rec = buf.view(-1, 4).cpu().numpy()
    ids = np.nonzero(rec[:, 1])[0]
    rec = rec[ids]
    ticks = rec[:, 3] - rec[:, 1]
    keep = ticks >= 1000
    if not keep.any():
        return None
    mhz = (rec[keep, 2] - rec[keep, 0]) / ticks[keep] * 100.0
    xcd = ids[keep] % 8
    return {"sclk_mhz_median": round(float(np.median(mhz)), 1),
            "sclk_mhz_per_xcd": [round(float(np.median(mhz[xcd == x])), 1) if (xcd == x).any() else None
                                 for x in range(8)],
            "workgroups": int(keep.sum()),
            "source": "forward step kernel's own cycle / 100 MHz counters (cp_debug_clock_probe), last launch "
                      "of two extra untimed passes"}


def gemm_reference(torch, n=16384, reps=10):
    """Context for the power-capped clock, not part of the measured path: the
    vendor library's dense bf16 GEMM (torch.matmul, n^3) on the same GPU in the
    same run, as TFLOP/s and as a fraction of the same bf16 peak."""
    a = torch.randn((n, n), device="cuda", dtype=torch.bfloat16)
    b = torch.randn((n, n), device="cuda", dtype=torch.bfloat16)
    torch.matmul(a, b)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(reps):
        torch.matmul(a, b)
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / reps
    t = tflops(2.0 * n ** 3, ms)
    return {"kind": "vendor library dense GEMM on the same GPU (context, not this library's code)",
            "shape": f"bf16 [{n}, {n}] x [{n}, {n}], torch.matmul", "tflops": round(t, 2),
            "pct_bf16_peak": round(100 * t / BF16_PEAK_TFLOPS, 2), "ms": round(ms, 3)}


def blas_threads():
    """Threads the oracle's BLAS calls use on this host."""
    try:
        from threadpoolctl import threadpool_info
        return max([int(i.get("num_threads", 1)) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        return len(os.sched_getaffinity(0))


def cpu_baseline(w, rank, heads, final=None):
    """The float64 oracle on a bounded sample: ``heads`` query heads of the GQA group
    of KV head 0, every ring step of the rank, every local row.  ``final`` (the
    GPU's final O and LSE of the same ring, optional): its errors against the
    oracle on that sample are reported too."""
    import oracle
    from context_long_attention_amd import inputs
    threads = blas_threads()
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
    ro, rl, _ = oracle.rank_forward(q, qpos, blocks, None, w.scale)
    dt = time.perf_counter() - t0
    out = {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
           "sample": f"{w.name} rank {rank}: forward of {heads} of {w.hq} query heads (KV head 0), "
                     f"all {R} ring steps, all {2 * c} local rows, float64 NumPy; {dt:.1f} s",
           "seconds": dt, "flops": flops}
    if final is not None:
        go = final[0][:, :heads].cpu().numpy().astype(np.float64)
        gl = final[1][:heads].cpu().numpy().astype(np.float64)
        live = np.isfinite(rl).T
        err_o = float(np.abs(go - ro)[live].max())
        dead = np.isneginf(rl)
        err_l = float((np.abs(gl[~dead] - rl[~dead]) / np.maximum(1.0, np.abs(rl[~dead]))).max())
        out["parity"] = {"checked": f"final O and LSE of the last measured ring against the oracle on this sample "
                                    f"({2 * c} rows x {heads} heads)",
                         "o_max_abs_err": err_o, "lse_max_rel_err": err_l, "o_bar": 2e-2, "lse_bar": 1e-3,
                         "same_minus_inf_rows": bool(np.array_equal(np.isneginf(gl), dead)),
                         "within_bar": bool(err_o <= 2e-2 and err_l <= 1e-3 and np.array_equal(np.isneginf(gl), dead))}
    return out


def cpu_baseline_extrapolated(w, rank, row_stride=4, steps=(0, 1)):
    """The float64 oracle on a bounded sample of a share too large to run whole:
    query head 0, every ``row_stride``-th local row, ring steps ``steps``; its rate
    (causal-counted FLOP of the sample over the sample's time) is the baseline,
    and the whole share's time is extrapolated from it.  K and V follow the input
    recipe; the sampled query rows are N(0,1) draws of their own (the recipe draws
    every head of a chunk at once, 4 GiB for a Llama-3-405B query chunk), rounded
    to bf16 -- the oracle's work does not depend on the values."""
    import oracle
    from context_long_attention_amd import inputs
    c, R = w.chunk, w.cp
    rows = np.arange(0, 2 * c, row_stride)
    qpos = oracle.zigzag_positions(w.seq_len, R, rank)[rows]
    q = inputs.round_bf16(np.random.default_rng([inputs.SEED_Q, 1 << 20, rank]).standard_normal(
        (len(rows), 1, w.dim), dtype=np.float32))
    blocks, flops = [], 0
    for t in steps:
        s_ = oracle.ring_source(rank, t, R)
        ka, kb = oracle.zigzag_chunks(R, s_)
        kv = [np.concatenate([inputs.round_bf16(inputs.chunk_normal(seed, ch, c, w.hkv, w.dim)[:, :1])
                              for ch in (ka, kb)]) for seed in (inputs.SEED_K, inputs.SEED_V)]
        kpos = oracle.zigzag_positions(w.seq_len, R, s_)
        blocks.append((kv[0], kv[1], kpos))
        flops += oracle.causal_flops(qpos, kpos, 1, w.dim)
    t0 = time.perf_counter()
    oracle.rank_forward(q, qpos, blocks, None, w.scale)
    dt = time.perf_counter() - t0
    rate = flops / dt
    return {"value": rate / 1e12, "unit": "TFLOP/s", "cores": blas_threads(), "kind": "oracle", "extrapolated": True,
            "sample": f"{w.name} rank {rank}: forward of query head 0 of {w.hq}, every {row_stride}th of the "
                      f"{2 * c} local rows, ring steps {list(steps)} of {R}, float64 NumPy; {dt:.1f} s; "
                      f"rate extrapolated to the whole share",
            "seconds": dt, "flops": flops}


def fwd_algorithmic_bytes(w, live_rows, merge):
    """Bytes one forward step launch must move at least: K and V read once
    (bf16); then for the rows that see a key in the step, Q read once (bf16)
    and O and LSE (fp32) written once, or, when the launch merges into the
    accumulator, read and written once."""
    q = live_rows * w.hq * w.dim * 2
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

    last = {}

    def one_step():
        # the host part of the path (partition, per-step classes) is redone every step
        r = RankRing(w, rank)
        o, lse, _ = r.forward(q, kv_of, stage=True, timer=timer)
        last["o"], last["lse"] = o, lse  # the final output of the last pass (kept for the parity check)
        if backward:
            r.backward(q, d_o, o, lse, kv_of, stage=True, keep_steps=False, timer=timer)

    for i in range(warmup):
        one_step()
        torch.cuda.synchronize()
        log(f"{w.name}: warmup {i + 1}/{warmup} done")
    fwd_timer.enabled = bwd_timer.enabled = True
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    start.record()
    marks[0].record()
    for i in range(steps):
        one_step()
        marks[i + 1].record()
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    rep_ms = [marks[i].elapsed_time(marks[i + 1]) for i in range(steps)]
    fwd_timer.enabled = bwd_timer.enabled = False
    clocks = probe_clock(torch, one_step)
    per_step = [ring.step_pairs(t) * w.hq * w.dim * 4 for t in range(w.cp)]
    launch = fwd_timer.launch_ms()
    merge_ms = [x for i, x in enumerate(launch) if i % w.cp > 0]
    # median launch time of each ring step over the timed passes (every step of
    # these causal rings is live, so each pass launches R forward kernels)
    fwd_steps = np.asarray(launch).reshape(steps, w.cp)
    out = {"ms": ms, "rep_ms": rep_ms, "fwd_step_ms": np.median(fwd_steps, axis=0).tolist(),
           "fwd_kernel_ms": fwd_timer.total_ms() / steps, "flops_fwd": flops_fwd,
           "flops_bwd": flops_bwd if backward else 0, "launches": w.cp, "clocks": clocks,
           # the launches that merge into the accumulator (ring steps 1..R-1)
           "merge_flops_per_launch": sum(per_step[1:]) / max(1, w.cp - 1),
           "merge_avg_launch_ms": sum(merge_ms) / max(1, len(merge_ms)),
           "merge_bytes_per_launch": sum(fwd_algorithmic_bytes(w, live_rows(w, rank, t), True)
                                         for t in range(1, w.cp)) / max(1, w.cp - 1)}
    out["final"] = (last["o"], last["lse"])
    if backward:
        out["bwd_kernel_ms"] = bwd_timer.total_ms() / steps
        out["bwd_step_ms"] = np.median(np.asarray(bwd_timer.launch_ms()).reshape(steps, w.cp), axis=0).tolist()
    log(f"{w.name}: {steps} steps, {ms:.3f} ms/step, fwd kernels {out['fwd_kernel_ms']:.3f} ms"
        + (f", bwd kernels {out['bwd_kernel_ms']:.3f} ms" if backward else ""))
    return out


def _hpw(w):
    """Query heads per forward workgroup (the kernel's second template argument)."""
    from context_long_attention_amd import cpattn
    bm, _ = cpattn.cp_tile_shape(w.hq, w.hkv, w.dim)
    return 256 // bm


def _dev_normal(torch, shape, seed):
    """Seeded N(0,1) draws made on the device and rounded to bf16 (the variant legs;
    the shapes, not the values, matter for timing)."""
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    return torch.randn(shape, generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)


def _time_leg(torch, fn, steps, warmup, timer=None):
    """(ms per call of fn over `steps` timed calls, kernel ms per call or None,
    the ms of each timed call)."""
    for _ in range(warmup):
        fn(None)
    torch.cuda.synchronize()
    if timer is not None:
        timer.enabled = True
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    marks[0].record()
    for i in range(steps):
        fn(timer)
        marks[i + 1].record()
    torch.cuda.synchronize()
    kern = timer.total_ms() / steps if timer is not None else None
    reps = [marks[i].elapsed_time(marks[i + 1]) for i in range(steps)]
    return marks[0].elapsed_time(marks[-1]) / steps, kern, reps


def rep_stats(rep_ms):
    """Median, min and max over the timed repetitions of a leg."""
    return {"reps": len(rep_ms), "ms_median": round(float(np.median(rep_ms)), 4),
            "ms_min": round(float(np.min(rep_ms)), 4), "ms_max": round(float(np.max(rep_ms)), 4)}


def measure_variants(torch, w, rank, steps, warmup):
    """The ring variants beside Pass KV, at the Llama-3-8B forward shape."""
    from context_long_attention_amd import cpattn
    from context_long_attention_amd.variants import (PartialPrefillRank, PassQRank, gathered_forward,
                                                     head_sharded_forward)
    out = {}
    c, R = w.chunk, w.cp
    fpp = w.hq * w.dim * 4  # forward FLOP per visible pair (all query heads)

    # Pass Q: the rank's K/V stay, every rank's Q block visits; then the owner's
    # merge of the R partials it receives (the rank's own partials stand in for them)
    pq = PassQRank(w, rank)
    k = _dev_normal(torch, (2 * c, w.hkv, w.dim), 101)
    v = _dev_normal(torch, (2 * c, w.hkv, w.dim), 102)
    qs = {s: _dev_normal(torch, (2 * c, w.hq, w.dim), 200 + s) for s in range(R)}
    pairs = sum(cpattn.cp_count_pairs(pq.problem(t)) for t in range(R))

    def pass_q(timer):
        parts = pq.forward(k, v, qs.__getitem__, stage=True, timer=timer)
        pq.restore([(o, l) for _, o, l in parts])

    ms, kern, _ = _time_leg(torch, pass_q, steps, warmup, KernelTimer(torch, "fwd"))
    out["pass_q"] = {"workload": f"{w.name} Pass Q rank {rank}", "tflops": round(tflops(pairs * fpp, ms), 2),
                     "kernel_tflops": round(tflops(pairs * fpp, kern), 2), "ms_per_step": round(ms, 4)}
    del qs
    log(f"pass_q: {ms:.3f} ms/step")

    # partial prefill: 96K cached + 32K new tokens over CP=8
    P, N = 3 * w.seq_len // 4, w.seq_len // 4
    pp = PartialPrefillRank(P, N, R, w.hq, w.hkv, w.dim, rank)
    q_new = _dev_normal(torch, (2 * pp.cn, w.hq, w.dim), 301)
    kvs = {s: (_dev_normal(torch, (2 * pp.cc, w.hkv, w.dim), 400 + s), _dev_normal(torch, (2 * pp.cc, w.hkv, w.dim), 500 + s),
               _dev_normal(torch, (2 * pp.cn, w.hkv, w.dim), 600 + s), _dev_normal(torch, (2 * pp.cn, w.hkv, w.dim), 700 + s))
           for s in range(R)}
    pairs = sum(cpattn.cp_count_pairs(p) for t in range(R) for p in pp.problems(t))
    ms, kern, _ = _time_leg(torch, lambda timer: pp.forward(q_new, kvs.__getitem__, stage=True, timer=timer), steps,
                         warmup, KernelTimer(torch, "fwd"))
    out["partial_prefill"] = {"workload": f"Llama-3-8B partial prefill, {P} cached + {N} new tokens, CP={R}, rank {rank}",
                              "tflops": round(tflops(pairs * fpp, ms), 2),
                              "kernel_tflops": round(tflops(pairs * fpp, kern), 2), "ms_per_step": round(ms, 4)}
    del kvs
    log(f"partial_prefill: {ms:.3f} ms/step")

    # USP with all-to-all groups of 2: the device's ring over cp/2 groups with half the heads
    from context_long_attention_amd.ring import RankRing
    from context_long_attention_amd.variants import usp_share
    wu = usp_share(w, 2)
    uq, ukv = make_rank_inputs(torch, wu, rank)
    pairs = sum(RankRing(wu, rank).step_pairs(t) for t in range(wu.cp))
    ms, kern, _ = _time_leg(torch, lambda timer: RankRing(wu, rank).forward(uq, ukv.__getitem__, stage=True, timer=timer),
                         steps, warmup, KernelTimer(torch, "fwd"))
    fpu = wu.hq * wu.dim * 4
    out["usp"] = {"workload": f"{w.name} USP share, all-to-all groups of 2: ring of {wu.cp} ranks, Hq={wu.hq}, "
                              f"Hkv={wu.hkv}, {wu.local} local tokens, rank {rank}",
                  "tflops": round(tflops(pairs * fpu, ms), 2), "kernel_tflops": round(tflops(pairs * fpu, kern), 2),
                  "ms_per_step": round(ms, 4)}
    del uq, ukv
    log(f"usp: {ms:.3f} ms/step")

    # gathered KV (all-gather strategy): the rank's query share against the whole sequence
    q_loc = _dev_normal(torch, (2 * c, w.hq, w.dim), 801)
    k_all = _dev_normal(torch, (w.seq_len, w.hkv, w.dim), 802)
    v_all = _dev_normal(torch, (w.seq_len, w.hkv, w.dim), 803)
    ring_pairs = 2 * R * c * c + c
    ms, _, _ = _time_leg(torch, lambda timer: gathered_forward(w, rank, q_loc, k_all, v_all), steps, warmup)
    out["all_gather"] = {"workload": f"{w.name} gathered KV, rank {rank}", "tflops": round(tflops(ring_pairs * fpp, ms), 2),
                         "ms_per_step": round(ms, 4)}
    log(f"all_gather: {ms:.3f} ms/step")

    # head-sharded (all-to-all strategy): the whole sequence for Hq/R and Hkv/R heads
    hq_d, hkv_d = w.hq // R, max(1, w.hkv // R)
    q_h = _dev_normal(torch, (w.seq_len, hq_d, w.dim), 901)
    k_h = _dev_normal(torch, (w.seq_len, hkv_d, w.dim), 902)
    v_h = _dev_normal(torch, (w.seq_len, hkv_d, w.dim), 903)
    pairs = w.seq_len * (w.seq_len + 1) // 2
    ms, _, _ = _time_leg(torch, lambda timer: head_sharded_forward(q_h, k_h, v_h, w.scale), steps, warmup)
    out["ulysses"] = {"workload": f"{w.name} head-sharded, {hq_d} query heads / {hkv_d} KV head over {w.seq_len} tokens",
                      "tflops": round(tflops(pairs * hq_d * w.dim * 4, ms), 2), "ms_per_step": round(ms, 4)}
    log(f"ulysses: {ms:.3f} ms/step")
    return out


def measure_window(torch, w, rank, steps, warmup):
    """A sliding-window layer (the pages' window layers of models such as Gemma):
    forward and backward ring of one rank, where only the blocks with visible
    pairs (the rank's own and its neighbours') are received and computed."""
    from context_long_attention_amd import cpattn, inputs
    from context_long_attention_amd.ring import RankRing
    q, kv = make_rank_inputs(torch, w, rank)
    c = w.chunk
    pos = cpattn.cp_partition_zigzag(w.seq_len, w.cp, rank)
    d_o = _dev_bf16(torch, inputs.chunks_normal(inputs.SEED_DO, [int(pos[0]) // c, int(pos[c]) // c], c, w.hq,
                                                w.dim))
    ring = RankRing(w, rank)
    pairs = sum(ring.step_pairs(t) for t in range(w.cp))
    live = [t for t in range(w.cp) if t == 0 or ring.source_live(ring.schedule()[t])]
    fwd_timer, bwd_timer = KernelTimer(torch, "fwd"), KernelTimer(torch, "bwd")

    def timer(step, what, stream):
        fwd_timer(step, what, stream)
        bwd_timer(step, what, stream)

    def one_step(tm):
        r = RankRing(w, rank)
        o, lse, _ = r.forward(q, kv.__getitem__, stage=True, timer=tm)
        r.backward(q, d_o, o, lse, kv.__getitem__, stage=True, keep_steps=False, timer=tm)

    for _ in range(warmup):
        one_step(None)
    torch.cuda.synchronize()
    fwd_timer.enabled = bwd_timer.enabled = True
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    marks[0].record()
    for i in range(steps):
        one_step(timer)
        marks[i + 1].record()
    torch.cuda.synchronize()
    reps = [marks[i].elapsed_time(marks[i + 1]) for i in range(steps)]
    ms = float(np.median(reps))
    f_fwd, f_bwd = pairs * w.hq * w.dim * 4, pairs * w.hq * w.dim * 10
    log(f"{w.name}: {ms:.3f} ms/step (median of {steps}), live steps {live}")
    return {"workload": f"{w.name}: window {w.window} over S={w.seq_len} at CP={w.cp}, rank {rank}, fwd+bwd",
            "window": w.window, "live_steps": live, "pairs_per_head": pairs,
            "tflops": round(tflops(f_fwd + f_bwd, ms), 2), "ms_per_step": round(ms, 4), "timing": rep_stats(reps),
            "fwd_kernel_tflops": round(tflops(f_fwd, fwd_timer.total_ms() / steps), 2),
            "bwd_kernel_tflops": round(tflops(f_bwd, bwd_timer.total_ms() / steps), 2)}


def measure_large(torch, w, rank, steps, warmup):
    """The Llama-3-405B prefill share: rank 0's whole forward ring (16 steps of
    64K-token KV blocks), with inputs drawn on the device (only shapes matter for
    timing; the parity tests use the seeded recipe)."""
    from context_long_attention_amd.ring import RankRing
    q = _dev_normal(torch, (w.local, w.hq, w.dim), 1001)
    kv = {s: (_dev_normal(torch, (w.local, w.hkv, w.dim), 1100 + s), _dev_normal(torch, (w.local, w.hkv, w.dim), 1200 + s))
          for s in range(w.cp)}
    ring = RankRing(w, rank)
    flops = sum(ring.step_pairs(t) for t in range(w.cp)) * w.hq * w.dim * 4
    timer = KernelTimer(torch, "fwd")

    def one(tm):
        RankRing(w, rank).forward(q, kv.__getitem__, stage=True, timer=tm)

    ms, kern, reps = _time_leg(torch, one, steps, warmup, timer)
    med = float(np.median(reps))
    log(f"{w.name}: {med:.1f} ms per ring (median of {steps})")
    return {"workload": f"{w.name}: Hq={w.hq} Hkv={w.hkv} D={w.dim}, rank {rank} of S={w.seq_len} at CP={w.cp}, "
                        f"{w.cp} ring steps of {w.local}-token KV blocks, fwd",
            "tflops": round(tflops(flops, med), 2), "pct_bf16_peak": round(100 * tflops(flops, med) / BF16_PEAK_TFLOPS, 2),
            "kernel_tflops": round(tflops(flops, kern), 2), "ms_per_ring": round(med, 2), "flops": flops,
            "timing": rep_stats(reps)}


def measure_packed(torch, w, steps, warmup):
    """The packed-document training workload over all of its ranks: every rank's
    forward and backward ring over the seeded document layout (block-diagonal
    causal masks, fully masked tiles and blocks skipped).  Per-rank work varies
    widely, so the leg times all ranks back to back; FLOPs count only the visible
    (document-causal) pairs.  Inputs are drawn on the device."""
    from context_long_attention_amd.ring import RankRing
    cu = w.cu_seqlens()
    q = _dev_normal(torch, (w.local, w.hq, w.dim), 2001)
    d_o = _dev_normal(torch, (w.local, w.hq, w.dim), 2002)
    kv = {s: (_dev_normal(torch, (w.local, w.hkv, w.dim), 2100 + s), _dev_normal(torch, (w.local, w.hkv, w.dim), 2200 + s))
          for s in range(w.cp)}
    rings = [RankRing(w, r, cu) for r in range(w.cp)]
    pairs = sum(ring.step_pairs(t) for ring in rings for t in range(w.cp))
    fwd_t, bwd_t = KernelTimer(torch, "fwd"), KernelTimer(torch, "bwd")

    def timer(step, what, stream):
        fwd_t(step, what, stream)
        bwd_t(step, what, stream)

    def one(tm):
        for ring in rings:
            o, lse, _ = ring.forward(q, kv.__getitem__, stage=True, timer=tm)
            ring.backward(q, d_o, o, lse, kv.__getitem__, stage=True, keep_steps=False, timer=tm)

    ms, _, reps = _time_leg(torch, one, steps, warmup, None)
    med = float(np.median(reps))
    fwd_t.enabled = bwd_t.enabled = True
    one(timer)
    torch.cuda.synchronize()
    f_fwd, f_bwd = pairs * w.hq * w.dim * 4, pairs * w.hq * w.dim * 10
    log(f"{w.name}: {med:.1f} ms for all {w.cp} ranks (median of {steps})")
    return {"workload": f"{w.name}: S={w.seq_len} at CP={w.cp}, {len(cu) - 1} documents, every rank's fwd+bwd ring",
            "pairs_per_head": pairs, "visible_fraction_of_causal": round(pairs / (w.seq_len * (w.seq_len + 1) / 2), 4),
            "tflops": round(tflops(f_fwd + f_bwd, med), 2), "ms_all_ranks": round(med, 2), "timing": rep_stats(reps),
            "fwd_kernel_tflops": round(tflops(f_fwd, fwd_t.total_ms()), 2),
            "bwd_kernel_tflops": round(tflops(f_bwd, bwd_t.total_ms()), 2)}


def tflops(flops, ms):
    return flops / (ms * 1e-3) / 1e12


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="llama3_8b_fwd")
    ap.add_argument("--bwd-workload", default="llama3_8b_fwdbwd")
    ap.add_argument("--rank", type=int, default=0)
    ap.add_argument("--cpu-heads", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-bwd", action="store_true")
    ap.add_argument("--no-variants", action="store_true", help="skip the Pass Q / prefill / gathered legs")
    ap.add_argument("--no-window", action="store_true", help="skip the sliding-window layer leg")
    ap.add_argument("--no-large", action="store_true", help="skip the Llama-3-405B prefill leg")
    ap.add_argument("--no-packed", action="store_true", help="skip the packed-document training leg")
    ap.add_argument("--no-gemm-reference", action="store_true",
                    help="skip the same-box vendor GEMM reference (context for the power-capped clock)")
    ap.add_argument("--window-workload", default="llama3_8b_window4k")
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
        "timing": dict(rep_stats(fwd["rep_ms"]),
                       tflops_median=round(tflops(fwd["flops_fwd"], float(np.median(fwd["rep_ms"]))), 2),
                       ring_step_ms=[round(x, 4) for x in fwd["fwd_step_ms"]]),
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
        fb = measure(torch, wb, args.rank, 10, 1, backward=True)
        total = fb["flops_fwd"] + fb["flops_bwd"]
        med = float(np.median(fb["rep_ms"]))
        record["fwd_bwd"] = {
            "workload": wb.name, "seq_len": wb.seq_len, "cp": wb.cp, "ring_steps": wb.cp,
            "tflops": round(tflops(total, med), 2),
            "pct_bf16_peak": round(100 * tflops(total, med) / BF16_PEAK_TFLOPS, 2),
            "ms_per_step": round(med, 4),
            "timing": dict(rep_stats(fb["rep_ms"]), fwd_ring_step_ms=[round(x, 4) for x in fb["fwd_step_ms"]],
                           bwd_ring_step_ms=[round(x, 4) for x in fb["bwd_step_ms"]]),
            "fwd_kernel_tflops": round(tflops(fb["flops_fwd"], fb["fwd_kernel_ms"]), 2),
            "bwd_kernel_tflops": round(tflops(fb["flops_bwd"], fb["bwd_kernel_ms"]), 2),
            "bwd_kernel_ms_per_step": round(fb["bwd_kernel_ms"], 4),
            "clocks": fb["clocks"],
        }
    if not args.no_variants:
        record["variants"] = measure_variants(torch, w, args.rank, max(1, args.steps // 2), 1)
    if not args.no_large:
        wl = inputs.WORKLOADS["llama3_405b_fwd"]
        record["llama3_405b_fwd"] = measure_large(torch, wl, args.rank, 3, 1)
        if not args.no_cpu_baseline:
            log("timing the float64 oracle on a sample of the Llama-3-405B share (extrapolated baseline)")
            cb = cpu_baseline_extrapolated(wl, args.rank)
            cb["seconds_for_share"] = round(record["llama3_405b_fwd"]["flops"] / (cb["value"] * 1e12), 1)
            record["llama3_405b_fwd"]["cpu_baseline"] = cb
    if not args.no_packed:
        record["llama3_8b_packed"] = measure_packed(torch, inputs.WORKLOADS["llama3_8b_packed"], 10, 1)
    if not args.no_window:
        record["sliding_window"] = measure_window(torch, inputs.WORKLOADS[args.window_workload], args.rank, 10, 1)
    if not args.no_gemm_reference:
        record["gemm_reference"] = gemm_reference(torch)
        record["gemm_reference"]["attention_over_gemm"] = round(value / record["gemm_reference"]["tflops"], 3)
    if not args.no_cpu_baseline:
        log("timing the float64 oracle on the host (cpu_baseline)")
        record["cpu_baseline"] = cpu_baseline(w, args.rank, args.cpu_heads, fwd["final"])
    print(json.dumps(record), flush=True)


if __name__ == "__main__":
    main()
