"""Host ring scheduler: replays one rank's Pass-KV ring steps on one GPU.

Pass KV keeps the rank's queries in place while KV blocks travel one hop per
step around the ring; each step runs the attention kernel on the local queries
and the block just received, and the partial outputs are merged ("Context
Parallelism for Scalable Million-Token Inference", section "Ring Attention
Algorithms"; "Announcing Long-Context Training on TPUs with MaxText Context
Parallelism", section "Context Parallelism in MaxText", P2P paragraph).

On one GPU there is no neighbour to receive from: every source rank's block
already sits in HBM, and a copy on a side stream into a double-buffered
receive buffer stands in for the transfer that would run under the kernel.
All arithmetic runs in libcpattn (``cpattn``); torch only provides device
memory, streams and events.
"""
from __future__ import annotations

import numpy as np
import torch

from . import cpattn
from .inputs import Workload


class RingScheduleError(RuntimeError):
    """A ring schedule that does not visit every source rank exactly once."""


def check_schedule(cp_size: int, sources) -> None:
    """Reject a schedule that drops or repeats a source before anything is merged."""
    seen = sorted(int(s) for s in sources)
    if seen != list(range(cp_size)):
        raise RingScheduleError(f"ring schedule visits sources {seen}, expected each of 0..{cp_size - 1} once")


class RankRing:
    """One rank's share of a context-parallel sequence of ``w.seq_len`` tokens."""

    def __init__(self, w: Workload, rank: int, cu_seqlens: np.ndarray | None = None, device="cuda"):
        self.w = w
        self.rank = rank
        self.R = w.cp
        self.c = w.chunk
        self.device = torch.device(device)
        self.pos = cpattn.cp_partition_zigzag(w.seq_len, w.cp, rank)
        self.packed = cu_seqlens is not None
        self._live_pairs = {}
        self._kv_split = {}
        self._ws = None
        if self.packed:
            self.cu_host = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
            self.cu_dev = torch.from_numpy(self.cu_host).to(self.device)
            self.n_docs = len(self.cu_host) - 1
        else:
            self.cu_host = None
            self.cu_dev = None
            self.n_docs = 0

    # ------------------------------------------------------------- problems
    def chunks_of(self, r: int) -> tuple[int, int]:
        pos = cpattn.cp_partition_zigzag(self.w.seq_len, self.R, r)
        return int(pos[0]) // self.c, int(pos[self.c]) // self.c

    def schedule(self) -> list[int]:
        return [cpattn.cp_ring_source(self.R, self.rank, t) for t in range(self.R)]

    def problem(self, step: int, source: int | None = None, host_docs: bool = False) -> cpattn.cp_attn_problem:
        w, c = self.w, self.c
        src = cpattn.cp_ring_source(self.R, self.rank, step) if source is None else source
        qa, qb = self.chunks_of(self.rank)
        ka, kb = self.chunks_of(src)
        masks = self.masks_of_source(src)
        cu_ptr, n_docs = None, 0
        if self.packed:
            cu_ptr = self.cu_host.ctypes.data if host_docs else self.cu_dev.data_ptr()
            n_docs = self.n_docs
        return cpattn.make_problem(w.hq, w.hkv, w.dim, w.scale, 2 * c, 2 * c,
                                   [(0, qa * c, c), (c, qb * c, c)], [(0, ka * c, c), (c, kb * c, c)],
                                   masks, cu_ptr, n_docs, w.window)

    def masks_of_source(self, src: int) -> list[list[int]]:
        """Chunk-pair classes of the local queries against ``src``'s block (the
        classes of the ring step at which that block arrives)."""
        step = (self.rank - src) % self.R
        return cpattn.cp_step_masks_window(self.w.seq_len, self.R, self.rank, step, self.packed, self.w.window)

    def source_live(self, src: int) -> bool:
        """Whether the local queries can see anything of ``src``'s block.  With a
        sliding window no longer than a chunk only the rank's own block and its
        ring neighbours' are live: the short exchange between neighbouring chips
        of window layers ("Announcing Long-Context Training ...", closing section).
        With packed documents the chunk classes cannot tell, so the visible pairs
        are counted on the host (once per source): a block that only other
        documents' queries could see is neither received nor computed."""
        if not any(m != cpattn.CP_MASK_SKIP for row in self.masks_of_source(src) for m in row):
            return False
        if not self.packed:
            return True
        if src not in self._live_pairs:
            step = (self.rank - src) % self.R
            self._live_pairs[src] = cpattn.cp_count_pairs(self.problem(step, src, host_docs=True))
        return self._live_pairs[src] > 0

    def kv_split(self, src: int) -> int:
        """dK/dV work split of the backward step on ``src``'s block, chosen by the
        library on the host (with the host copy of the documents, which the device
        step cannot read), so that the ring can size the workspace it needs."""
        if src not in self._kv_split:
            step = (self.rank - src) % self.R
            n_cu = torch.cuda.get_device_properties(self.device).multi_processor_count
            self._kv_split[src] = cpattn.cp_bwd_kv_split(self.problem(step, src, host_docs=True), n_cu)
        return self._kv_split[src]

    def workspace(self, p: cpattn.cp_attn_problem):
        """Device workspace for the backward step p (None when its split needs
        none); one buffer per ring, grown when a step needs more."""
        if p.kv_split <= 1:
            return None
        need = cpattn.cp_bwd_workspace_size(p, p.kv_split)
        if self._ws is None or self._ws.numel() < need:
            self._ws = torch.empty(need, dtype=torch.uint8, device=self.device)
        return self._ws

    def step_pairs(self, step: int) -> int:
        """Visible (query, key) pairs per query head at ``step`` (host count)."""
        return cpattn.cp_count_pairs(self.problem(step, host_docs=True))

    # ------------------------------------------------------------- forward
    def forward(self, q, kv_of_source, stage: bool = True, keep_steps: bool = False, schedule=None,
                timer=None, fused: bool = True, start: int = 0, stop: int | None = None, state=None):
        """Run the rank's forward ring.

        q: device bf16 [2c, Hq, D]; kv_of_source(src) -> (k, v) device bf16 [2c, Hkv, D].
        Returns (O fp32 [2c, Hq, D], LSE fp32 [Hq, 2c], per-step partials if keep_steps).
        ``timer`` (optional) is called as timer(step, "fwd_begin"/"fwd_end", stream).
        fused: step 0 writes the accumulator and later steps merge into it inside the
        kernel (cp_attn_fwd_step_merge); otherwise every step writes its partial and
        cp_merge_partials folds it in (always so when keep_steps asks for the partials).

        start, stop, state: run only ring steps start .. stop - 1.  The merge is
        associative ("Context Parallelism for Scalable Million-Token Inference",
        section "Ring Attention Algorithms"), so the running (O, LSE) after any
        step is a complete ring state: ``state`` = (O, LSE) device fp32 tensors
        holding the merge of steps 0 .. start - 1 (required when start > 0) are
        merged into in place and returned, and the ring continues as if it had
        never stopped.
        """
        w = self.w
        rows = 2 * self.c
        sched = self.schedule() if schedule is None else list(schedule)
        check_schedule(self.R, sched)
        stop = _step_range(start, stop, len(sched), state, "(O, LSE)")
        dev = self.device
        fused = fused and not keep_steps
        steps = []
        compute = torch.cuda.current_stream(dev)
        if state is not None:
            o_acc, lse_acc = state
            _check_state(o_acc, (rows, w.hq, w.dim), dev, "O")
            _check_state(lse_acc, (w.hq, rows), dev, "LSE")
        elif fused:
            # the query segments cover every local row, so step 0 writes all of them
            o_acc = torch.empty((rows, w.hq, w.dim), dtype=torch.float32, device=dev)
            lse_acc = torch.empty((w.hq, rows), dtype=torch.float32, device=dev)
        else:
            o_acc = torch.zeros((rows, w.hq, w.dim), dtype=torch.float32, device=dev)
            lse_acc = torch.full((w.hq, rows), float("-inf"), dtype=torch.float32, device=dev)
        if not fused:
            o_t = torch.empty_like(o_acc)
            lse_t = torch.empty_like(lse_acc)
        # steps with no visible pair are neither received nor computed (their
        # partial is the merge identity); step 0 (the diagonal) is always live
        live = [t for t in range(start, stop) if keep_steps or t == 0 or self.source_live(sched[t])]
        feeder = _Feeder(kv_of_source, [sched[t] for t in live], stage, dev, local=self.rank)
        for i, t in enumerate(live):
            src = sched[t]
            k, v = feeder.get(i, compute)
            p = self.problem(t, src)
            if timer:
                timer(t, "fwd_begin", compute)
            if not fused:
                cpattn.cp_attn_fwd_step(p, q, k, v, o_t, lse_t, stream=compute)
            elif t == 0:
                cpattn.cp_attn_fwd_step(p, q, k, v, o_acc, lse_acc, stream=compute)
            else:
                cpattn.cp_attn_fwd_step_merge(p, q, k, v, o_acc, lse_acc, stream=compute)
            if timer:
                timer(t, "fwd_end", compute)
            feeder.release(i, compute)
            if not fused:
                if keep_steps:
                    steps.append((o_t.clone(), lse_t.clone()))
                cpattn.cp_merge_partials(o_acc, lse_acc, o_t, lse_t, rows, w.hq, w.dim, stream=compute)
        return o_acc, lse_acc, steps

    # ------------------------------------------------------------- backward
    def backward(self, q, d_o, o, lse, kv_of_source, stage: bool = True, schedule=None, keep_steps=True,
                 timer=None, start: int = 0, stop: int | None = None, state=None):
        """Run the rank's backward ring from the final O and LSE.

        Returns (dQ fp32 [2c, Hq, D], per-step list of (source, dK_t, dV_t) fp32 [2c, Hkv, D]).
        With keep_steps=False only the last step's dK/dV buffers are kept (benchmarking).

        start, stop, state: run only ring steps start .. stop - 1, as in forward.
        ``state`` is the dQ accumulator (device fp32 [2c, Hq, D]) summed over steps
        0 .. start - 1 (required when start > 0); it is added to in place and
        returned, and the per-step list covers the steps run.  Delta is recomputed
        from the final O and dO on every call (the same bits each time).
        """
        w = self.w
        rows = 2 * self.c
        sched = self.schedule() if schedule is None else list(schedule)
        check_schedule(self.R, sched)
        stop = _step_range(start, stop, len(sched), state, "dQ")
        dev = self.device
        compute = torch.cuda.current_stream(dev)
        delta = torch.empty((w.hq, rows), dtype=torch.float32, device=dev)
        cpattn.cp_attn_bwd_prep(d_o, o, delta, rows, w.hq, w.dim, stream=compute)
        if state is not None:
            _check_state(state, (rows, w.hq, w.dim), dev, "dQ")
            dq = state
        else:
            dq = torch.zeros((rows, w.hq, w.dim), dtype=torch.float32, device=dev)
        out = []
        # as in the forward: steps with no visible pair are skipped (their dK/dV
        # are zero; with keep_steps they are returned as zeros)
        live = [t for t in range(start, stop) if t == 0 or self.source_live(sched[t])]
        feeder = _Feeder(kv_of_source, [sched[t] for t in live], stage, dev, local=self.rank)
        dk = dv = None
        for t in range(start, stop):
            src = sched[t]
            if t not in live:
                if keep_steps:
                    z = torch.zeros((rows, w.hkv, w.dim), dtype=torch.float32, device=dev)
                    out.append((src, z, torch.zeros_like(z)))
                continue
            i = live.index(t)
            k, v = feeder.get(i, compute)
            if keep_steps or dk is None:
                dk = torch.empty((rows, w.hkv, w.dim), dtype=torch.float32, device=dev)
                dv = torch.empty_like(dk)
            p = self.problem(t, src)
            p.kv_split = self.kv_split(src)
            ws = self.workspace(p)
            if timer:
                timer(t, "bwd_begin", compute)
            cpattn.cp_attn_bwd_step(p, q, k, v, d_o, lse, delta, dq, dk, dv, workspace=ws, stream=compute)
            if timer:
                timer(t, "bwd_end", compute)
            feeder.release(i, compute)
            out.append((src, dk, dv))
        return dq, out


def _step_range(start, stop, n, state, what):
    """The end of a ring run over steps start .. stop - 1 (stop None: to the end),
    checked against the schedule's length and the resume state."""
    stop = n if stop is None else stop
    if not 0 <= start <= stop <= n:
        raise ValueError(f"ring steps {start} .. {stop - 1} outside 0 .. {n - 1}")
    if (state is None) != (start == 0):
        raise ValueError(f"a ring resumed after step 0 needs the {what} state of the steps before it, "
                         "and one started at step 0 takes none")
    return stop


def _check_state(x, shape, dev, what):
    """A resume state tensor must be contiguous fp32 of the accumulator's shape on the ring's device."""
    index = dev.index if dev.index is not None else torch.cuda.current_device()
    if (tuple(x.shape) != tuple(shape) or x.dtype != torch.float32 or not x.is_cuda or x.device.index != index
            or not x.is_contiguous()):
        raise ValueError(f"ring state {what} must be a contiguous fp32 tensor of shape {tuple(shape)} on the device")


_SIDE_STREAMS = {}


def _side_stream(dev):
    """One receive stream per device for the whole process.  A fresh stream per
    ring would be taken round-robin from torch's pool and could share a hardware
    queue with the compute stream, serialising the copies with the kernels."""
    key = torch.device(dev).index if torch.device(dev).index is not None else torch.cuda.current_device()
    if key not in _SIDE_STREAMS:
        _SIDE_STREAMS[key] = torch.cuda.Stream(torch.device("cuda", key))
    return _SIDE_STREAMS[key]


class _Feeder:
    """Supplies the block of each step (a tuple of tensors: (K, V) for Pass KV,
    (Q,) for Pass Q), optionally through a double-buffered receive buffer filled
    on a side stream (the stand-in for the ring transfer).  ``pack`` (optional)
    groups the source's tensors: each group lands row-wise concatenated in one
    buffer, e.g. [(0, 2), (1, 3)] turns (K_a, V_a, K_b, V_b) into
    ([K_a; K_b], [V_a; V_b]).  ``local`` (optional) is the source whose block
    the device already holds (the rank itself): it is read in place, as a ring
    reads its own block without a transfer (only without ``pack``)."""

    def __init__(self, block_of_source, sched, stage, dev, pack=None, local=None):
        self.block_of_source = block_of_source
        self.sched = sched
        self.stage = stage
        self.dev = dev
        self.pack = pack
        self.local = local if pack is None else None
        if stage:
            self.side = _side_stream(dev)
            # The receive buffers come from torch's caching allocator, which may hand
            # back blocks whose previous users are still queued on the compute stream:
            # the first copy must not start before that earlier work.
            self.side.wait_stream(torch.cuda.current_stream(dev))
            self.buf = [None, None]
            self.ready = [torch.cuda.Event(), torch.cuda.Event()]
            self.free = [torch.cuda.Event(), torch.cuda.Event()]
            self.free_recorded = [False, False]
            if self.sched:
                self._issue(0)

    def _groups(self, src):
        return [(i,) for i in range(len(src))] if self.pack is None else self.pack

    def _in_place(self, t):
        return self.local is not None and self.sched[t] == self.local

    def _issue(self, t):
        if self._in_place(t):
            return
        src = tuple(self.block_of_source(self.sched[t]))
        groups = self._groups(src)
        slot = t % 2
        if self.buf[slot] is None:
            bufs = tuple(torch.empty((sum(src[i].shape[0] for i in g), *src[g[0]].shape[1:]), dtype=src[g[0]].dtype,
                                     device=src[g[0]].device) for g in groups)
            for b in bufs:
                # written on the side stream: keep the blocks until its work is done
                b.record_stream(self.side)
            self.buf[slot] = bufs
        bufs = self.buf[slot]
        with torch.cuda.stream(self.side):
            if self.free_recorded[slot]:
                self.side.wait_event(self.free[slot])
            for b, g in zip(bufs, groups):
                row = 0
                for i in g:
                    n = src[i].shape[0]
                    b[row:row + n].copy_(src[i], non_blocking=True)
                    row += n
            self.ready[slot].record(self.side)

    def get(self, t, compute):
        if not self.stage or self._in_place(t):
            if self.stage and t + 1 < len(self.sched):
                self._issue(t + 1)
            src = tuple(self.block_of_source(self.sched[t]))
            if self.pack is None:
                return src
            return tuple(torch.cat([src[i] for i in g], dim=0) for g in self.pack)
        slot = t % 2
        compute.wait_event(self.ready[slot])
        if t + 1 < len(self.sched):
            self._issue(t + 1)
        return self.buf[slot]

    def release(self, t, compute):
        if self.stage and not self._in_place(t):
            slot = t % 2
            self.free[slot].record(compute)
            self.free_recorded[slot] = True
