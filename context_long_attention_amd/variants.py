"""Host schedulers for the ring variants beside Pass KV, on the same C-ABI calls
(``cp_attn_fwd_step``, ``cp_attn_fwd_step_merge``, ``cp_merge_partials``).

* Pass Q -- "Context Parallelism for Scalable Million-Token Inference", section
  "Ring Attention Algorithms": K/V stay on their rank while the Q blocks travel
  around the ring; each rank computes, per step, the partial attention of the
  visiting queries over its own keys; after the rotation the partials are
  permuted and sent (all-to-all) to their owners, who merge them.  One GPU
  replays one rank: its R partials, and an owner's merge of the R partials it
  receives (host indexing stands in for the all-to-all).
* Partial prefill -- same page, sections "Attention Compute Patterns in
  Multi-Turn Chat" and "Load Balancing in CP": new tokens attend to every cached
  token and causally to each other; both the cached prefix and the new tokens
  are split in 2R chunks, rank r holding chunks r and 2R-1-r of each, and the
  ring passes both parts of every rank's KV.
* USP (all-to-all inside groups of U devices, a ring across the groups) -- same
  MaxText section: after the all-to-all a device holds Hq/U query heads and
  Hkv/U KV heads of its group's pooled tokens, and the ring over the R/U groups
  passes blocks U times larger.  Its attention work is the Pass-KV ring of
  ``usp_share`` (``RankRing`` unchanged).
* Gathered KV and head-sharded attention -- "Announcing Long-Context Training on
  TPUs with MaxText Context Parallelism", section "Context Parallelism in
  MaxText": the per-device work of the all-gather strategy (the rank's query
  share against the whole gathered sequence) and of the all-to-all strategy
  (full-sequence attention for a subset of heads) are single step calls.

All arithmetic runs in libcpattn; torch only provides memory, streams and events.
"""
from __future__ import annotations

import dataclasses

import torch

from . import cpattn
from .inputs import Workload
from .ring import _Feeder, check_schedule

# largest KV segment (bytes of one KV tensor) one call may address
_SPAN_LIMIT = (1 << 30) - 1


def usp_share(w: Workload, u: int) -> Workload:
    """One device's attention work under USP with all-to-all groups of ``u``
    devices: a Pass-KV ring of w.cp / u ranks over the same sequence, with
    w.hq / u query heads and w.hkv / u KV heads (u must divide w.cp, w.hq and
    w.hkv, so each device keeps whole GQA groups)."""
    if u < 1 or w.cp % u or w.hq % u or w.hkv % u:
        raise ValueError(f"USP group size {u} must divide cp={w.cp}, hq={w.hq} and hkv={w.hkv}")
    return dataclasses.replace(w, name=f"{w.name}_usp{u}", cp=w.cp // u, hq=w.hq // u, hkv=w.hkv // u)


class PassQRank:
    """One rank of Pass Q.  The rank's K/V (its two zigzag chunks) stay; at step
    t the Q block of rank ``cp_ring_source(R, rank, t)`` is held."""

    def __init__(self, w: Workload, rank: int, cu_seqlens=None, device="cuda"):
        import numpy as np
        self.w = w
        self.rank = rank
        self.R = w.cp
        self.c = w.chunk
        self.device = torch.device(device)
        self.packed = cu_seqlens is not None
        if self.packed:
            self.cu_host = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
            self.cu_dev = torch.from_numpy(self.cu_host).to(self.device) if self.device.type == "cuda" else None
            self.n_docs = len(self.cu_host) - 1

    def chunks_of(self, r: int):
        pos = cpattn.cp_partition_zigzag(self.w.seq_len, self.R, r)
        return int(pos[0]) // self.c, int(pos[self.c]) // self.c

    def schedule(self):
        return [cpattn.cp_ring_source(self.R, self.rank, t) for t in range(self.R)]

    def problem(self, step: int, source=None, host_docs: bool = False) -> cpattn.cp_attn_problem:
        """Queries of the visiting rank against this rank's keys.  The chunk classes
        are those of the visiting rank at the Pass KV step where it holds this
        rank's block."""
        w, c, R = self.w, self.c, self.R
        s = cpattn.cp_ring_source(R, self.rank, step) if source is None else source
        qa, qb = self.chunks_of(s)
        ka, kb = self.chunks_of(self.rank)
        masks = cpattn.cp_step_masks(R, s, (s - self.rank) % R, self.packed)
        cu_ptr, n_docs = None, 0
        if self.packed:
            cu_ptr = self.cu_host.ctypes.data if host_docs else self.cu_dev.data_ptr()
            n_docs = self.n_docs
        return cpattn.make_problem(w.hq, w.hkv, w.dim, w.scale, 2 * c, 2 * c, [(0, qa * c, c), (c, qb * c, c)],
                                   [(0, ka * c, c), (c, kb * c, c)], masks, cu_ptr, n_docs)

    def forward(self, k, v, q_of_source, stage: bool = True, timer=None):
        """The rank's R partials, in step order: [(owner, O_t, LSE_t)] with O_t fp32
        [2c, Hq, D] and LSE_t fp32 [Hq, 2c] over the owner's local rows."""
        w, rows = self.w, 2 * self.c
        sched = self.schedule()
        check_schedule(self.R, sched)
        compute = torch.cuda.current_stream(self.device)
        feeder = _Feeder(lambda s: (q_of_source(s),), sched, stage, self.device, local=self.rank)
        out = []
        for t, s in enumerate(sched):
            (q,) = feeder.get(t, compute)
            o_t = torch.empty((rows, w.hq, w.dim), dtype=torch.float32, device=self.device)
            l_t = torch.empty((w.hq, rows), dtype=torch.float32, device=self.device)
            if timer:
                timer(t, "fwd_begin", compute)
            cpattn.cp_attn_fwd_step(self.problem(t, s), q, k, v, o_t, l_t, stream=compute)
            if timer:
                timer(t, "fwd_end", compute)
            feeder.release(t, compute)
            out.append((s, o_t, l_t))
        return out

    def restore(self, received):
        """The owner's side of the permutation and all-to-all: merge the partials
        that every rank computed for this owner's rows (``received``: list of
        (O_t, LSE_t)).  Returns the owner's (O, LSE)."""
        w, rows = self.w, 2 * self.c
        o = torch.empty((rows, w.hq, w.dim), dtype=torch.float32, device=self.device)
        lse = torch.empty((w.hq, rows), dtype=torch.float32, device=self.device)
        cpattn.cp_merge_partials_n(o, lse, [x[0] for x in received], [x[1] for x in received], rows, w.hq, w.dim)
        return o, lse


class PartialPrefillRank:
    """One rank of Pass KV over a partial prefill: ``n_cached`` cached tokens at
    positions [0, n_cached) followed by ``n_new`` new tokens.  The rank's queries
    are its share of the new tokens; each visiting rank brings its cached share
    and its new share of K/V."""

    def __init__(self, n_cached: int, n_new: int, cp: int, hq: int, hkv: int, dim: int, rank: int, device="cuda"):
        if n_cached % (2 * cp) or n_new % (2 * cp):
            raise ValueError("the cached and new token counts must each split into 2*cp chunks")
        self.P, self.N, self.R = n_cached, n_new, cp
        self.hq, self.hkv, self.dim, self.rank = hq, hkv, dim, rank
        self.scale = dim ** -0.5
        self.cc, self.cn = n_cached // (2 * cp), n_new // (2 * cp)
        self.device = torch.device(device)

    def _chunks(self, n, r):
        c = n // (2 * self.R)
        if c == 0:
            return 0, 2 * self.R - 1
        pos = cpattn.cp_partition_zigzag(n, self.R, r)
        return int(pos[0]) // c, int(pos[c]) // c

    def schedule(self):
        return [cpattn.cp_ring_source(self.R, self.rank, t) for t in range(self.R)]

    def problems(self, step: int):
        """The step's calls on the visiting rank's receive buffer, which holds its
        cached share (rows [0, 2 cc)) and then its new share (rows [2 cc, 2 cc + 2 cn)).
        Every cached key is visible to every new token (FULL); the new tokens follow
        the causal chunk classes of the Pass KV step.  Off the diagonal step those
        classes are FULL or SKIP, so one call covers the step: the cached share as one
        FULL segment and the visible new chunks as the other (a segment whose pairs are
        all FULL or SKIP may span several position ranges).  The diagonal step takes
        two calls."""
        R, cc, cn, P = self.R, self.cc, self.cn, self.P
        s = cpattn.cp_ring_source(R, self.rank, step)
        qa, qb = self._chunks(self.N, self.rank)
        q_seg = [(0, P + qa * cn, cn), (cn, P + qb * cn, cn)]
        ca, cb = self._chunks(P, s)
        na, nb = self._chunks(self.N, s)
        F, S_ = cpattn.CP_MASK_FULL, cpattn.CP_MASK_SKIP
        rows = 2 * cc + 2 * cn
        mk = lambda kv_seg, masks: cpattn.make_problem(self.hq, self.hkv, self.dim, self.scale, 2 * cn, rows, q_seg,
                                                        kv_seg, masks)
        m = cpattn.cp_step_masks(R, self.rank, step, False)  # (query chunk, new chunk) classes
        new_segs = [(2 * cc, P + na * cn, cn), (2 * cc + cn, P + nb * cn, cn)]
        cached_one = (0, ca * cc, 2 * cc)  # FULL only: its position is never read
        if any(c not in (F, S_) for row in m for c in row):
            return [mk([(0, ca * cc, cc), (cc, cb * cc, cc)], [[F, F], [F, F]]), mk(new_segs, m)]
        live = [j for j in range(2) if any(m[i][j] != S_ for i in range(2))]
        if not live:
            return [mk([cached_one], [[F, S_], [F, S_]])]
        if len(live) == 1:
            j = live[0]
            return [mk([cached_one, new_segs[j]], [[F, m[0][j]], [F, m[1][j]]])]
        if all(m[i][0] == m[i][1] for i in range(2)):
            return [mk([cached_one, (2 * cc, P + na * cn, 2 * cn)], [[F, m[0][0]], [F, m[1][0]]])]
        return [mk([(0, ca * cc, cc), (cc, cb * cc, cc)], [[F, F], [F, F]]), mk(new_segs, m)]

    def forward(self, q_new, kv_of_source, stage: bool = True, timer=None):
        """q_new: device bf16 [2*cn, Hq, D]; kv_of_source(s) -> (k_cached, v_cached,
        k_new, v_new) with [2*cc or 2*cn, Hkv, D], received into one buffer per
        tensor kind (cached rows, then new rows).  Returns merged (O, LSE)."""
        rows = 2 * self.cn
        sched = self.schedule()
        check_schedule(self.R, sched)
        compute = torch.cuda.current_stream(self.device)
        o = torch.empty((rows, self.hq, self.dim), dtype=torch.float32, device=self.device)
        lse = torch.empty((self.hq, rows), dtype=torch.float32, device=self.device)
        feeder = _Feeder(kv_of_source, sched, stage, self.device, pack=[(0, 2), (1, 3)])
        first = True
        for t in range(self.R):
            k, v = feeder.get(t, compute)
            if timer:
                timer(t, "fwd_begin", compute)
            for p in self.problems(t):
                if first:  # the query segments cover every row: this call writes them all
                    cpattn.cp_attn_fwd_step(p, q_new, k, v, o, lse, stream=compute)
                    first = False
                else:
                    cpattn.cp_attn_fwd_step_merge(p, q_new, k, v, o, lse, stream=compute)
            if timer:
                timer(t, "fwd_end", compute)
            feeder.release(t, compute)
        return o, lse


def _kv_pieces(n_keys: int, hkv: int, dim: int):
    """Split keys [0, n_keys) into pieces whose K span stays under the per-call limit."""
    per = max(1, _SPAN_LIMIT // (hkv * dim * 2))
    return [(a, min(n_keys, a + per)) for a in range(0, n_keys, per)]


def _attend_sequence(q, q_segments, k_all, v_all, hq, hkv, dim, scale, cu_dev=None, n_docs=0, stream=None):
    """q (device bf16 [rows, Hq, D], segments (row0, pos0, len)) against keys at
    positions 0 .. S-1 of k_all / v_all, causal (document) mask, merged over as
    many calls as the KV span needs."""
    rows = q.shape[0]
    dev = q.device
    o = torch.empty((rows, hq, dim), dtype=torch.float32, device=dev)
    lse = torch.empty((hq, rows), dtype=torch.float32, device=dev)
    m = cpattn.CP_MASK_DOC if cu_dev is not None else cpattn.CP_MASK_DIAG_CAUSAL
    pieces = _kv_pieces(k_all.shape[0], hkv, dim)
    calls = [pieces[i:i + 2] for i in range(0, len(pieces), 2)]
    for i, call in enumerate(calls):
        kv_seg = [(a, a, b - a) for a, b in call]
        masks = [[m] * 2 for _ in range(2)]
        p = cpattn.make_problem(hq, hkv, dim, scale, rows, k_all.shape[0], list(q_segments), kv_seg, masks,
                                None if cu_dev is None else cu_dev.data_ptr(), n_docs)
        if i == 0:
            cpattn.cp_attn_fwd_step(p, q, k_all, v_all, o, lse, stream=stream)
        else:
            cpattn.cp_attn_fwd_step_merge(p, q, k_all, v_all, o, lse, stream=stream)
    return o, lse


def gathered_forward(w: Workload, rank: int, q_local, k_all, v_all, cu_dev=None, n_docs=0, stream=None):
    """The all-gather strategy's per-device work: the rank's two zigzag query
    chunks against the whole gathered sequence (device bf16 [S, Hkv, D])."""
    c = w.chunk
    pos = cpattn.cp_partition_zigzag(w.seq_len, w.cp, rank)
    qa, qb = int(pos[0]) // c, int(pos[c]) // c
    return _attend_sequence(q_local, [(0, qa * c, c), (c, qb * c, c)], k_all, v_all, w.hq, w.hkv, w.dim, w.scale,
                            cu_dev, n_docs, stream)


def head_sharded_forward(q_all, k_all, v_all, scale, cu_dev=None, n_docs=0, stream=None):
    """The all-to-all strategy's per-device work: causal attention over the whole
    sequence for the heads this device holds (q [S, Hq', D], k/v [S, Hkv', D])."""
    S, hq, dim = q_all.shape
    return _attend_sequence(q_all, [(0, 0, S)], k_all, v_all, hq, k_all.shape[1], dim, scale, cu_dev, n_docs,
                            stream)
