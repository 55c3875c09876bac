"""Float64 reference arithmetic for one rank's Pass-KV ring attention (test infrastructure only).

Layouts follow the library boundary so results compare element by element:
queries/outputs ``[n, Hq, D]``, keys/values ``[m, Hkv, D]``, LSE ``[Hq, n]``.
Query head h reads key/value head ``h // (Hq // Hkv)`` (consecutive GQA groups).
All arithmetic is float64 NumPy; rows are processed in blocks only to bound
memory, never with an online softmax.
"""
from __future__ import annotations

import numpy as np

# Chunk-pair classes of one ring step (integer codes shared with the C ABI by value only).
CLS_FULL, CLS_DIAG, CLS_DOC, CLS_SKIP = 0, 1, 2, 3
# Tile classes of the block map.
TILE_SKIP, TILE_PARTIAL, TILE_FULL = 0, 1, 2

_ROW_BLOCK = 512


# --------------------------------------------------------------------------------------
# Partition and ring order
# --------------------------------------------------------------------------------------
def zigzag_chunks(cp_size: int, rank: int) -> tuple[int, int]:
    """The two chunk indices held by ``rank`` when the sequence is cut into 2R chunks.

    "Context Parallelism for Scalable Million-Token Inference", section "Load
    Balancing in CP": with R ranks the sequence is cut into 2R equal chunks and
    each rank holds two, pairing one from the front with its mirror from the
    back (4 tokens on 2 ranks: rank 0 holds tokens 0 and 3, rank 1 holds 1 and 2).
    """
    return rank, 2 * cp_size - 1 - rank


def zigzag_positions(seq_len: int, cp_size: int, rank: int) -> np.ndarray:
    """Global positions of a rank's local tokens, in local order [chunk r ; chunk 2R-1-r]."""
    if seq_len % (2 * cp_size):
        raise ValueError("sequence length must be a multiple of 2 * cp_size")
    c = seq_len // (2 * cp_size)
    a, b = zigzag_chunks(cp_size, rank)
    return np.concatenate([np.arange(a * c, (a + 1) * c), np.arange(b * c, (b + 1) * c)]).astype(np.int64)


def ring_source(rank: int, step: int, cp_size: int) -> int:
    """Rank whose KV block is held by ``rank`` at ring step ``step``.

    Pass-KV keeps queries in place and moves each KV block one hop per step
    around the ring ("Context Parallelism for Scalable Million-Token Inference",
    section "Ring Attention Algorithms"; "Announcing Long-Context Training ...",
    Figure 3).  Reading adopted: blocks move from rank r to rank r+1, so at step
    t rank r holds the block that started on rank (r - t) mod R; step 0 is the
    rank's own block.
    """
    return (rank - step) % cp_size


# --------------------------------------------------------------------------------------
# Visibility, chunk classes, tile map
# --------------------------------------------------------------------------------------
def document_index(positions: np.ndarray, cu_seqlens: np.ndarray) -> np.ndarray:
    """Index of the packed document containing each global position."""
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    return np.searchsorted(cu, np.asarray(positions, dtype=np.int64), side="right") - 1


def visibility(qpos: np.ndarray, kpos: np.ndarray, cu_seqlens=None, window=None) -> np.ndarray:
    """Boolean [n, m]: may the query at qpos[i] attend to the key at kpos[j]?

    Causal prefill: a token sees itself and every earlier token ("Context
    Parallelism for Scalable Million-Token Inference", section "Attention
    Compute Patterns in Multi-Turn Chat").  With packed documents a token
    additionally sees only tokens of its own document ("Announcing Long-Context
    Training ...", section "Built on a fast attention kernel").  A sliding
    window of ``window`` tokens ("Announcing Long-Context Training ...", the
    closing section on window layers of models such as Gemma) further limits a
    token to the ``window`` most recent positions, itself included: key k is
    visible to query q iff q - window < k <= q.  ``window`` None or 0 means
    no window.
    """
    qpos = np.asarray(qpos, dtype=np.int64)
    kpos = np.asarray(kpos, dtype=np.int64)
    vis = kpos[None, :] <= qpos[:, None]
    if window:
        vis &= (qpos[:, None] - kpos[None, :]) < int(window)
    if cu_seqlens is not None:
        vis &= document_index(kpos, cu_seqlens)[None, :] == document_index(qpos, cu_seqlens)[:, None]
    return vis


def chunk_pair_class(qpos_chunk: np.ndarray, kpos_chunk: np.ndarray, cu_seqlens=None, window=None) -> int:
    """Brute-force class of one (query chunk, key chunk) pair from its visibility block.

    No visible pair: SKIP.  With packed documents every other pair is DOC.
    Otherwise: every pair visible and the chunks distinct: FULL; else DIAG
    (the causal diagonal, or a pair that the sliding window cuts).
    """
    vis = visibility(qpos_chunk, kpos_chunk, cu_seqlens, window)
    if not vis.any():
        return CLS_SKIP
    if cu_seqlens is not None:
        return CLS_DOC
    same_chunk = qpos_chunk[0] == kpos_chunk[0]
    if vis.all() and not same_chunk:
        return CLS_FULL
    return CLS_DIAG


def _tiles(segments, size):
    """(first position, length) of every tile of every segment, in segment order."""
    out = []
    for pos0, length in segments:
        for start in range(0, length, size):
            out.append((pos0 + start, min(size, length - start)))
    return out


def tile_map(q_segments, kv_segments, bm: int, bn: int, cu_seqlens=None, window=None) -> np.ndarray:
    """Block map of one step by brute force: uint8 [query tiles, key tiles].

    Segments are (global start position, length); tiles of ``bm`` query rows and
    ``bn`` keys start at each segment's first row, the last one possibly short.
    A tile with no visible pair is SKIP (0), one with every pair visible is FULL
    (2), anything else PARTIAL (1).  The kernel skips the SKIP tiles entirely,
    as the pages' block-sparse kernel does with fully masked blocks
    ("Announcing Long-Context Training ...", section "Built on a fast attention
    kernel").
    """
    qt = _tiles(q_segments, bm)
    kt = _tiles(kv_segments, bn)
    out = np.zeros((len(qt), len(kt)), dtype=np.uint8)
    for i, (q0, ql) in enumerate(qt):
        qpos = np.arange(q0, q0 + ql)
        for j, (k0, kl) in enumerate(kt):
            vis = visibility(qpos, np.arange(k0, k0 + kl), cu_seqlens, window)
            if vis.all():
                out[i, j] = TILE_FULL
            elif vis.any():
                out[i, j] = TILE_PARTIAL
    return out


# --------------------------------------------------------------------------------------
# Forward: one step's partial attention and the merge
# --------------------------------------------------------------------------------------
def _group(hq: int, hkv: int) -> int:
    if hq % hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    return hq // hkv


def attention_partial(q, k, v, vis, scale):
    """Softmax attention of the queries over the visible keys of one KV block.

    Returns (O [n, Hq, D], LSE [Hq, n]) in float64, O normalised over the
    visible keys and LSE = ln sum_j exp(scale * q_i . k_j).  A row with no
    visible key gets O = 0 and LSE = -inf, the identity of ``merge``.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n, hq, d = q.shape
    hkv = k.shape[1]
    g = _group(hq, hkv)
    o = np.zeros((n, hq, d), dtype=np.float64)
    lse = np.full((hq, n), -np.inf, dtype=np.float64)
    for r0 in range(0, n, _ROW_BLOCK):
        r1 = min(n, r0 + _ROW_BLOCK)
        vb = vis[r0:r1]
        live = vb.any(axis=1)
        if not live.any():
            continue
        for h in range(hq):
            kv = h // g
            s = scale * (q[r0:r1, h, :] @ k[:, kv, :].T)
            s = np.where(vb, s, -np.inf)
            mx = np.where(live, s.max(axis=1, initial=-np.inf), 0.0)
            e = np.exp(s - mx[:, None])
            den = e.sum(axis=1)
            num = e @ v[:, kv, :]
            with np.errstate(invalid="ignore", divide="ignore"):
                o[r0:r1, h, :] = np.where(live[:, None], num / np.where(live, den, 1.0)[:, None], 0.0)
                lse[h, r0:r1] = np.where(live, mx + np.log(np.where(live, den, 1.0)), -np.inf)
    return o, lse


def merge(o_acc, lse_acc, o_t, lse_t):
    """Combine two partial attention results over disjoint key sets.

    Pass KV ends by merging the partial outputs of all steps into the full
    attention output ("Context Parallelism for Scalable Million-Token
    Inference", section "Ring Attention Algorithms").  With L = ln(e^La + e^Lb)
    the merged output is e^(La-L) O_a + e^(Lb-L) O_b.  Two empty partials
    (both LSE = -inf) merge to (0, -inf).
    """
    lse_acc = np.asarray(lse_acc, dtype=np.float64)
    lse_t = np.asarray(lse_t, dtype=np.float64)
    lse = np.logaddexp(lse_acc, lse_t)
    empty = np.isneginf(lse)
    safe = np.where(empty, 0.0, lse)
    wa = np.where(empty, 0.0, np.exp(lse_acc - safe))   # [H, n]
    wb = np.where(empty, 0.0, np.exp(lse_t - safe))
    o = wa.T[:, :, None] * np.asarray(o_acc, dtype=np.float64) + wb.T[:, :, None] * np.asarray(o_t, dtype=np.float64)
    return o, lse


# --------------------------------------------------------------------------------------
# Backward: one step's gradient terms from the final LSE
# --------------------------------------------------------------------------------------
def delta_rows(do, o):
    """Delta[h, i] = sum_d dO[i, h, d] * O[i, h, d] (float64, [Hq, n])."""
    return np.einsum("nhd,nhd->hn", np.asarray(do, dtype=np.float64), np.asarray(o, dtype=np.float64))


def attention_backward_partial(q, k, v, do, lse, delta, vis, scale):
    """Gradient terms of one step, given the final (merged) LSE and Delta of each row.

    With P = exp(scale q.k - LSE) restricted to the visible keys of this block,
    the exact gradient of the full attention splits over blocks as
      dV_j   = sum_i P_ij dO_i
      dS_ij  = P_ij (dO_i . v_j - Delta_i)
      dQ_i  += scale sum_j dS_ij k_j
      dK_j   = scale sum_i dS_ij q_i
    dK/dV are summed over the query heads that share a KV head.
    Returns (dQ part [n, Hq, D], dK [m, Hkv, D], dV [m, Hkv, D]) in float64.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    n, hq, d = q.shape
    m, hkv, _ = k.shape
    g = _group(hq, hkv)
    dq = np.zeros_like(q)
    dk = np.zeros((m, hkv, d), dtype=np.float64)
    dv = np.zeros((m, hkv, d), dtype=np.float64)
    for r0 in range(0, n, _ROW_BLOCK):
        r1 = min(n, r0 + _ROW_BLOCK)
        vb = vis[r0:r1]
        if not vb.any():
            continue
        for h in range(hq):
            kv = h // g
            lrow = lse[h, r0:r1]
            finite = np.isfinite(lrow)
            s = scale * (q[r0:r1, h, :] @ k[:, kv, :].T)
            arg = np.where(vb & finite[:, None], s - np.where(finite, lrow, 0.0)[:, None], -np.inf)
            p = np.exp(arg)
            dov = do[r0:r1, h, :]
            dv[:, kv, :] += p.T @ dov
            dp = dov @ v[:, kv, :].T
            ds = p * (dp - delta[h, r0:r1][:, None])
            dq[r0:r1, h, :] += scale * (ds @ k[:, kv, :])
            dk[:, kv, :] += scale * (ds.T @ q[r0:r1, h, :])
    return dq, dk, dv


# --------------------------------------------------------------------------------------
# One rank's whole ring
# --------------------------------------------------------------------------------------
def rank_forward(q_local, qpos, kv_blocks, cu_seqlens, scale, rows=None, window=None):
    """Replay one rank's R forward steps and merge them step by step.

    ``kv_blocks`` lists, in ring order, (k, v, kpos) of the block held at each
    step.  ``rows`` optionally restricts the computation to a subset of local
    query rows (the result then covers only those rows).  ``window`` is the
    sliding window of ``visibility``.
    Returns (O, LSE, per-step list of (O_t, LSE_t)).
    """
    if rows is not None:
        q_local = np.asarray(q_local)[rows]
        qpos = np.asarray(qpos)[rows]
    n, hq, d = np.asarray(q_local).shape
    o = np.zeros((n, hq, d))
    lse = np.full((hq, n), -np.inf)
    steps = []
    for k, v, kpos in kv_blocks:
        vis = visibility(qpos, kpos, cu_seqlens, window)
        o_t, lse_t = attention_partial(q_local, k, v, vis, scale)
        steps.append((o_t, lse_t))
        o, lse = merge(o, lse, o_t, lse_t)
    return o, lse, steps


def rank_backward(q_local, qpos, do_local, o, lse, kv_blocks, cu_seqlens, scale, window=None):
    """Replay one rank's R backward steps from the final O and LSE.

    dQ accumulates over the steps; dK/dV are returned per step (the part of the
    gradient of that step's KV block due to this rank's queries).
    """
    delta = delta_rows(do_local, o)
    dq = np.zeros(np.asarray(q_local).shape)
    per_step = []
    for k, v, kpos in kv_blocks:
        vis = visibility(qpos, kpos, cu_seqlens, window)
        dq_t, dk_t, dv_t = attention_backward_partial(q_local, k, v, do_local, lse, delta, vis, scale)
        dq += dq_t
        per_step.append((dk_t, dv_t))
    return dq, per_step, delta


def causal_flops(qpos, kpos, hq, dim, cu_seqlens=None, backward=False, window=None):
    """Causal-counted FLOPs of one step: 4*D (forward) or 10*D (backward) per
    visible (query, key) pair and query head.  Convention only: parity unpinned."""
    pairs = int(visibility(qpos, kpos, cu_seqlens, window).sum())
    return pairs * hq * dim * (10 if backward else 4)
