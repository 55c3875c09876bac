"""Float64 oracle for the ring variants beside Pass KV.

TEST INFRASTRUCTURE ONLY, like the rest of this package: nothing on the product
path imports or calls it.  Each function composes the pinned primitives of
``oracle.ring`` (partition, visibility, exact partial attention, merge) in the
order the pages describe:

* Pass Q -- "Context Parallelism for Scalable Million-Token Inference", section
  "Ring Attention Algorithms" (the Pass Q algorithm): K/V stay on their rank,
  the Q blocks travel around the ring; after the rotation every rank holds one
  partial output per Q owner, which a permutation and an all-to-all deliver to
  the owners, who merge them.
* Partial prefill -- same page, section "Attention Compute Patterns in
  Multi-Turn Chat" (new prompt tokens attend to themselves causally and to all
  cached tokens) and section "Load Balancing in CP" (the same two-chunks-per-rank
  sharding applies to partial prefill, with previously cached tokens).
* Gathered KV and head-sharded attention -- "Announcing Long-Context Training on
  TPUs with MaxText Context Parallelism", section "Context Parallelism in
  MaxText": with all-gather each device attends its load-balanced query share
  to the whole gathered sequence; with the all-to-all (Ulysses) strategy each
  device runs ordinary attention over the full sequence for a subset of heads.

Pins (``tests/test_oracle_variants.py``): across all ranks Pass Q reproduces
full causal attention and each of its partials equals the Pass KV partial of
the same (query owner, KV block); partial prefill reproduces the plain causal
attention of the new tokens; the gathered call equals the Pass KV ring result;
the head-sharded call equals full attention restricted to its heads.
"""
from __future__ import annotations

import numpy as np

from .ring import attention_partial, merge, ring_source, visibility, zigzag_positions


def pass_q_partials(rank, cp_size, q_of_rank, qpos_of_rank, k, v, kpos, cu_seqlens, scale):
    """Pass Q at one rank.  The rank's K/V (positions ``kpos``) stay put; at step
    t the Q block of rank ring_source(rank, t) is held.  Returns, in step order,
    (owner, O_t, LSE_t): the partial attention of the visiting queries over the
    local keys."""
    out = []
    for t in range(cp_size):
        s = ring_source(rank, t, cp_size)
        vis = visibility(qpos_of_rank(s), kpos, cu_seqlens)
        o_t, lse_t = attention_partial(q_of_rank(s), k, v, vis, scale)
        out.append((s, o_t, lse_t))
    return out


def pass_q_restore(partials_by_rank, owner):
    """The owner's side of the permutation and all-to-all: gather, from every
    rank, the partial computed for the owner's queries, and merge them (in rank
    order; the merge is exact, so the order only affects rounding)."""
    o = lse = None
    for r in sorted(partials_by_rank):
        for s, o_t, lse_t in partials_by_rank[r]:
            if s != owner:
                continue
            if o is None:
                o = np.zeros_like(o_t)
                lse = np.full_like(lse_t, -np.inf)
            o, lse = merge(o, lse, o_t, lse_t)
    return o, lse


def partial_prefill_positions(n_cached: int, n_new: int, cp_size: int, rank: int):
    """Global positions held by a rank in a partial prefill: its two chunks of the
    cached prefix [0, n_cached) and its two chunks of the new tokens
    [n_cached, n_cached + n_new), each part split into 2R chunks."""
    cached = zigzag_positions(n_cached, cp_size, rank)
    new = n_cached + zigzag_positions(n_new, cp_size, rank)
    return cached, new


def partial_prefill_rank(q_new, qpos_new, kv_blocks, scale):
    """Pass KV over a partial prefill at one rank: the rank's new-token queries
    against, at each step, the cached and new K/V held by the visiting rank.
    ``kv_blocks`` lists in ring order ((k_cached, v_cached, pos_cached),
    (k_new, v_new, pos_new)).  Visibility is causal by global position, so every
    cached key is visible to every new token.  Returns the merged (O, LSE)."""
    n, hq, d = np.asarray(q_new).shape
    o = np.zeros((n, hq, d))
    lse = np.full((hq, n), -np.inf)
    for part in kv_blocks:
        for k, v, kpos in part:
            o_t, lse_t = attention_partial(q_new, k, v, visibility(qpos_new, kpos), scale)
            o, lse = merge(o, lse, o_t, lse_t)
    return o, lse


def gathered_attention(q_local, qpos, k_all, v_all, scale, cu_seqlens=None):
    """All-gather strategy at one rank: the rank's query share against the whole
    gathered sequence (keys at positions 0 .. S-1), one exact partial."""
    kpos = np.arange(np.asarray(k_all).shape[0])
    return attention_partial(q_local, k_all, v_all, visibility(qpos, kpos, cu_seqlens), scale)


def head_sharded_attention(q_all, k_all, v_all, q_heads, kv_heads, scale, cu_seqlens=None):
    """All-to-all (Ulysses) strategy at one device: full-sequence causal attention
    for the query heads ``q_heads`` and their KV heads ``kv_heads``."""
    pos = np.arange(np.asarray(q_all).shape[0])
    q = np.asarray(q_all)[:, q_heads]
    k = np.asarray(k_all)[:, kv_heads]
    v = np.asarray(v_all)[:, kv_heads]
    return attention_partial(q, k, v, visibility(pos, pos, cu_seqlens), scale)
