"""Pins of the oracle's ring variants (CPU only): Pass Q, partial prefill, the
gathered-KV call and the head-sharded call.

References are PyTorch's CPU attention over the whole sequence (independent of
the oracle) and the already pinned Pass KV replay of ``oracle.rank_forward``.
"""
import math

import numpy as np
import pytest

import oracle
from oracle import variants
from tests.test_oracle_forward import _torch_attention


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _doc_mask(n, cu):
    pos = np.arange(n)
    vis = pos[None, :] <= pos[:, None]
    if cu is not None:
        doc = np.searchsorted(cu, pos, side="right") - 1
        vis &= doc[None, :] == doc[:, None]
    return vis


@pytest.mark.parametrize("S,R,hq,hkv,d,docs", [(64, 4, 4, 2, 16, False), (48, 3, 2, 2, 8, True),
                                               (40, 2, 6, 3, 8, True)])
def test_pass_q_over_all_ranks_is_full_causal_attention(S, R, hq, hkv, d, docs):
    """Every rank's partials, delivered to the query owners and merged there,
    reproduce full causal (document) attention of the whole sequence."""
    q, k, v = _rand((S, hq, d), 1), _rand((S, hkv, d), 2), _rand((S, hkv, d), 3)
    cu = np.array([0, 5, 6, S // 2 + 1, S], dtype=np.int64) if docs else None
    scale = 1 / math.sqrt(d)
    pos = {r: oracle.zigzag_positions(S, R, r) for r in range(R)}
    parts = {r: variants.pass_q_partials(r, R, lambda s: q[pos[s]], lambda s: pos[s], k[pos[r]], v[pos[r]], pos[r],
                                         cu, scale) for r in range(R)}
    o = np.zeros((S, hq, d))
    lse = np.zeros((hq, S))
    for owner in range(R):
        # every rank produced exactly one partial for this owner
        assert sum(s == owner for r in range(R) for s, _, _ in parts[r]) == R
        oo, ll = variants.pass_q_restore(parts, owner)
        o[pos[owner]] = oo
        lse[:, pos[owner]] = ll
    ro, rl = _torch_attention(q, k, v, scale, mask=_doc_mask(S, cu))
    np.testing.assert_allclose(o, ro, atol=1e-12)
    np.testing.assert_allclose(lse, rl, atol=1e-12)


def test_pass_q_partial_is_the_pass_kv_partial_of_the_same_pair():
    """The partial Pass Q computes at rank r for owner s is the partial Pass KV
    computes at rank s while it holds rank r's KV block."""
    S, R, hq, hkv, d = 64, 4, 4, 2, 8
    q, k, v = _rand((S, hq, d), 4), _rand((S, hkv, d), 5), _rand((S, hkv, d), 6)
    pos = {r: oracle.zigzag_positions(S, R, r) for r in range(R)}
    for r in range(R):
        parts = variants.pass_q_partials(r, R, lambda s: q[pos[s]], lambda s: pos[s], k[pos[r]], v[pos[r]], pos[r],
                                         None, 0.3)
        for s, o_t, l_t in parts:
            blocks = [(k[pos[oracle.ring_source(s, t, R)]], v[pos[oracle.ring_source(s, t, R)]],
                       pos[oracle.ring_source(s, t, R)]) for t in range(R)]
            _, _, steps = oracle.rank_forward(q[pos[s]], pos[s], blocks, None, 0.3)
            t_kv = [oracle.ring_source(s, t, R) for t in range(R)].index(r)
            np.testing.assert_allclose(o_t, steps[t_kv][0], atol=1e-13)
            np.testing.assert_array_equal(np.isneginf(l_t), np.isneginf(steps[t_kv][1]))


@pytest.mark.parametrize("P,N,R", [(48, 32, 2), (24, 48, 3), (64, 16, 4)])
def test_partial_prefill_is_causal_attention_of_the_new_tokens(P, N, R):
    """New tokens (zigzag-sharded) against the cached prefix and each other, over
    the ring, equal the rows of plain causal attention of the whole sequence."""
    S, hq, hkv, d = P + N, 4, 2, 8
    q, k, v = _rand((S, hq, d), 7), _rand((S, hkv, d), 8), _rand((S, hkv, d), 9)
    scale = 0.35
    ro, rl = _torch_attention(q, k, v, scale, causal=True)
    seen = []
    for r in range(R):
        cached_r, new_r = variants.partial_prefill_positions(P, N, R, r)
        assert len(cached_r) == P // R and len(new_r) == N // R
        blocks = []
        for t in range(R):
            s = oracle.ring_source(r, t, R)
            cs, ns = variants.partial_prefill_positions(P, N, R, s)
            blocks.append(((k[cs], v[cs], cs), (k[ns], v[ns], ns)))
        o, lse = variants.partial_prefill_rank(q[new_r], new_r, blocks, scale)
        np.testing.assert_allclose(o, ro[new_r], atol=1e-12)
        np.testing.assert_allclose(lse, rl[:, new_r], atol=1e-12)
        seen.append(new_r)
    # the ranks' new-token shares partition the new tokens
    assert np.array_equal(np.sort(np.concatenate(seen)), np.arange(P, S))


@pytest.mark.parametrize("docs", [False, True])
def test_gathered_call_equals_the_pass_kv_ring(docs):
    S, R, hq, hkv, d = 64, 4, 4, 2, 8
    q, k, v = _rand((S, hq, d), 10), _rand((S, hkv, d), 11), _rand((S, hkv, d), 12)
    cu = np.array([0, 9, 40, S], dtype=np.int64) if docs else None
    for r in (0, R - 1):
        pos = oracle.zigzag_positions(S, R, r)
        blocks = [(k[p], v[p], p) for p in (oracle.zigzag_positions(S, R, oracle.ring_source(r, t, R))
                                             for t in range(R))]
        o_ring, l_ring, _ = oracle.rank_forward(q[pos], pos, blocks, cu, 0.25)
        o_g, l_g = variants.gathered_attention(q[pos], pos, k, v, 0.25, cu)
        np.testing.assert_allclose(o_g, o_ring, atol=1e-12)
        np.testing.assert_allclose(l_g, l_ring, atol=1e-12)


def test_head_sharded_call_is_full_attention_of_its_heads():
    S, hq, hkv, d, R = 40, 8, 4, 8, 4
    q, k, v = _rand((S, hq, d), 13), _rand((S, hkv, d), 14), _rand((S, hkv, d), 15)
    ro, rl = _torch_attention(q, k, v, 0.3, causal=True)
    g = hq // hkv
    for dev in range(R):
        qh = list(range(dev * hq // R, (dev + 1) * hq // R))
        kvh = sorted({h // g for h in qh})
        o, lse = variants.head_sharded_attention(q, k, v, qh, kvh, 0.3)
        np.testing.assert_allclose(o, ro[:, qh], atol=1e-12)
        np.testing.assert_allclose(lse, rl[qh], atol=1e-12)


@pytest.mark.parametrize("S,R,U,hq,hkv,d", [(64, 4, 2, 4, 2, 16), (96, 6, 3, 6, 3, 8), (64, 4, 4, 8, 4, 8)])
def test_usp_shares_reassemble_full_attention(S, R, U, hq, hkv, d):
    """USP: inside groups of U devices an all-to-all trades tokens for heads, and a
    ring runs across the R/U groups.  Device (head group g, ring rank p) runs the
    Pass-KV ring of R/U ranks on heads g of the whole sequence; over all devices
    the shares cover full causal attention exactly once."""
    q, k, v = _rand((S, hq, d), 21), _rand((S, hkv, d), 22), _rand((S, hkv, d), 23)
    scale = 1 / math.sqrt(d)
    ro, rl = _torch_attention(q, k, v, scale, causal=True)
    P, gq, gk = R // U, hq // U, hkv // U
    o = np.full((S, hq, d), np.nan)
    lse = np.full((hq, S), np.nan)
    for g in range(U):
        qh, kh = np.arange(g * gq, (g + 1) * gq), np.arange(g * gk, (g + 1) * gk)
        for p in range(P):
            pos = oracle.zigzag_positions(S, P, p)
            blocks = [(k[ps][:, kh], v[ps][:, kh], ps) for ps in (oracle.zigzag_positions(S, P, s) for s in range(P))]
            oo, ll, _ = oracle.rank_forward(q[pos][:, qh], pos, blocks, None, scale)
            o[np.ix_(pos, qh)] = oo
            lse[np.ix_(qh, pos)] = ll
    np.testing.assert_allclose(o, ro, atol=1e-12)
    np.testing.assert_allclose(lse, rl, atol=1e-12)
