"""Pins of the oracle's sliding-window visibility (CPU only).

Window layers of models such as Gemma are the extension the MaxText page names
in its closing section: a token sees only the ``window`` most recent positions,
itself included.  The references here are independent of the oracle's code:
PyTorch's float64 CPU attention (forward and autograd) under a band mask built
with ``np.tril``, closed forms of special inputs, brute force on tiny inputs and
the pages' statement that window layers need only a short exchange between
neighbouring chips.
"""
import math

import numpy as np
import pytest
import torch

import oracle


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _band(n, window):
    """Query i may see key j iff i - window < j <= i: lower triangle minus everything
    at or below diagonal -window."""
    ones = np.ones((n, n), dtype=bool)
    return np.tril(ones) & ~np.tril(ones, -window)


def _torch_attention(q, k, v, scale, mask):
    g = q.shape[1] // k.shape[1]
    tq = torch.from_numpy(np.ascontiguousarray(q.transpose(1, 0, 2)))[None]
    tk = torch.from_numpy(np.ascontiguousarray(np.repeat(k, g, axis=1).transpose(1, 0, 2)))[None]
    tv = torch.from_numpy(np.ascontiguousarray(np.repeat(v, g, axis=1).transpose(1, 0, 2)))[None]
    am = torch.from_numpy(np.where(mask, 0.0, -np.inf))[None, None]
    out, lse = torch.ops.aten._scaled_dot_product_flash_attention_for_cpu(tq, tk, tv, 0.0, False, attn_mask=am,
                                                                          scale=scale)
    return out[0].numpy().transpose(1, 0, 2), lse[0].numpy()


def _ring_all_ranks(q, k, v, S, R, scale, window, cu=None):
    out = np.zeros_like(q)
    lse_out = np.zeros((q.shape[1], S))
    for r in range(R):
        qpos = oracle.zigzag_positions(S, R, r)
        blocks = []
        for t in range(R):
            kpos = oracle.zigzag_positions(S, R, oracle.ring_source(r, t, R))
            blocks.append((k[kpos], v[kpos], kpos))
        o, lse, _ = oracle.rank_forward(q[qpos], qpos, blocks, cu, scale, window=window)
        out[qpos] = o
        lse_out[:, qpos] = lse
    return out, lse_out


def test_band_mask_construction():
    m = _band(6, 2)
    assert m[3].tolist() == [False, False, True, True, False, False]
    assert m[0].tolist() == [True] + [False] * 5
    assert np.array_equal(oracle.visibility(np.arange(6), np.arange(6), window=2), m)


@pytest.mark.parametrize("S,R,window", [(64, 2, 5), (96, 3, 16), (128, 4, 1), (128, 4, 40), (80, 5, 8)])
def test_ring_with_window_equals_banded_attention(S, R, window):
    """Merging every rank's ring partials reproduces full attention under the band mask."""
    hq, hkv, d = 4, 2, 8
    q, k, v = _rand((S, hq, d), 1), _rand((S, hkv, d), 2), _rand((S, hkv, d), 3)
    scale = 1 / math.sqrt(d)
    o, lse = _ring_all_ranks(q, k, v, S, R, scale, window)
    ro, rlse = _torch_attention(q, k, v, scale, _band(S, window))
    np.testing.assert_allclose(o, ro, atol=1e-12)
    np.testing.assert_allclose(lse, rlse, atol=1e-12)


def test_window_at_least_sequence_is_causal():
    S = 48
    pos = np.arange(S)
    causal = oracle.visibility(pos, pos)
    for w in (S, S + 7, 10 ** 6):
        assert np.array_equal(oracle.visibility(pos, pos, window=w), causal)
    assert np.array_equal(oracle.visibility(pos, pos, window=0), causal)


def test_window_one_sees_only_itself():
    """window = 1: O_i = v_i and LSE_i = scale q_i . k_i."""
    n, hq, hkv, d = 20, 4, 2, 8
    q, k, v = _rand((n, hq, d), 4), _rand((n, hkv, d), 5), _rand((n, hkv, d), 6)
    pos = np.arange(n)
    o, lse = oracle.attention_partial(q, k, v, oracle.visibility(pos, pos, window=1), 0.4)
    g = hq // hkv
    for h in range(hq):
        np.testing.assert_allclose(o[:, h], v[:, h // g], atol=1e-13)
        np.testing.assert_allclose(lse[h], 0.4 * np.einsum("nd,nd->n", q[:, h], k[:, h // g]), atol=1e-13)


def test_zero_queries_average_the_window():
    """Q = 0: O_i = mean of v over the last min(i+1, W) keys, LSE_i = ln min(i+1, W)."""
    n, hq, hkv, d, w = 30, 2, 1, 4, 7
    q = np.zeros((n, hq, d))
    k, v = _rand((n, hkv, d), 7), _rand((n, hkv, d), 8)
    pos = np.arange(n)
    o, lse = oracle.attention_partial(q, k, v, oracle.visibility(pos, pos, window=w), 1.0)
    for i in range(n):
        lo = max(0, i - w + 1)
        np.testing.assert_allclose(o[i, 0], v[lo:i + 1, 0].mean(axis=0), atol=1e-13)
        assert lse[0, i] == pytest.approx(math.log(i + 1 - lo), abs=1e-13)


@pytest.mark.parametrize("R", [2, 3, 4, 6])
def test_short_window_needs_only_neighbour_blocks(R):
    """With a window no longer than a chunk, a rank's ring steps with any visible
    pair are its own block and its neighbours' (steps 0, 1 and R-1): the pages'
    short exchange between neighbouring chips for window layers.  Rank r's first
    chunk needs chunk r-1 (rank r-1, step 1; none for rank 0) and its second
    chunk needs chunk 2R-2-r (rank r+1, step R-1; its own first chunk for rank
    R-1)."""
    c = 8
    S = 2 * R * c
    for w in (1, 3, c):
        for r in range(R):
            qpos = oracle.zigzag_positions(S, R, r)
            live = [t for t in range(R)
                    if oracle.visibility(qpos, oracle.zigzag_positions(S, R, oracle.ring_source(r, t, R)),
                                         window=w).any()]
            expected = {0}
            if w > 1:
                expected |= ({1} if r > 0 else set()) | ({R - 1} if r < R - 1 else set())
            expected = sorted(expected)
            assert live == expected, (r, w, live)


def test_chunk_classes_under_a_window():
    """Brute-force chunk classes: a window that cuts a causal-full pair makes it DIAG,
    one beyond reach makes it SKIP."""
    c = 4
    q = np.arange(3 * c, 4 * c)  # chunk 3
    assert oracle.chunk_pair_class(q, np.arange(2 * c, 3 * c)) == oracle.CLS_FULL
    assert oracle.chunk_pair_class(q, np.arange(2 * c, 3 * c), window=2 * c) == oracle.CLS_FULL
    assert oracle.chunk_pair_class(q, np.arange(2 * c, 3 * c), window=2 * c - 1) == oracle.CLS_DIAG
    # chunk 0 is 2c + 1 positions back at the closest pair (query 3c, key c - 1)
    assert oracle.chunk_pair_class(q, np.arange(0, c), window=2 * c + 2) == oracle.CLS_DIAG
    assert oracle.chunk_pair_class(q, np.arange(0, c), window=2 * c + 1) == oracle.CLS_SKIP
    assert oracle.chunk_pair_class(q, q, window=1) == oracle.CLS_DIAG


def test_documents_with_window_are_independent_windowed_sequences():
    """Packed documents under a window: each document equals windowed attention on it alone."""
    S, hq, hkv, d, w = 60, 2, 2, 8, 9
    cu = np.array([0, 13, 14, 41, 60])
    q, k, v = _rand((S, hq, d), 9), _rand((S, hkv, d), 10), _rand((S, hkv, d), 11)
    pos = np.arange(S)
    o, lse = oracle.attention_partial(q, k, v, oracle.visibility(pos, pos, cu, window=w), 0.3)
    for a, b in zip(cu[:-1], cu[1:]):
        ro, rlse = _torch_attention(q[a:b], k[a:b], v[a:b], 0.3, _band(b - a, w))
        np.testing.assert_allclose(o[a:b], ro, atol=1e-12)
        np.testing.assert_allclose(lse[:, a:b], rlse, atol=1e-12)


@pytest.mark.parametrize("S,R,window", [(32, 2, 6), (48, 3, 5), (64, 4, 20)])
def test_backward_with_window_matches_autograd(S, R, window):
    """All-rank replay of the windowed backward equals PyTorch autograd under the band mask."""
    hq, hkv, d = 4, 2, 8
    q, k, v, do = (_rand((S, hq, d), 12), _rand((S, hkv, d), 13), _rand((S, hkv, d), 14),
                   _rand((S, hq, d), 15))
    scale = 1 / math.sqrt(d)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for r in range(R):
        qpos = oracle.zigzag_positions(S, R, r)
        blocks = []
        for t in range(R):
            kpos = oracle.zigzag_positions(S, R, oracle.ring_source(r, t, R))
            blocks.append((k[kpos], v[kpos], kpos))
        o, lse, _ = oracle.rank_forward(q[qpos], qpos, blocks, None, scale, window=window)
        dq_r, per_step, _ = oracle.rank_backward(q[qpos], qpos, do[qpos], o, lse, blocks, None, scale,
                                                 window=window)
        dq[qpos] = dq_r
        for (dk_t, dv_t), (_, _, kpos) in zip(per_step, blocks):
            dk[kpos] += dk_t
            dv[kpos] += dv_t
    g = hq // hkv
    tq = torch.tensor(q.transpose(1, 0, 2)[None], requires_grad=True)
    tk = torch.tensor(k.transpose(1, 0, 2)[None], requires_grad=True)
    tv = torch.tensor(v.transpose(1, 0, 2)[None], requires_grad=True)
    am = torch.from_numpy(np.where(_band(S, window), 0.0, -np.inf))[None, None]
    out = torch.nn.functional.scaled_dot_product_attention(
        tq, tk.repeat_interleave(g, dim=1), tv.repeat_interleave(g, dim=1), attn_mask=am, scale=scale)
    out.backward(torch.from_numpy(do.transpose(1, 0, 2)[None].copy()))
    t = lambda x: x.grad[0].numpy().transpose(1, 0, 2)
    np.testing.assert_allclose(dq, t(tq), atol=1e-11)
    np.testing.assert_allclose(dk, t(tk), atol=1e-11)
    np.testing.assert_allclose(dv, t(tv), atol=1e-11)


def test_backward_window_finite_differences():
    """Central differences of f = sum dO * O on a tiny windowed problem."""
    S, hq, hkv, d, w = 10, 2, 1, 3, 3
    q, k, v, do = _rand((S, hq, d), 16), _rand((S, hkv, d), 17), _rand((S, hkv, d), 18), _rand((S, hq, d), 19)
    pos = np.arange(S)
    vis = oracle.visibility(pos, pos, window=w)

    def f(q_, k_, v_):
        o, _ = oracle.attention_partial(q_, k_, v_, vis, 0.5)
        return float((do * o).sum())

    o, lse = oracle.attention_partial(q, k, v, vis, 0.5)
    delta = oracle.delta_rows(do, o)
    dq, dk, dv = oracle.attention_backward_partial(q, k, v, do, lse, delta, vis, 0.5)
    eps = 1e-6
    for arr, grad in ((q, dq), (k, dk), (v, dv)):
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            a0 = arr[idx]
            arr[idx] = a0 + eps
            fp = f(q, k, v)
            arr[idx] = a0 - eps
            fm = f(q, k, v)
            arr[idx] = a0
            num[idx] = (fp - fm) / (2 * eps)
        np.testing.assert_allclose(grad, num, atol=1e-7, rtol=1e-6)


def test_window_tile_map_brute_force_rule():
    """The oracle's tile map under a window agrees with the interval rule the kernels
    use: a tile [q0, q1] x [k0, k1] is skipped iff k0 > q1 or k1 < q0 - W + 1, and
    full iff k1 <= q0 and k0 >= q1 - W + 1."""
    rng = np.random.default_rng(20)
    for _ in range(300):
        w = int(rng.integers(1, 60))
        q0 = int(rng.integers(0, 200))
        ql = int(rng.integers(1, 40))
        k0 = int(rng.integers(0, 200))
        kl = int(rng.integers(1, 40))
        m = oracle.tile_map([(q0, ql)], [(k0, kl)], ql, kl, window=w)[0, 0]
        q1, k1 = q0 + ql - 1, k0 + kl - 1
        if k0 > q1 or k1 < q0 - w + 1:
            expect = oracle.TILE_SKIP
        elif k1 <= q0 and k0 >= q1 - w + 1:
            expect = oracle.TILE_FULL
        else:
            expect = oracle.TILE_PARTIAL
        assert m == expect, (w, q0, ql, k0, kl)
