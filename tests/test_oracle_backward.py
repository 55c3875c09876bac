"""Pins of the oracle's backward step (CPU only): finite differences, PyTorch
autograd through its float64 CPU attention, closed forms and the all-rank sum."""
import math

import numpy as np
import pytest
import torch

import oracle
from context_long_attention_amd import inputs


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _rank_grads(q, k, v, do, S, R, cu, scale):
    """Replay every rank forward then backward; scatter dQ and sum per-source dK/dV."""
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    out = np.zeros_like(q)
    for r in range(R):
        qpos = oracle.zigzag_positions(S, R, r)
        blocks = []
        for t in range(R):
            kpos = oracle.zigzag_positions(S, R, oracle.ring_source(r, t, R))
            blocks.append((k[kpos], v[kpos], kpos))
        o, lse, _ = oracle.rank_forward(q[qpos], qpos, blocks, cu, scale)
        out[qpos] = o
        dq_r, per_step, _ = oracle.rank_backward(q[qpos], qpos, do[qpos], o, lse, blocks, cu, scale)
        dq[qpos] = dq_r
        for (dk_t, dv_t), (_, _, kpos) in zip(per_step, blocks):
            dk[kpos] += dk_t
            dv[kpos] += dv_t
    return out, dq, dk, dv


def _torch_grads(q, k, v, do, scale, mask):
    g = q.shape[1] // k.shape[1]
    tq = torch.tensor(q.transpose(1, 0, 2)[None], requires_grad=True)
    tk = torch.tensor(k.transpose(1, 0, 2)[None], requires_grad=True)
    tv = torch.tensor(v.transpose(1, 0, 2)[None], requires_grad=True)
    am = torch.from_numpy(np.where(mask, 0.0, -np.inf))[None, None]
    out = torch.nn.functional.scaled_dot_product_attention(
        tq, tk.repeat_interleave(g, dim=1), tv.repeat_interleave(g, dim=1), attn_mask=am, scale=scale)
    out.backward(torch.from_numpy(do.transpose(1, 0, 2)[None].copy()))
    t = lambda x: x.detach()[0].numpy().transpose(1, 0, 2)
    return t(out), t(tq.grad), t(tk.grad), t(tv.grad)


@pytest.mark.parametrize("S,R,hq,hkv,d,packed", [(16, 2, 2, 1, 4, False), (24, 3, 4, 2, 8, True),
                                                  (32, 4, 4, 2, 8, False)])
def test_backward_finite_differences(S, R, hq, hkv, d, packed):
    """Central differences of f = sum(dO * O) with respect to every input entry."""
    q, k, v, do = _rand((S, hq, d), 1), _rand((S, hkv, d), 2), _rand((S, hkv, d), 3), _rand((S, hq, d), 4)
    cu = np.array([0, 5, 6, S]) if packed else None
    scale = 1 / math.sqrt(d)
    _, dq, dk, dv = _rank_grads(q, k, v, do, S, R, cu, scale)

    def f(q_, k_, v_):
        out, _, _, _ = _rank_grads(q_, k_, v_, do, S, R, cu, scale)
        return float((out * do).sum())

    eps = 1e-5
    rng = np.random.default_rng(0)
    for arr, grad, which in ((q, dq, 0), (k, dk, 1), (v, dv, 2)):
        for _ in range(12):
            idx = tuple(rng.integers(0, s) for s in arr.shape)
            plus = [q.copy(), k.copy(), v.copy()]
            minus = [q.copy(), k.copy(), v.copy()]
            plus[which][idx] += eps
            minus[which][idx] -= eps
            fd = (f(*plus) - f(*minus)) / (2 * eps)
            assert abs(fd - grad[idx]) <= 1e-7 * max(1.0, abs(fd)), (which, idx, fd, grad[idx])


@pytest.mark.parametrize("packed", [False, True])
def test_all_ranks_backward_equals_autograd(packed):
    """Tiny workload: dQ scattered from every rank and per-source dK/dV summed over
    ranks equal the gradients of full-sequence attention (PyTorch autograd, float64)."""
    w = inputs.WORKLOADS["tiny"]
    S, R, c = w.seq_len, w.cp, w.chunk
    q = inputs.chunks_normal(inputs.SEED_Q, range(2 * R), c, w.hq, w.dim).astype(np.float64)
    k = inputs.chunks_normal(inputs.SEED_K, range(2 * R), c, w.hkv, w.dim).astype(np.float64)
    v = inputs.chunks_normal(inputs.SEED_V, range(2 * R), c, w.hkv, w.dim).astype(np.float64)
    do = inputs.chunks_normal(inputs.SEED_DO, range(2 * R), c, w.hq, w.dim).astype(np.float64)
    cu = np.array([0, 100, 101, 300, 512]) if packed else None
    mask = oracle.visibility(np.arange(S), np.arange(S), cu)
    out, dq, dk, dv = _rank_grads(q, k, v, do, S, R, cu, w.scale)
    ro, rdq, rdk, rdv = _torch_grads(q, k, v, do, w.scale, mask)
    np.testing.assert_allclose(out, ro, atol=1e-12)
    np.testing.assert_allclose(dq, rdq, atol=1e-11)
    np.testing.assert_allclose(dk, rdk, atol=1e-11)
    np.testing.assert_allclose(dv, rdv, atol=1e-11)


def test_backward_closed_forms():
    S, R, hq, hkv, d = 32, 2, 4, 2, 8
    scale = 0.3
    q, k, do = _rand((S, hq, d), 5), _rand((S, hkv, d), 6), _rand((S, hq, d), 7)
    vconst = np.broadcast_to(_rand((1, hkv, d), 8), (S, hkv, d)).copy()
    # constant V: the output does not depend on Q or K at all
    _, dq, dk, dv = _rank_grads(q, k, vconst, do, S, R, None, scale)
    np.testing.assert_allclose(dq, 0, atol=1e-12)
    np.testing.assert_allclose(dk, 0, atol=1e-12)
    # rows of P sum to one: sum_j dV_j = sum of dO over the query heads of the group
    v = _rand((S, hkv, d), 9)
    _, dq, dk, dv = _rank_grads(q, k, v, do, S, R, None, scale)
    g = hq // hkv
    for kv in range(hkv):
        np.testing.assert_allclose(dv[:, kv].sum(0), do[:, kv * g:(kv + 1) * g].sum((0, 1)), atol=1e-12)
    # token 0 attends only to itself: its softmax is constant, dQ_0 = 0
    np.testing.assert_allclose(dq[0], 0, atol=1e-14)
    # the sum over keys of dS is zero for every row, so sum_j dK_j = 0 ... only when each
    # query's keys share a head; check the per-head identity sum_i dQ_i . q_i = sum_j dK_j . k_j
    lhs = float((dq * q).sum())
    rhs = float((dk * k).sum())
    assert abs(lhs - rhs) <= 1e-10 * max(1.0, abs(lhs))


def test_delta_is_row_dot_product():
    do, o = _rand((5, 3, 4), 10), _rand((5, 3, 4), 11)
    d = oracle.delta_rows(do, o)
    for h in range(3):
        for i in range(5):
            assert abs(d[h, i] - float(np.dot(do[i, h], o[i, h]))) < 1e-14


def test_delta_equals_probability_weighted_scores():
    """Delta_i = sum_d dO_i,d O_i,d must equal sum_j P_ij (dO_i . v_j), with P taken
    from a library softmax of the scores (scipy), not from the oracle's forward:
    a different route to the same row term, which a wrong index, operand or
    reduction axis in delta_rows would break."""
    from scipy.special import softmax
    n, hq, hkv, d = 9, 4, 2, 6
    q, k, v, do = _rand((n, hq, d), 20), _rand((n, hkv, d), 21), _rand((n, hkv, d), 22), _rand((n, hq, d), 23)
    pos = np.arange(n)
    vis = oracle.visibility(pos, pos)
    o, _ = oracle.attention_partial(q, k, v, vis, 0.4)
    delta = oracle.delta_rows(do, o)
    g = hq // hkv
    for h in range(hq):
        s = np.where(vis, 0.4 * q[:, h] @ k[:, h // g].T, -np.inf)
        p = softmax(s, axis=1)
        want = (p * (do[:, h] @ v[:, h // g].T)).sum(axis=1)
        np.testing.assert_allclose(delta[h], want, rtol=0, atol=1e-12)


def test_delta_makes_dq_vanish_for_identical_keys():
    """With every key identical, the scores of a row do not depend on which key
    they belong to, so dQ = scale * sum_j dS_ij k = 0 exactly when Delta is the
    row sum of P (dO . v): Delta from delta_rows of the oracle's own output gives
    dQ = 0, and a perturbed Delta does not."""
    n, hq, hkv, d = 12, 2, 1, 5
    q, v, do = _rand((n, hq, d), 30), _rand((n, hkv, d), 31), _rand((n, hq, d), 32)
    k = np.broadcast_to(_rand((1, hkv, d), 33), (n, hkv, d)).copy()
    pos = np.arange(n)
    vis = oracle.visibility(pos, pos)
    o, lse = oracle.attention_partial(q, k, v, vis, 0.7)
    delta = oracle.delta_rows(do, o)
    dq, _, _ = oracle.attention_backward_partial(q, k, v, do, lse, delta, vis, 0.7)
    np.testing.assert_allclose(dq, 0, atol=1e-12)
    dq_bad, _, _ = oracle.attention_backward_partial(q, k, v, do, lse, delta + 0.1, vis, 0.7)
    assert np.abs(dq_bad).max() > 1e-3
