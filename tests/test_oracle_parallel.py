"""The parallel whole-tensor composition used by the full-size GPU tests equals the
oracle's own rank_forward / rank_backward (CPU only).

The full-size parity tests evaluate the oracle per (query head, ring step, block
of rows) in worker processes and compose the results in the parent
(tests/oracle_par.py).  Here that composition is held against the oracle's
sequential functions on small shapes that exercise every part of it: several
row blocks, GQA groups, keys that a row block cannot see (left out of a task),
rows with no visible key in a step, packed documents and a sliding window."""
import numpy as np
import pytest

import oracle
from context_long_attention_amd import inputs
from tests import oracle_par


@pytest.fixture(scope="module", autouse=True)
def _pool():
    # small key blocks, so that the shapes below span several of them
    old = oracle_par._KEY_BLOCK
    oracle_par._KEY_BLOCK = 24
    oracle_par.pool(workers=2)
    yield
    oracle_par.shutdown()
    oracle_par._KEY_BLOCK = old


CASES = [
    # name, S, R, Hq, Hkv, D, rank, documents, window
    ("causal_r0", 2 * 4 * 48, 4, 4, 2, 16, 0, None, 0),
    ("causal_last", 2 * 4 * 48, 4, 6, 2, 8, 3, None, 0),
    ("docs", 384, 4, 4, 1, 16, 1, [0, 5, 6, 100, 101, 250, 384], 0),
    ("window", 2 * 4 * 48, 4, 4, 2, 16, 2, None, 40),
]


def _draw(w, rank):
    c, R = w.chunk, w.cp
    qa, qb = oracle.zigzag_chunks(R, rank)
    q_bits = inputs.bf16_bits(inputs.chunks_normal(inputs.SEED_Q, [qa, qb], c, w.hq, w.dim))
    do_bits = inputs.bf16_bits(inputs.chunks_normal(inputs.SEED_DO, [qa, qb], c, w.hq, w.dim))
    kv_bits, kpos = {}, {}
    for s in range(R):
        ka, kb = oracle.zigzag_chunks(R, s)
        kv_bits[s] = (inputs.bf16_bits(inputs.chunks_normal(inputs.SEED_K, [ka, kb], c, w.hkv, w.dim)),
                      inputs.bf16_bits(inputs.chunks_normal(inputs.SEED_V, [ka, kb], c, w.hkv, w.dim)))
        kpos[s] = oracle.zigzag_positions(w.seq_len, R, s)
    return q_bits, do_bits, kv_bits, kpos


@pytest.mark.parametrize("name,S,R,hq,hkv,d,rank,cu,window", CASES, ids=[c[0] for c in CASES])
def test_parallel_composition_equals_rank_functions(name, S, R, hq, hkv, d, rank, cu, window):
    w = inputs.Workload(name, S, R, hq, hkv, d, backward=True, window=window)
    cu = None if cu is None else np.asarray(cu, dtype=np.int32)
    q_bits, do_bits, kv_bits, kpos = _draw(w, rank)
    qpos = oracle.zigzag_positions(S, R, rank)
    order = [oracle.ring_source(rank, t, R) for t in range(R)]
    f64 = lambda b: inputs.bf16_to_f32(b).astype(np.float64)
    blocks = [(f64(kv_bits[s][0]), f64(kv_bits[s][1]), kpos[s]) for s in order]
    ro, rl, rsteps = oracle.rank_forward(f64(q_bits), qpos, blocks, cu, w.scale, window=window or None)
    rdq, rkv, rdelta = oracle.rank_backward(f64(q_bits), qpos, f64(do_bits), ro, rl, blocks, cu, w.scale,
                                            window=window or None)
    # a subset of heads that covers whole GQA groups, in a permuted order
    g = hq // hkv
    heads = [h for kvh in reversed(range(hkv)) for h in range(kvh * g, (kvh + 1) * g)]
    with oracle_par.Shared(q_bits, qpos, kv_bits, kpos, w.scale, cu, window, do_bits=do_bits) as sh:
        o, lse, steps = oracle_par.Forward(sh, heads, order, rows_per_task=40, keep_steps=True).result()
        np.testing.assert_allclose(o, ro[:, heads], rtol=0, atol=1e-12)
        assert np.array_equal(np.isneginf(lse), np.isneginf(rl[heads]))
        np.testing.assert_allclose(lse[np.isfinite(lse)], rl[heads][np.isfinite(lse)], rtol=0, atol=1e-12)
        for (ot, lt), (rot, rlt) in zip(steps, rsteps):
            np.testing.assert_allclose(ot, rot[:, heads], rtol=0, atol=1e-12)
            assert np.array_equal(np.isneginf(lt), np.isneginf(rlt[heads]))
        dq, per_step, delta = oracle_par.Backward(sh, heads, order, o, lse, rows_per_task=40).result()
        np.testing.assert_allclose(delta, rdelta[heads], rtol=0, atol=1e-12)
        np.testing.assert_allclose(dq, rdq[:, heads], rtol=0, atol=1e-12)
        for t, ((rdk, rdv), dkv) in enumerate(zip(rkv, per_step)):
            for kvh, (dk, dv) in dkv.items():
                np.testing.assert_allclose(dk, rdk[:, kvh], rtol=0, atol=1e-12, err_msg=f"dK step {t}")
                np.testing.assert_allclose(dv, rdv[:, kvh], rtol=0, atol=1e-12, err_msg=f"dV step {t}")
    if name == "causal_r0":  # the first chunk's rows see nothing at every step after the first
        assert all(np.isneginf(rlt[:, :w.chunk]).all() for _, rlt in rsteps[1:])
