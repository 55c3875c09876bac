"""GPU parity of sliding-window layers (forward, backward, block maps) against the
float64 oracle, through the C ABI.  Window layers are the extension the MaxText
page names for models such as Gemma; with a window inside one chunk only the
rank's own block and its ring neighbours' are exchanged and computed."""
import numpy as np
import pytest

import oracle
from context_long_attention_amd import inputs
from tests.gpu_common import RankInputs, assert_lse_close, assert_o_close, note, sampled_rows, widen

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _needs_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from context_long_attention_amd import cpattn
    cpattn.lib()


def _check_rank(w, rank, cu=None, backward=True):
    """Forward (per step, merged, fused) and backward of one rank against the oracle,
    plus the kernel's own block map on every step."""
    from context_long_attention_amd import cpattn
    from context_long_attention_amd.ring import RankRing
    note(f"window {w.name} S={w.seq_len} R={w.cp} Hq={w.hq} Hkv={w.hkv} D={w.dim} W={w.window} rank={rank} "
         f"docs={cu is not None}")
    inp = RankInputs(w, rank, want_do=backward)
    ring = RankRing(w, rank, cu)
    sched = ring.schedule()
    blocks = [inp.kv64[s] for s in sched]
    o, lse, steps = ring.forward(inp.q, inp.kv_of_source, keep_steps=True)
    of, lf, _ = ring.forward(inp.q, inp.kv_of_source)  # fused, empty steps skipped
    torch.cuda.synchronize()
    ro, rl, rsteps = oracle.rank_forward(inp.q64, inp.qpos, blocks, cu, w.scale, window=w.window)
    live = np.isfinite(rl).T
    assert_o_close(o.cpu().numpy(), ro, f"merged O rank {rank}", live)
    assert_lse_close(lse.cpu().numpy(), rl, f"merged LSE rank {rank}")
    assert_o_close(of.cpu().numpy(), ro, f"fused O rank {rank}", live)
    assert_lse_close(lf.cpu().numpy(), rl, f"fused LSE rank {rank}")
    for t, ((ot, lt), (rot, rlt)) in enumerate(zip(steps, rsteps)):
        assert_o_close(ot.cpu().numpy(), rot, f"O_t rank {rank} step {t}", np.isfinite(rlt).T)
        assert_lse_close(lt.cpu().numpy(), rlt, f"LSE_t rank {rank} step {t}")
    bm, bn = cpattn.cp_tile_shape(w.hq, w.hkv, w.dim)
    for t in range(w.cp):
        p = ring.problem(t)
        nq, nk = cpattn.cp_block_map_size(p)
        tm = torch.full((nq, nk), 255, dtype=torch.uint8, device="cuda")
        k, v = inp.kv_of_source(sched[t])
        o_t = torch.empty_like(o)
        l_t = torch.empty_like(lse)
        cpattn.cp_attn_fwd_step(p, inp.q, k, v, o_t, l_t, tile_map=tm)
        qseg = [(int(p.q_seg[i].pos0), int(p.q_seg[i].len)) for i in range(p.n_q_seg)]
        kseg = [(int(p.kv_seg[j].pos0), int(p.kv_seg[j].len)) for j in range(p.n_kv_seg)]
        ref = oracle.tile_map(qseg, kseg, bm, bn, cu, w.window)
        assert np.array_equal(tm.cpu().numpy(), ref), f"kernel block map differs at step {t}"
    if not backward:
        return o, lse, None, None
    dq, per_step = ring.backward(inp.q, inp.do, of, lf, inp.kv_of_source)
    torch.cuda.synchronize()
    rdq, rsteps_b, _ = oracle.rank_backward(inp.q64, inp.qpos, inp.do64, ro, rl, blocks, cu, w.scale,
                                            window=w.window)
    assert_o_close(dq.cpu().numpy(), rdq, f"dQ rank {rank}")
    for t, ((src, dk, dv), (rdk, rdv)) in enumerate(zip(per_step, rsteps_b)):
        assert src == sched[t]
        assert_o_close(dk.cpu().numpy(), rdk, f"dK rank {rank} step {t}")
        assert_o_close(dv.cpu().numpy(), rdv, f"dV rank {rank} step {t}")
    return o, lse, dq, per_step


@pytest.mark.parametrize("name", ["tiny_window", "tiny_window_wide"])
def test_tiny_window_every_rank_equals_banded_attention(name):
    """All ranks x steps; the scattered outputs and per-source gradient sums equal
    full attention and its gradient under the band mask."""
    w = inputs.WORKLOADS[name]
    S, R, c = w.seq_len, w.cp, w.chunk
    o_g = np.zeros((S, w.hq, w.dim))
    l_g = np.zeros((w.hq, S))
    dq_g = np.zeros((S, w.hq, w.dim))
    dk_g = np.zeros((S, w.hkv, w.dim))
    dv_g = np.zeros((S, w.hkv, w.dim))
    for r in range(R):
        o, lse, dq, per_step = _check_rank(w, r)
        pos = oracle.zigzag_positions(S, R, r)
        o_g[pos] = o.cpu().numpy()
        l_g[:, pos] = lse.cpu().numpy()
        dq_g[pos] = dq.cpu().numpy()
        for src, dk, dv in per_step:
            kpos = oracle.zigzag_positions(S, R, src)
            dk_g[kpos] += dk.cpu().numpy()
            dv_g[kpos] += dv.cpu().numpy()
    rb = lambda seed, h: inputs.round_bf16(inputs.chunks_normal(seed, range(2 * R), c, h, w.dim)).astype(np.float64)
    q, k, v, do = rb(inputs.SEED_Q, w.hq), rb(inputs.SEED_K, w.hkv), rb(inputs.SEED_V, w.hkv), rb(inputs.SEED_DO, w.hq)
    pos = np.arange(S)
    vis = oracle.visibility(pos, pos, window=w.window)
    ro, rl = oracle.attention_partial(q, k, v, vis, w.scale)
    assert_o_close(o_g, ro, "scattered O")
    assert_lse_close(l_g, rl, "scattered LSE")
    rdq, rdk, rdv = oracle.attention_backward_partial(q, k, v, do, rl, oracle.delta_rows(do, ro), vis, w.scale)
    assert_o_close(dq_g, rdq, "full dQ")
    assert_o_close(dk_g, rdk, "full dK")
    assert_o_close(dv_g, rdv, "full dV")


WINDOW_RAGGED = [
    # name, S, R, Hq, Hkv, D, window   (chunks that are not multiples of the tiles)
    ("g4_d128_w37", 2 * 2 * 100, 2, 8, 2, 128, 37),
    ("g1_d64_w100", 2 * 3 * 77, 3, 4, 4, 64, 100),
    ("g16_d64_w1", 2 * 4 * 33, 4, 16, 1, 64, 1),
    ("g2_d128_w200", 2 * 2 * 90, 2, 6, 3, 128, 200),
    ("g4_d128_w64", 2 * 4 * 192, 4, 8, 2, 128, 64),
]


@pytest.mark.parametrize("name,S,R,hq,hkv,d,window", WINDOW_RAGGED, ids=[r[0] for r in WINDOW_RAGGED])
def test_window_ragged_shapes(name, S, R, hq, hkv, d, window):
    w = inputs.Workload(name, S, R, hq, hkv, d, backward=True, window=window)
    for r in sorted({0, R // 2, R - 1}):
        _check_rank(w, r)


def test_window_one_returns_own_value():
    """window = 1: every row sees only itself, so O equals its own (bf16) value row
    (up to the rounding of the one-term normalisation)."""
    w = inputs.Workload("w1", 2 * 2 * 96, 2, 8, 2, 128, backward=False, window=1)
    for r in range(w.cp):
        o, lse, _, _ = _check_rank(w, r, backward=False)
        inp = RankInputs(w, r)
        v = widen(inp.kv_bits[r][1])
        g = w.hq // w.hkv
        np.testing.assert_allclose(o.cpu().numpy(), v[:, np.arange(w.hq) // g], rtol=1e-6, atol=1e-7)


def test_window_with_packed_documents():
    cu = np.array([0, 1, 2, 130, 131, 300, 301, 520, 767, 768], dtype=np.int32)
    w = inputs.Workload("packed_window", 768, 4, 8, 2, 128, backward=True, packed=True, window=70)
    for r in range(w.cp):
        _check_rank(w, r, cu)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("rank", [0, 3, 7])
def test_llama3_8b_window4k_full_size(rank):
    """Hq=32, Hkv=8, D=128, a 4K window over S=128K at CP=8 (local 16K): only the
    rank's own and its neighbours' blocks are live.  For one whole GQA group (KV head
    rank mod 8) every local row's O, LSE and dQ and every live step's dK/dV of every
    key against the float64 oracle, whose backward starts from its own O and LSE;
    for all heads, sampled rows of O, LSE and dQ."""
    from context_long_attention_amd.ring import RankRing
    from tests.gpu_common import GroupReference, gqa_heads
    w = inputs.WORKLOADS["llama3_8b_window4k"]
    ring = RankRing(w, rank)
    sched = ring.schedule()
    live = [t for t in range(w.cp) if ring.source_live(sched[t])]
    expect = {0} | ({1} if rank > 0 else set()) | ({w.cp - 1} if rank < w.cp - 1 else set())
    assert set(live) == expect
    kvh = rank % w.hkv
    heads = gqa_heads(kvh, w.hq, w.hkv)
    h0, h1 = heads[0], heads[-1] + 1
    note(f"window {w.name} full size rank={rank} live steps={live} whole group of KV head {kvh}")
    inp = RankInputs(w, rank, sources=sorted({sched[t] for t in live}), want_do=True)
    with GroupReference(inp, [sched[t] for t in live], heads, window=w.window, backward=True) as ref:
        o, lse, _ = ring.forward(inp.q, inp.kv_of_source)
        dq, per_step = ring.backward(inp.q, inp.do, o, lse, inp.kv_of_source)
        torch.cuda.synchronize()
        ro, rl = ref.forward()
        assert_o_close(o[:, h0:h1].cpu().numpy(), ro, f"window O heads {h0}..{h1 - 1}")
        assert_lse_close(lse[h0:h1].cpu().numpy(), rl, f"window LSE heads {h0}..{h1 - 1}")
        rdq, rsteps = ref.backward()
        assert_o_close(dq[:, h0:h1].cpu().numpy(), rdq, f"window dQ heads {h0}..{h1 - 1}")
        for i, t in enumerate(live):
            src, dk, dv = per_step[t]
            assert src == sched[t]
            rdk, rdv = rsteps[i][kvh]
            assert_o_close(dk[:, kvh].cpu().numpy(), rdk, f"window dK KV head {kvh} step {t}")
            assert_o_close(dv[:, kvh].cpu().numpy(), rdv, f"window dV KV head {kvh} step {t}")
    rows = sampled_rows(w.local, w.chunk, 24, rank + 11)
    q_rows, do_rows = widen(inp.q_bits[rows]), widen(inp.do_bits[rows])
    blocks = lambda: inp.blocks([sched[t] for t in live])
    ro, rl, _ = oracle.rank_forward(q_rows, inp.qpos[rows], blocks(), None, w.scale, window=w.window)
    assert_o_close(o[rows].cpu().numpy(), ro, "window O")
    assert_lse_close(lse[:, rows].cpu().numpy(), rl, "window LSE")
    rdq, _, _ = oracle.rank_backward(q_rows, inp.qpos[rows], do_rows, ro, rl, blocks(), None, w.scale,
                                     window=w.window)
    assert_o_close(dq[rows].cpu().numpy(), rdq, "window dQ")
    for t in range(w.cp):
        if t not in live:
            _, dk, dv = per_step[t]
            assert torch.all(dk == 0).item() and torch.all(dv == 0).item()
