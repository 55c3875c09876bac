"""Full-size GPU parity of the Llama-3-405B-shaped forward and the packed-document
Llama-3-8B training step (forward and backward), on sampled outputs that the
oracle computes one by one from every key they depend on."""
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


def _protocol_rows(w, seed):
    """The row sample of the Llama-3-405B protocol: in each of the two zigzag query
    chunks, its first and last 256 rows and 1024 uniform rows (seeded)."""
    rng = np.random.default_rng(seed)
    c = w.chunk
    rows = []
    for base in (0, c):
        rows += [np.arange(base, base + 256), np.arange(base + c - 256, base + c), base + rng.integers(0, c, 1024)]
    return np.unique(np.concatenate(rows))


@pytest.mark.timeout(900)
def test_llama3_405b_forward_full_size_sampled():
    """Hq=128, Hkv=8 (G=16), D=128: rank 0's share of S=1M at CP=16 (local 64K), 16
    ring steps of 64K-token KV blocks.  On the protocol's row sample (per query chunk
    the first and last 256 rows and 1024 uniform rows), all 128 heads: the final
    O/LSE of the bench's fused ring, and every step's partial (O_t, LSE_t) recomputed
    with the non-merging step kernel, against the float64 oracle (evaluated in the
    worker pool; each row sees every key it depends on)."""
    from context_long_attention_amd import cpattn
    from context_long_attention_amd.ring import RankRing
    from tests import oracle_par
    w = inputs.WORKLOADS["llama3_405b_fwd"]
    inp = RankInputs(w, 0)
    ring = RankRing(w, 0)
    sched = ring.schedule()
    rows = _protocol_rows(w, 3)
    note(f"fwd {w.name} full size rank 0, {len(rows)} sampled rows")
    with oracle_par.Shared(inp.q_bits[rows], inp.qpos[rows], {s: inp.kv_bits[s] for s in sched},
                           {s: inp.kpos[s] for s in sched}, w.scale) as sh:
        ref = oracle_par.Forward(sh, range(w.hq), sched, keep_steps=True)
        o, lse, _ = ring.forward(inp.q, inp.kv_of_source, keep_steps=False)
        torch.cuda.synchronize()
        rows_dev = torch.from_numpy(rows).cuda()
        got_o, got_l = o.index_select(0, rows_dev).cpu().numpy(), lse.index_select(1, rows_dev).cpu().numpy()
        assert not torch.isnan(o).any().item()
        o_t = torch.empty_like(o)
        l_t = torch.empty_like(lse)
        steps = []
        for t in range(w.cp):
            k, v = inp.kv_of_source(sched[t])
            cpattn.cp_attn_fwd_step(ring.problem(t), inp.q, k, v, o_t, l_t)
            steps.append((o_t.index_select(0, rows_dev).cpu().numpy(), l_t.index_select(1, rows_dev).cpu().numpy()))
        del o, lse, o_t, l_t
        ro, rl, rsteps = ref.result()
    assert_o_close(got_o, ro, "405B O sampled rows")
    assert_lse_close(got_l, rl, "405B LSE sampled rows")
    for t, ((go, gl), (rot, rlt)) in enumerate(zip(steps, rsteps)):
        assert_lse_close(gl, rlt, f"405B LSE_t step {t}")
        assert_o_close(go, rot, f"405B O_t step {t}", np.isfinite(rlt).T)


def _packed_setup():
    """Document layout of the packed workload and the visible pairs of every (rank, step)."""
    from context_long_attention_amd.ring import RankRing
    w = inputs.WORKLOADS["llama3_8b_packed"]
    cu = w.cu_seqlens()
    pairs = np.zeros((w.cp, w.cp), dtype=np.int64)
    for r in range(w.cp):
        ring = RankRing(w, r, cu, device="cpu")
        for t in range(w.cp):
            pairs[r, t] = ring.step_pairs(t)
    return w, cu, pairs


@pytest.fixture(scope="module")
def packed():
    return _packed_setup()


@pytest.mark.timeout(900)
@pytest.mark.parametrize("which", ["rank0", "max_work"])
def test_llama3_8b_packed_fwd_bwd_full_size(packed, which):
    """S=2M at CP=64 (local 32K), lognormal documents, doc masks with fully masked
    tiles skipped; forward and backward on the GPU over all 64 ring steps.  For one
    whole GQA group (KV head 2 on rank 0, KV head 6 on the rank with the most
    visible pairs) every local row's O, LSE and dQ and every live step's dK/dV of
    every key, against the float64 oracle, whose backward starts from its own O and
    LSE; for all heads, sampled rows of O, LSE and dQ."""
    from context_long_attention_amd import cpattn
    from context_long_attention_amd.ring import RankRing
    from tests.gpu_common import GroupReference, gqa_heads
    w, cu, pairs = packed
    rank = 0 if which == "rank0" else int(np.argmax(pairs.sum(axis=1)))
    kvh = 2 if which == "rank0" else 6
    heads = gqa_heads(kvh, w.hq, w.hkv)
    h0, h1 = heads[0], heads[-1] + 1
    ring = RankRing(w, rank, cu)
    sched = ring.schedule()
    live_steps = [t for t in range(w.cp) if pairs[rank, t] > 0]
    sources = sorted({sched[t] for t in live_steps})
    note(f"packed {w.name} rank={rank} live steps={len(live_steps)} pairs={int(pairs[rank].sum())} "
         f"whole group of KV head {kvh}")
    inp = RankInputs(w, rank, sources=sources, want_do=True)
    with GroupReference(inp, [sched[t] for t in live_steps], heads, cu, backward=True) as ref:
        o, lse, _ = ring.forward(inp.q, inp.kv_of_source)
        dq, per_step = ring.backward(inp.q, inp.do, o, lse, inp.kv_of_source)
        torch.cuda.synchronize()
        ro, rl = ref.forward()
        assert_o_close(o[:, h0:h1].cpu().numpy(), ro, f"packed O heads {h0}..{h1 - 1}", np.isfinite(rl).T)
        assert_lse_close(lse[h0:h1].cpu().numpy(), rl, f"packed LSE heads {h0}..{h1 - 1}")
        rdq, rsteps = ref.backward()
        assert_o_close(dq[:, h0:h1].cpu().numpy(), rdq, f"packed dQ heads {h0}..{h1 - 1}")
        for i, t in enumerate(live_steps):
            src, dk, dv = per_step[t]
            assert src == sched[t]
            rdk, rdv = rsteps[i][kvh]
            assert_o_close(dk[:, kvh].cpu().numpy(), rdk, f"packed dK KV head {kvh} step {t}")
            assert_o_close(dv[:, kvh].cpu().numpy(), rdv, f"packed dV KV head {kvh} step {t}")

    rows = sampled_rows(w.local, w.chunk, 24, rank + 1)
    q_rows, do_rows = widen(inp.q_bits[rows]), widen(inp.do_bits[rows])
    blocks = lambda: inp.blocks([sched[t] for t in live_steps])
    ro, rl, _ = oracle.rank_forward(q_rows, inp.qpos[rows], blocks(), cu, w.scale)
    assert_o_close(o[rows].cpu().numpy(), ro, "packed O", np.isfinite(rl).T)
    assert_lse_close(lse[:, rows].cpu().numpy(), rl, "packed LSE")
    rdq, _, _ = oracle.rank_backward(q_rows, inp.qpos[rows], do_rows, ro, rl, blocks(), cu, w.scale)
    assert_o_close(dq[rows].cpu().numpy(), rdq, "packed dQ")
    busiest = sorted(live_steps, key=lambda t: -pairs[rank, t])[:2]
    rng = np.random.default_rng(7)
    # steps with nothing visible leave zero gradients for their blocks
    for t in range(w.cp):
        if pairs[rank, t] == 0:
            _, dk, dv = per_step[t]
            assert torch.all(dk == 0).item() and torch.all(dv == 0).item()
    # block map the kernel used on the busiest step, against the host rule everywhere and
    # against the oracle's brute force on sampled query-tile rows
    t = busiest[0]
    p = ring.problem(t)
    nq, nk = cpattn.cp_block_map_size(p)
    tm = torch.full((nq, nk), 255, dtype=torch.uint8, device="cuda")
    k, v = inp.kv_of_source(sched[t])
    o_t = torch.empty_like(o)
    l_t = torch.empty_like(lse)
    cpattn.cp_attn_fwd_step(p, inp.q, k, v, o_t, l_t, tile_map=tm)
    got = tm.cpu().numpy()
    host = cpattn.cp_block_map(ring.problem(t, host_docs=True))
    assert np.array_equal(got, host)
    bm, bn = cpattn.cp_tile_shape(w.hq, w.hkv, w.dim)
    kseg = [(int(p.kv_seg[j].pos0), int(p.kv_seg[j].len)) for j in range(p.n_kv_seg)]
    tiles_per_seg = w.chunk // bm
    for qt in np.unique(np.concatenate([[0, nq - 1], rng.integers(0, nq, 6)])):
        seg = 0 if qt < tiles_per_seg else 1
        pos0 = int(p.q_seg[seg].pos0) + (qt - seg * tiles_per_seg) * bm
        ref = oracle.tile_map([(pos0, bm)], kseg, bm, bn, cu)
        assert np.array_equal(got[qt:qt + 1], ref), f"tile map row {qt}"


def _periodic_bits(seed, rows, heads, d, period=4099):
    """bf16 bit patterns of rows that repeat with a prime period, so that no
    shift by fewer than 4099 whole 64-row tiles maps a tile onto an equal one."""
    bits = inputs.bf16_bits(inputs.chunk_normal(seed, 0, period, heads, d))
    return np.tile(bits, ((rows + period - 1) // period, 1, 1))[:rows]


@pytest.mark.timeout(900)
def test_kv_segment_just_under_the_span_limit():
    """The step kernels' one hard size limit: a KV segment spanning just under
    1 GiB (524207 rows x Hkv=8 x D=128 bf16, a ragged last tile).  With a
    256-token window, 16 query rows at the segment's start see its first tile
    and 16 rows straddling its end see only its last tiles, so every output
    depends on tiles at the two ends of the span.  Forward O/LSE, dQ and the
    dK/dV of every visible key against the oracle (which needs only those keys);
    dK/dV of all other keys exactly zero."""
    from context_long_attention_amd import cpattn
    from tests.gpu_common import _to_device, device_bf16
    hq, hkv, d, n, win = 8, 8, 128, 32, 256
    m = (1 << 30) // (hkv * d * 2) - 64 - 17
    assert m * hkv * d * 2 < (1 << 30) and m % 64 == 47
    note(f"KV span {m * hkv * d * 2} bytes")
    q64, q = device_bf16(inputs.chunk_normal(31, 0, n, hq, d))
    do64, do = device_bf16(inputs.chunk_normal(34, 0, n, hq, d))
    kbits, vbits = _periodic_bits(32, m, hkv, d), _periodic_bits(33, m, hkv, d)
    k, v = _to_device(kbits), _to_device(vbits)
    D_ = cpattn.CP_MASK_DIAG_CAUSAL
    qpos = np.concatenate([np.arange(16), np.arange(m - 8, m + 8)])
    p = cpattn.make_problem(hq, hkv, d, d ** -0.5, n, m, [(0, 0, 16), (16, m - 8, 16)], [(0, 0, m)],
                            [[D_, D_], [D_, D_]], window=win)
    o = torch.empty((n, hq, d), dtype=torch.float32, device="cuda")
    lse = torch.empty((hq, n), dtype=torch.float32, device="cuda")
    cpattn.cp_attn_fwd_step(p, q, k, v, o, lse)
    delta = torch.empty((hq, n), dtype=torch.float32, device="cuda")
    cpattn.cp_attn_bwd_prep(do, o, delta, n, hq, d)
    dq = torch.zeros((n, hq, d), dtype=torch.float32, device="cuda")
    dk = torch.full((m, hkv, d), 7.0, dtype=torch.float32, device="cuda")
    dv = torch.full((m, hkv, d), 7.0, dtype=torch.float32, device="cuda")
    cpattn.cp_attn_bwd_step(p, q, k, v, do, lse, delta, dq, dk, dv)
    torch.cuda.synchronize()
    # keys no row sees add nothing: the oracle takes only the visible ones
    keys = np.concatenate([np.arange(16), np.arange(m - 8 - win + 1, m)])
    vis = oracle.visibility(qpos, keys, None, win)
    assert vis[:, :16].any() and vis[:, 16:].any() and vis.any(axis=0).all()
    k64, v64 = widen(kbits[keys]), widen(vbits[keys])
    ro, rl = oracle.attention_partial(q64, k64, v64, vis, d ** -0.5)
    assert_o_close(o.cpu().numpy(), ro, "O at both ends of a 1 GiB KV span")
    assert_lse_close(lse.cpu().numpy(), rl, "LSE at both ends of a 1 GiB KV span")
    rdq, rdk, rdv = oracle.attention_backward_partial(q64, k64, v64, do64, rl, oracle.delta_rows(do64, ro), vis,
                                                      d ** -0.5)
    assert_o_close(dq.cpu().numpy(), rdq, "dQ at both ends of a 1 GiB KV span")
    keys_dev = torch.from_numpy(keys).cuda()
    assert_o_close(dk.index_select(0, keys_dev).cpu().numpy(), rdk, "dK of the visible keys")
    assert_o_close(dv.index_select(0, keys_dev).cpu().numpy(), rdv, "dV of the visible keys")
    rest = torch.ones(m, dtype=torch.bool, device="cuda")
    rest[keys_dev] = False
    assert torch.count_nonzero(dk[rest]).item() == 0 and torch.count_nonzero(dv[rest]).item() == 0
