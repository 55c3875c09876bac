"""GPU parity of the backward ring step (and delta preprocessing) against the
float64 oracle, through the C ABI."""
import numpy as np
import pytest

import oracle
from context_long_attention_amd import inputs
from tests.gpu_common import RankInputs, assert_lse_close, assert_o_close, note, widen

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _needs_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from context_long_attention_amd import cpattn
    cpattn.lib()


def _run(w, rank, cu=None):
    from context_long_attention_amd.ring import RankRing
    note(f"bwd {w.name} S={w.seq_len} R={w.cp} Hq={w.hq} Hkv={w.hkv} D={w.dim} rank={rank} docs={cu is not None}")
    inp = RankInputs(w, rank, want_do=True)
    ring = RankRing(w, rank, cu)
    o, lse, _ = ring.forward(inp.q, inp.kv_of_source)
    dq, per_step = ring.backward(inp.q, inp.do, o, lse, inp.kv_of_source)
    torch.cuda.synchronize()
    return inp, ring, o, lse, dq, per_step


def _check_rank(w, rank, cu=None):
    inp, ring, o, lse, dq, per_step = _run(w, rank, cu)
    blocks = [inp.kv64[s] for s in ring.schedule()]
    ro, rl, _ = oracle.rank_forward(inp.q64, inp.qpos, blocks, cu, w.scale)
    rdq, rsteps, rdelta = oracle.rank_backward(inp.q64, inp.qpos, inp.do64, ro, rl, blocks, cu, w.scale)
    assert_o_close(dq.cpu().numpy(), rdq, f"dQ rank {rank}")
    for t, ((src, dk, dv), (rdk, rdv)) in enumerate(zip(per_step, rsteps)):
        assert src == ring.schedule()[t]
        assert_o_close(dk.cpu().numpy(), rdk, f"dK rank {rank} step {t}")
        assert_o_close(dv.cpu().numpy(), rdv, f"dV rank {rank} step {t}")
    return dq, per_step


def test_delta_kernel():
    from context_long_attention_amd import cpattn
    from tests.gpu_common import device_bf16
    rows, hq, d = 130, 3, 128
    do64, do = device_bf16(inputs.chunk_normal(4, 0, rows, hq, d))
    o = np.random.default_rng(1).standard_normal((rows, hq, d)).astype(np.float32)
    delta = torch.empty((hq, rows), device="cuda")
    cpattn.cp_attn_bwd_prep(do, torch.from_numpy(o).cuda(), delta, rows, hq, d)
    np.testing.assert_allclose(delta.cpu().numpy(), oracle.delta_rows(do64, o), atol=1e-4)


def test_tiny_every_rank_sums_to_full_gradient():
    """All 4 ranks x 4 steps of the tiny workload: per-step dK/dV and local dQ match
    the oracle, and the per-source sums equal the full-sequence gradients."""
    w = inputs.WORKLOADS["tiny"]
    S, R, c = w.seq_len, w.cp, w.chunk
    dq_g = np.zeros((S, w.hq, w.dim))
    dk_g = np.zeros((S, w.hkv, w.dim))
    dv_g = np.zeros((S, w.hkv, w.dim))
    for r in range(R):
        dq, per_step = _check_rank(w, r)
        dq_g[oracle.zigzag_positions(S, R, r)] = dq.cpu().numpy()
        for src, dk, dv in per_step:
            kpos = oracle.zigzag_positions(S, R, src)
            dk_g[kpos] += dk.cpu().numpy()
            dv_g[kpos] += dv.cpu().numpy()
    rb = lambda seed, h: inputs.round_bf16(inputs.chunks_normal(seed, range(2 * R), c, h, w.dim)).astype(np.float64)
    q, k, v, do = rb(inputs.SEED_Q, w.hq), rb(inputs.SEED_K, w.hkv), rb(inputs.SEED_V, w.hkv), rb(inputs.SEED_DO, w.hq)
    pos = np.arange(S)
    vis = oracle.visibility(pos, pos)
    o, lse = oracle.attention_partial(q, k, v, vis, w.scale)
    rdq, rdk, rdv = oracle.attention_backward_partial(q, k, v, do, lse, oracle.delta_rows(do, o), vis, w.scale)
    assert_o_close(dq_g, rdq, "full dQ")
    assert_o_close(dk_g, rdk, "full dK")
    assert_o_close(dv_g, rdv, "full dV")


RAGGED = [
    ("g4_d128", 2 * 2 * 100, 2, 8, 2, 128),
    ("g1_d64", 2 * 3 * 77, 3, 4, 4, 64),
    ("g2_d128", 2 * 2 * 150, 2, 6, 3, 128),
    ("g16_d64", 2 * 2 * 40, 2, 16, 1, 64),
    ("g3_d128", 2 * 2 * 70, 2, 6, 2, 128),
    # chunk lengths that are multiples of the 128-key workgroup tile (unmasked full tiles)
    ("aligned_g4_d128", 2 * 2 * 512, 2, 8, 2, 128),
    ("aligned_g1_d64", 2 * 4 * 256, 4, 4, 4, 64),
    ("r16_c256", 2 * 16 * 256, 16, 8, 2, 128),
    # the Llama-3-8B head shape (Hq=32, Hkv=8) and a group of 8 at D=64
    ("hkv8_g4_d128", 2 * 2 * 96, 2, 32, 8, 128),
    ("g8_d64", 2 * 2 * 66, 2, 8, 1, 64),
]


@pytest.mark.parametrize("name,S,R,hq,hkv,d", RAGGED, ids=[r[0] for r in RAGGED])
def test_ragged_shapes(name, S, R, hq, hkv, d):
    w = inputs.Workload(name, S, R, hq, hkv, d, backward=True)
    for r in sorted({0, R - 1}):
        _check_rank(w, r)


def test_packed_documents_small():
    cu = np.array([0, 1, 2, 130, 131, 300, 301, 520, 767, 768], dtype=np.int32)
    w = inputs.Workload("packed_small", 768, 4, 8, 2, 128, backward=True, packed=True)
    for r in range(w.cp):
        _check_rank(w, r, cu)


def test_single_token_chunks():
    w = inputs.Workload("c1", 4, 2, 4, 2, 64, backward=True)
    for r in range(2):
        _check_rank(w, r)


SPLIT_CASES = [
    # name, S, R, Hq, Hkv, D, window, packed documents, rank
    ("ragged_g4_d128", 2 * 2 * 100, 2, 8, 2, 128, 0, False, 0),
    ("ragged_g1_d64", 2 * 3 * 77, 3, 4, 4, 64, 0, False, 2),
    ("aligned_g4_d128", 2 * 2 * 512, 2, 8, 2, 128, 0, False, 1),
    ("window_g4_d128", 2 * 4 * 192, 4, 8, 2, 128, 64, False, 0),
    ("packed_g4_d128", 768, 4, 8, 2, 128, 0, True, 1),
]


@pytest.mark.parametrize("name,S,R,hq,hkv,d,window,packed,rank", SPLIT_CASES, ids=[c[0] for c in SPLIT_CASES])
def test_dkdv_split_matches_oracle(name, S, R, hq, hkv, d, window, packed, rank):
    """Each key block's query tiles spread over 2, 3 or 8 workgroups, the later
    parts' sums added to dK/dV from the workspace in part order: every step's
    dK/dV match the oracle (outputs pre-filled with garbage, so every row is
    written; the workspace pre-filled with NaN, so no slot is read that was not
    written), the same bits come out of a second run, and dQ is bit-identical to
    the unsplit step."""
    from context_long_attention_amd import cpattn
    cu = np.array([0, 1, 2, 130, 131, 300, 301, 520, 767, 768], dtype=np.int32) if packed else None
    w = inputs.Workload(name, S, R, hq, hkv, d, backward=True, packed=packed, window=window)
    inp, ring, o, lse, _, _ = _run(w, rank, cu)
    sched = ring.schedule()
    blocks = [inp.kv64[s] for s in sched]
    ro, rl, _ = oracle.rank_forward(inp.q64, inp.qpos, blocks, cu, w.scale, window=window or None)
    _, rsteps, _ = oracle.rank_backward(inp.q64, inp.qpos, inp.do64, ro, rl, blocks, cu, w.scale,
                                        window=window or None)
    rows = 2 * w.chunk
    delta = torch.empty((w.hq, rows), device="cuda")
    cpattn.cp_attn_bwd_prep(inp.do, o, delta, rows, w.hq, w.dim)

    def step(p, k, v, split):
        p.kv_split = split
        need = cpattn.cp_bwd_workspace_size(p, split)
        ws = torch.full((max(need // 4, 1),), float("nan"), device="cuda") if need else None
        dq = torch.zeros((rows, w.hq, w.dim), device="cuda")
        dk = torch.full((rows, w.hkv, w.dim), 7.0, device="cuda")
        dv = torch.full_like(dk, 7.0)
        cpattn.cp_attn_bwd_step(p, inp.q, k, v, inp.do, lse, delta, dq, dk, dv, workspace=ws)
        torch.cuda.synchronize()
        return dq, dk, dv

    for t, src in enumerate(sched):
        k, v = inp.kv_of_source(src)
        p = ring.problem(t, src)
        outs = {}
        for split in (1, 2, 3, 8):
            note(f"split {name} step {t} kv_split={split}")
            outs[split] = step(p, k, v, split)
            rdk, rdv = rsteps[t]
            assert_o_close(outs[split][1].cpu().numpy(), rdk, f"dK step {t} split {split}")
            assert_o_close(outs[split][2].cpu().numpy(), rdv, f"dV step {t} split {split}")
            again = step(p, k, v, split)
            for a, b, what in zip(again, outs[split], ("dQ", "dK", "dV")):
                assert torch.equal(a, b), f"{what} differs between two runs with split {split} at step {t}"
        for split in (2, 3, 8):
            assert torch.equal(outs[split][0], outs[1][0]), f"dQ changed with split {split} at step {t}"
            for a, b in zip(outs[split][1:], outs[1][1:]):
                assert (a - b).abs().max().item() <= 1e-4 * max(1.0, b.abs().max().item())


@pytest.mark.timeout(600)
@pytest.mark.parametrize("rank,kvh", [(0, 5), (15, 2)])
def test_llama3_8b_fwd_bwd_full_size(rank, kvh):
    """Llama-3-8B shape, one rank's share of S=256K at CP=16 (local 16K), 16 ring
    steps forward and backward on the GPU (rank 0: the first and last chunks; rank
    15: the two middle ones).  For the query heads of one KV head (a whole GQA
    group) every local row's O, LSE and dQ and every step's dK/dV of every key of
    the visiting block, against the float64 oracle, whose backward starts from its
    own O and LSE.  For all 32 heads, sampled rows of O, LSE and dQ."""
    from tests.gpu_common import GroupReference, gqa_heads
    w = inputs.WORKLOADS["llama3_8b_fwdbwd"]
    heads = gqa_heads(kvh, w.hq, w.hkv)
    from context_long_attention_amd.ring import RankRing
    note(f"bwd {w.name} full size rank={rank} whole group of KV head {kvh}")
    inp = RankInputs(w, rank, want_do=True)
    ring = RankRing(w, rank)
    sched = ring.schedule()
    with GroupReference(inp, sched, heads, backward=True) as ref:
        o, lse, _ = ring.forward(inp.q, inp.kv_of_source)
        dq, per_step = ring.backward(inp.q, inp.do, o, lse, inp.kv_of_source)
        torch.cuda.synchronize()
        h0, h1 = heads[0], heads[-1] + 1
        ro, rl = ref.forward()
        assert_o_close(o[:, h0:h1].cpu().numpy(), ro, f"O heads {h0}..{h1 - 1}, all rows")
        assert_lse_close(lse[h0:h1].cpu().numpy(), rl, f"LSE heads {h0}..{h1 - 1}, all rows")
        rdq, rsteps = ref.backward()
        assert_o_close(dq[:, h0:h1].cpu().numpy(), rdq, f"dQ heads {h0}..{h1 - 1}, all rows")
        for t, (src, dk, dv) in enumerate(per_step):
            assert src == sched[t]
            rdk, rdv = rsteps[t][kvh]
            assert_o_close(dk[:, kvh].cpu().numpy(), rdk, f"dK KV head {kvh} step {t}, all keys")
            assert_o_close(dv[:, kvh].cpu().numpy(), rdv, f"dV KV head {kvh} step {t}, all keys")
    # every head on sampled rows (the oracle sees every key they depend on)
    rng = np.random.default_rng(11)
    c, L = w.chunk, w.local
    rows = np.unique(np.concatenate([[0, 1, c - 1, c, c + 1, L - 1], rng.integers(0, L, 20)]))
    blocks = [inp.kv64[s] for s in sched]
    q_rows, do_rows = widen(inp.q_bits[rows]), widen(inp.do_bits[rows])
    ro, rl, _ = oracle.rank_forward(q_rows, inp.qpos[rows], blocks, None, w.scale)
    assert_o_close(o[rows].cpu().numpy(), ro, "O sampled rows")
    assert_lse_close(lse[:, rows].cpu().numpy(), rl, "LSE sampled rows")
    rdq, _, _ = oracle.rank_backward(q_rows, inp.qpos[rows], do_rows, ro, rl, blocks, None, w.scale)
    assert_o_close(dq[rows].cpu().numpy(), rdq, "dQ sampled rows")


@pytest.mark.parametrize("masks", ["dead_first", "dead_second", "all_dead"])
def test_dead_query_segments_left_out(masks):
    """Query segments that pair only with SKIP are left out of the merging forward
    launch and of the dQ launch: their rows keep the accumulator and dQ bit for
    bit, while the live segment (moved to the front when the first is dead) gets
    the oracle's result, and dK/dV hold only the live rows' terms."""
    from context_long_attention_amd import cpattn
    from tests.gpu_common import device_bf16
    hq, hkv, d, na, nb, m = 8, 2, 128, 64, 96, 128
    n = na + nb
    note(f"dead query segments {masks}")
    q64, q = device_bf16(inputs.chunk_normal(21, 0, n, hq, d))
    do64, do = device_bf16(inputs.chunk_normal(24, 0, n, hq, d))
    k64, k = device_bf16(inputs.chunk_normal(22, 0, m, hkv, d))
    v64, v = device_bf16(inputs.chunk_normal(23, 0, m, hkv, d))
    F, S_ = cpattn.CP_MASK_FULL, cpattn.CP_MASK_SKIP
    live_a, live_b = {"dead_first": (False, True), "dead_second": (True, False), "all_dead": (False, False)}[masks]
    mk = [[F if live_a else S_, S_], [F if live_b else S_, S_]]
    p = cpattn.make_problem(hq, hkv, d, d ** -0.5, n, m, [(0, 2000, na), (na, 5000, nb)], [(0, 1000, m)], mk)
    live = np.zeros(n, dtype=bool)
    live[:na], live[na:] = live_a, live_b
    vis = np.repeat(live[:, None], m, axis=1)
    rng = np.random.default_rng(9)
    # forward: merge into a random valid accumulator
    o0 = rng.standard_normal((n, hq, d)).astype(np.float32)
    l0 = (rng.standard_normal((hq, n)) * 3).astype(np.float32)
    o_acc, l_acc = torch.from_numpy(o0.copy()).cuda(), torch.from_numpy(l0.copy()).cuda()
    cpattn.cp_attn_fwd_step_merge(p, q, k, v, o_acc, l_acc)
    ro_t, rl_t = oracle.attention_partial(q64, k64, v64, vis, d ** -0.5)
    ro, rl = oracle.merge(o0.astype(np.float64), l0.astype(np.float64), ro_t, rl_t)
    got_o, got_l = o_acc.cpu().numpy(), l_acc.cpu().numpy()
    assert np.array_equal(got_o[~live], o0[~live]) and np.array_equal(got_l[:, ~live], l0[:, ~live])
    # asking for the tile map launches every query tile: same results bit for bit, and the map
    nq, nk = cpattn.cp_block_map_size(p)
    tm = torch.full((nq, nk), 255, dtype=torch.uint8, device="cuda")
    o_map, l_map = torch.from_numpy(o0.copy()).cuda(), torch.from_numpy(l0.copy()).cuda()
    cpattn.cp_attn_fwd_step_merge(p, q, k, v, o_map, l_map, tile_map=tm)
    assert np.array_equal(o_map.cpu().numpy(), got_o) and np.array_equal(l_map.cpu().numpy(), got_l)
    bm, bn = cpattn.cp_tile_shape(hq, hkv, d)
    ref_map = np.concatenate([oracle.tile_map([(2000, na)], [(1000, m)], bm, bn) if live_a else
                              np.zeros((-(-na // bm), nk), dtype=np.uint8),
                              oracle.tile_map([(5000, nb)], [(1000, m)], bm, bn) if live_b else
                              np.zeros((-(-nb // bm), nk), dtype=np.uint8)])
    assert np.array_equal(tm.cpu().numpy(), ref_map)
    if live.any():
        assert_o_close(got_o[live], ro[live], "merged O of the live segment")
        assert_lse_close(got_l[:, live], rl[:, live], "merged LSE of the live segment")
    # backward from the step's own LSE (P <= 1) and a small random Delta
    lse = torch.from_numpy(np.where(np.isfinite(rl_t), rl_t, 0.0).astype(np.float32)).cuda()
    delta64 = 0.1 * rng.standard_normal((hq, n))
    delta = torch.from_numpy(delta64.astype(np.float32)).cuda()
    dq0 = rng.standard_normal((n, hq, d)).astype(np.float32)
    dq = torch.from_numpy(dq0.copy()).cuda()
    dk = torch.full((m, hkv, d), 7.0, device="cuda")
    dv = torch.full((m, hkv, d), 7.0, device="cuda")
    cpattn.cp_attn_bwd_step(p, q, k, v, do, lse, delta, dq, dk, dv)
    torch.cuda.synchronize()
    rdq, rdk, rdv = oracle.attention_backward_partial(q64, k64, v64, do64, lse.cpu().numpy().astype(np.float64),
                                                      delta.cpu().numpy().astype(np.float64), vis, d ** -0.5)
    got_dq = dq.cpu().numpy()
    assert np.array_equal(got_dq[~live], dq0[~live])
    if live.any():
        assert_o_close(got_dq[live], dq0[live] + rdq[live], "dQ of the live segment")
    assert_o_close(dk.cpu().numpy(), rdk, "dK")
    assert_o_close(dv.cpu().numpy(), rdv, "dV")


DETERMINISM_CASES = [
    # name, S, R, Hq, Hkv, D, window, documents, rank
    ("dense", 2 * 4 * 96, 4, 8, 2, 128, 0, None, 1),
    ("packed", 768, 4, 8, 2, 128, 0, [0, 1, 2, 130, 131, 300, 301, 520, 767, 768], 1),
    ("window", 2 * 4 * 192, 4, 8, 2, 128, 64, None, 0),
]


@pytest.mark.parametrize("name,S,R,hq,hkv,d,window,cu,rank", DETERMINISM_CASES, ids=[c[0] for c in DETERMINISM_CASES])
def test_ring_is_deterministic(name, S, R, hq, hkv, d, window, cu, rank):
    """Two runs of the same forward and backward ring, with the library's default
    dK/dV split (which splits some steps of each case), give bit-identical O, LSE,
    dQ and per-step dK/dV."""
    from context_long_attention_amd.ring import RankRing
    cu = None if cu is None else np.asarray(cu, dtype=np.int32)
    w = inputs.Workload(name, S, R, hq, hkv, d, backward=True, packed=cu is not None, window=window)
    note(f"determinism {name}")
    inp = RankInputs(w, rank, want_do=True)
    runs = []
    for _ in range(2):
        ring = RankRing(w, rank, cu)
        assert max(ring.kv_split(s) for s in ring.schedule()) > 1
        o, lse, _ = ring.forward(inp.q, inp.kv_of_source)
        dq, steps = ring.backward(inp.q, inp.do, o, lse, inp.kv_of_source)
        torch.cuda.synchronize()
        runs.append([o.cpu().numpy(), lse.cpu().numpy(), dq.cpu().numpy()]
                    + [x.cpu().numpy() for _, dk, dv in steps for x in (dk, dv)])
    for a, b in zip(*runs):
        assert np.array_equal(a, b)


def test_max_query_heads():
    """Hq = 8192 (the largest the library accepts), Hkv = 2048: head indices,
    head blocks and the per-head strides at their limits, with ragged causal
    tiles; forward O/LSE and dQ/dK/dV against the oracle."""
    from context_long_attention_amd import cpattn
    from tests.gpu_common import device_bf16
    hq, hkv, d, n, m = 8192, 2048, 64, 100, 130
    note("max query heads")
    q64, q = device_bf16(inputs.chunk_normal(41, 0, n, hq, d))
    do64, do = device_bf16(inputs.chunk_normal(44, 0, n, hq, d))
    k64, k = device_bf16(inputs.chunk_normal(42, 0, m, hkv, d))
    v64, v = device_bf16(inputs.chunk_normal(43, 0, m, hkv, d))
    D_ = cpattn.CP_MASK_DIAG_CAUSAL
    p = cpattn.make_problem(hq, hkv, d, d ** -0.5, n, m, [(0, 30, n)], [(0, 0, m)], [[D_, D_], [D_, D_]])
    o = torch.empty((n, hq, d), dtype=torch.float32, device="cuda")
    lse = torch.empty((hq, n), dtype=torch.float32, device="cuda")
    cpattn.cp_attn_fwd_step(p, q, k, v, o, lse)
    delta = torch.empty((hq, n), dtype=torch.float32, device="cuda")
    cpattn.cp_attn_bwd_prep(do, o, delta, n, hq, d)
    dq = torch.zeros((n, hq, d), dtype=torch.float32, device="cuda")
    dk = torch.empty((m, hkv, d), dtype=torch.float32, device="cuda")
    dv = torch.empty((m, hkv, d), dtype=torch.float32, device="cuda")
    cpattn.cp_attn_bwd_step(p, q, k, v, do, lse, delta, dq, dk, dv)
    torch.cuda.synchronize()
    vis = oracle.visibility(np.arange(30, 30 + n), np.arange(m))
    ro, rl = oracle.attention_partial(q64, k64, v64, vis, d ** -0.5)
    assert_o_close(o.cpu().numpy(), ro, "O at Hq = 8192")
    assert_lse_close(lse.cpu().numpy(), rl, "LSE at Hq = 8192")
    rdq, rdk, rdv = oracle.attention_backward_partial(q64, k64, v64, do64, rl, oracle.delta_rows(do64, ro), vis,
                                                      d ** -0.5)
    assert_o_close(dq.cpu().numpy(), rdq, "dQ at Hq = 8192")
    assert_o_close(dk.cpu().numpy(), rdk, "dK at Hq = 8192")
    assert_o_close(dv.cpu().numpy(), rdv, "dV at Hq = 8192")


@pytest.mark.parametrize("case", ["tiny", "packed", "window"])
def test_backward_ring_resumes_from_a_host_copy_of_dq(case):
    """The backward ring stopped after step k, its dQ accumulator copied to host
    memory and the device copy freed, then resumed from a fresh device copy:
    dQ and every step's dK/dV are bit-identical to the uninterrupted ring (the
    library's default dK/dV split on the packed and window rings included)."""
    from context_long_attention_amd.ring import RankRing
    cu = None
    if case == "tiny":
        w = inputs.WORKLOADS["tiny"]
    elif case == "packed":
        w = inputs.Workload("resume_bwd_packed", 1024, 4, 8, 2, 128, backward=True, packed=True)
        cu = np.array([0, 5, 130, 131, 600, 700, 1024], dtype=np.int32)
    else:
        w = inputs.WORKLOADS["tiny_window_wide"]
    for rank in sorted({0, w.cp - 1}):
        note(f"bwd resume {w.name} rank={rank}")
        inp = RankInputs(w, rank, want_do=True)
        ring = RankRing(w, rank, cu)
        o, lse, _ = ring.forward(inp.q, inp.kv_of_source)
        dq_full, steps_full = ring.backward(inp.q, inp.do, o, lse, inp.kv_of_source)
        torch.cuda.synchronize()
        want_dq = dq_full.cpu().numpy()
        want_steps = [(s, dk.cpu().numpy(), dv.cpu().numpy()) for s, dk, dv in steps_full]
        for k in range(1, w.cp):
            dq_k, steps_a = ring.backward(inp.q, inp.do, o, lse, inp.kv_of_source, stop=k)
            host = dq_k.cpu().numpy().copy()
            got_a = [(s, dk.cpu().numpy(), dv.cpu().numpy()) for s, dk, dv in steps_a]
            del dq_k, steps_a
            torch.cuda.synchronize()
            state = torch.from_numpy(host).cuda()
            dq, steps_b = ring.backward(inp.q, inp.do, o, lse, inp.kv_of_source, start=k, state=state)
            torch.cuda.synchronize()
            assert dq.data_ptr() == state.data_ptr()
            assert np.array_equal(dq.cpu().numpy(), want_dq), f"dQ after resuming at step {k}"
            got = got_a + [(s, dk.cpu().numpy(), dv.cpu().numpy()) for s, dk, dv in steps_b]
            assert len(got) == len(want_steps)
            for t, ((s, dk, dv), (ws, wdk, wdv)) in enumerate(zip(got, want_steps)):
                assert s == ws and np.array_equal(dk, wdk) and np.array_equal(dv, wdv), \
                    f"dK/dV of step {t} after resuming at step {k}"
    with pytest.raises(ValueError):
        ring.backward(inp.q, inp.do, o, lse, inp.kv_of_source, start=1)
    with pytest.raises(ValueError):
        ring.backward(inp.q, inp.do, o, lse, inp.kv_of_source, start=1, state=torch.zeros(3, device="cuda"))
