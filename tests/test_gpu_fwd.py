"""GPU parity of the forward ring step, the merge and the kernel's own block map
against the float64 oracle, through the C ABI (libcpattn.so)."""
import numpy as np
import pytest

import oracle
from context_long_attention_amd import inputs
from tests.gpu_common import RankInputs, assert_lse_close, assert_o_close, device_bf16, note

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _needs_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from context_long_attention_amd import cpattn
    cpattn.lib()


def _ring(w, rank, cu=None):
    from context_long_attention_amd.ring import RankRing
    return RankRing(w, rank, cu)


def _oracle_blocks(inp, ring):
    return [inp.kv64[s] for s in ring.schedule()]


def _check_rank(w, rank, cu=None, check_steps=True, check_map=True):
    from context_long_attention_amd import cpattn
    note(f"fwd {w.name} S={w.seq_len} R={w.cp} Hq={w.hq} Hkv={w.hkv} D={w.dim} rank={rank} docs={cu is not None}")
    inp = RankInputs(w, rank)
    ring = _ring(w, rank, cu)
    o, lse, steps = ring.forward(inp.q, inp.kv_of_source, stage=True, keep_steps=True)
    torch.cuda.synchronize()
    ro, rlse, rsteps = oracle.rank_forward(inp.q64, inp.qpos, _oracle_blocks(inp, ring), cu, w.scale)
    live = np.isfinite(rlse).T  # [rows, Hq]
    assert_o_close(o.cpu().numpy(), ro, f"merged O rank {rank}", live)
    assert_lse_close(lse.cpu().numpy(), rlse, f"merged LSE rank {rank}")
    # the fused ring (merge inside the step kernel) reaches the same result
    of, lf, _ = ring.forward(inp.q, inp.kv_of_source, stage=True, fused=True)
    torch.cuda.synchronize()
    assert_o_close(of.cpu().numpy(), ro, f"fused merged O rank {rank}", live)
    assert_lse_close(lf.cpu().numpy(), rlse, f"fused merged LSE rank {rank}")
    if check_steps:
        for t, ((ot, lt), (rot, rlt)) in enumerate(zip(steps, rsteps)):
            assert_o_close(ot.cpu().numpy(), rot, f"O_t rank {rank} step {t}", np.isfinite(rlt).T)
            assert_lse_close(lt.cpu().numpy(), rlt, f"LSE_t rank {rank} step {t}")
    if check_map:
        bm, bn = cpattn.cp_tile_shape(w.hq, w.hkv, w.dim)
        for t in range(w.cp):
            p = ring.problem(t)
            nq, nk = cpattn.cp_block_map_size(p)
            tm = torch.full((nq, nk), 255, dtype=torch.uint8, device="cuda")
            k, v = inp.kv_of_source(ring.schedule()[t])
            o_t = torch.empty((w.local, w.hq, w.dim), dtype=torch.float32, device="cuda")
            l_t = torch.empty((w.hq, w.local), dtype=torch.float32, device="cuda")
            cpattn.cp_attn_fwd_step(p, inp.q, k, v, o_t, l_t, tile_map=tm)
            got = tm.cpu().numpy()
            qseg = [(int(p.q_seg[i].pos0), int(p.q_seg[i].len)) for i in range(p.n_q_seg)]
            kseg = [(int(p.kv_seg[j].pos0), int(p.kv_seg[j].len)) for j in range(p.n_kv_seg)]
            ref = oracle.tile_map(qseg, kseg, bm, bn, cu)
            assert np.array_equal(got, ref), f"kernel block map differs at step {t}"
            assert np.array_equal(cpattn.cp_block_map(ring.problem(t, host_docs=True)), ref)
    return o, lse


def test_tiny_every_rank_and_step():
    """The tiny workload on all 4 ranks x 4 steps; scattered outputs equal full attention."""
    w = inputs.WORKLOADS["tiny"]
    o_glob = np.zeros((w.seq_len, w.hq, w.dim))
    l_glob = np.zeros((w.hq, w.seq_len))
    q_all = None
    for r in range(w.cp):
        o, lse = _check_rank(w, r)
        pos = oracle.zigzag_positions(w.seq_len, w.cp, r)
        o_glob[pos] = o.cpu().numpy()
        l_glob[:, pos] = lse.cpu().numpy()
    c = w.chunk
    q = inputs.round_bf16(inputs.chunks_normal(inputs.SEED_Q, range(2 * w.cp), c, w.hq, w.dim)).astype(np.float64)
    k = inputs.round_bf16(inputs.chunks_normal(inputs.SEED_K, range(2 * w.cp), c, w.hkv, w.dim)).astype(np.float64)
    v = inputs.round_bf16(inputs.chunks_normal(inputs.SEED_V, range(2 * w.cp), c, w.hkv, w.dim)).astype(np.float64)
    pos = np.arange(w.seq_len)
    ro, rl = oracle.attention_partial(q, k, v, oracle.visibility(pos, pos), w.scale)
    assert_o_close(o_glob, ro, "tiny scattered O")
    assert_lse_close(l_glob, rl, "tiny scattered LSE")
    del q_all


RAGGED = [
    # name, S, R, Hq, Hkv, D   (chunk lengths that are not multiples of the tiles)
    ("g4_d128", 2 * 2 * 100, 2, 8, 2, 128),
    ("g1_d64", 2 * 3 * 77, 3, 4, 4, 64),
    ("g2_d128", 2 * 2 * 90, 2, 6, 3, 128),
    ("g16_d64", 2 * 4 * 33, 4, 16, 1, 64),
    ("g8_d128", 2 * 2 * 130, 2, 8, 1, 128),
    ("g3_d64", 2 * 2 * 70, 2, 6, 2, 64),
    ("r16_c256", 2 * 16 * 256, 16, 8, 2, 128),
    # Hkv a multiple of 8 with several head blocks per KV head: the work order renumbers
    # head blocks so a KV head's blocks share an XCD (2 and 4 blocks per KV head)
    ("hkv8_g8_d128", 2 * 2 * 160, 2, 64, 8, 128),
    ("hkv8_g16_d128", 2 * 2 * 96, 2, 128, 8, 128),
    ("hkv16_g4_d64", 2 * 2 * 72, 2, 64, 16, 64),
]


@pytest.mark.parametrize("name,S,R,hq,hkv,d", RAGGED, ids=[r[0] for r in RAGGED])
def test_ragged_shapes(name, S, R, hq, hkv, d):
    w = inputs.Workload(name, S, R, hq, hkv, d, backward=False)
    for r in sorted({0, R - 1}):
        _check_rank(w, r)


def test_packed_documents_small():
    cu = np.array([0, 1, 2, 130, 131, 300, 301, 520, 767, 768], dtype=np.int32)
    w = inputs.Workload("packed_small", 768, 4, 8, 2, 128, backward=False, packed=True)
    for r in range(w.cp):
        _check_rank(w, r, cu)


def test_single_token_chunks():
    """c = 1: every chunk is one token (the pages' 4-token, 2-rank example shape)."""
    w = inputs.Workload("c1", 4, 2, 4, 2, 64, backward=False)
    for r in range(2):
        _check_rank(w, r)


def test_empty_and_skip_segments():
    """An empty KV segment, an empty query segment and an all-SKIP step."""
    from context_long_attention_amd import cpattn
    hq, hkv, d = 4, 2, 128
    n = 96
    q64, q = device_bf16(inputs.chunk_normal(1, 0, n, hq, d))
    k64, k = device_bf16(inputs.chunk_normal(2, 0, n, hkv, d))
    v64, v = device_bf16(inputs.chunk_normal(3, 0, n, hkv, d))
    o = torch.full((n, hq, d), 7.0, device="cuda")
    lse = torch.full((hq, n), 7.0, device="cuda")
    F, D_, S_ = cpattn.CP_MASK_FULL, cpattn.CP_MASK_DIAG_CAUSAL, cpattn.CP_MASK_SKIP
    # query rows [0, 96) at positions 1000..; KV segment 0 empty, segment 1 = rows [0, 96) at 1000..
    p = cpattn.make_problem(hq, hkv, d, 0.125, n, n, [(0, 1000, n)], [(0, 0, 0), (0, 1000, n)], [[F, D_], [S_, S_]])
    cpattn.cp_attn_fwd_step(p, q, k, v, o, lse)
    pos = np.arange(1000, 1000 + n)
    ro, rl = oracle.attention_partial(q64, k64, v64, oracle.visibility(pos, pos), 0.125)
    assert_o_close(o.cpu().numpy(), ro, "empty KV segment O")
    assert_lse_close(lse.cpu().numpy(), rl, "empty KV segment LSE")
    # all SKIP: every row gets (0, -inf)
    p = cpattn.make_problem(hq, hkv, d, 0.125, n, n, [(0, 0, 48), (48, 48, 48)], [(0, 500, n)], [[S_, S_], [S_, S_]])
    cpattn.cp_attn_fwd_step(p, q, k, v, o, lse)
    assert torch.all(o == 0).item() and torch.all(torch.isneginf(lse)).item()
    # an empty query segment writes nothing
    o.fill_(7.0)
    p = cpattn.make_problem(hq, hkv, d, 0.125, n, n, [(0, 0, 0)], [(0, 0, n)], [[F, F], [F, F]])
    cpattn.cp_attn_fwd_step(p, q, k, v, o, lse)
    torch.cuda.synchronize()
    assert torch.all(o == 7.0).item()


@pytest.mark.parametrize("d", [128, 64])
def test_fused_step_merge_from_arbitrary_state(d):
    """cp_attn_fwd_step_merge on a random valid accumulator (some rows empty, -inf)
    equals the oracle's merge of that state with the step's partial; rows that see
    no key in the step (documents) keep the accumulator untouched."""
    from context_long_attention_amd import cpattn
    hq, hkv, n, m = 8, 2, 200, 150
    note(f"fused merge d={d}")
    q64, q = device_bf16(inputs.chunk_normal(11, 0, n, hq, d))
    k64, k = device_bf16(inputs.chunk_normal(12, 0, m, hkv, d))
    v64, v = device_bf16(inputs.chunk_normal(13, 0, m, hkv, d))
    cu = np.array([0, 950, 1100, 1150, 5000], dtype=np.int32)
    cu_dev = torch.from_numpy(cu).cuda()
    qpos, kpos = np.arange(1000, 1000 + n), np.arange(900, 900 + m)
    DOC = cpattn.CP_MASK_DOC
    p = cpattn.make_problem(hq, hkv, d, d ** -0.5, n, m, [(0, 1000, n)], [(0, 900, m)], [[DOC, DOC], [DOC, DOC]],
                            cu_dev.data_ptr(), len(cu) - 1)
    rng = np.random.default_rng(5)
    o0 = rng.standard_normal((n, hq, d)).astype(np.float32)
    l0 = (rng.standard_normal((hq, n)) * 4).astype(np.float32)
    l0[:, ::7] = -np.inf
    l0[2, 100:130] = 30.0  # a dominant accumulator
    o0.transpose(1, 0, 2)[np.isneginf(l0)] = 0  # (0, -inf) is the empty state
    o_acc = torch.from_numpy(o0.copy()).cuda()
    l_acc = torch.from_numpy(l0.copy()).cuda()
    cpattn.cp_attn_fwd_step_merge(p, q, k, v, o_acc, l_acc)
    # the same through a separate partial and cp_merge_partials
    o_sep = torch.from_numpy(o0.copy()).cuda()
    l_sep = torch.from_numpy(l0.copy()).cuda()
    o_t = torch.empty((n, hq, d), dtype=torch.float32, device="cuda")
    l_t = torch.empty((hq, n), dtype=torch.float32, device="cuda")
    cpattn.cp_attn_fwd_step(p, q, k, v, o_t, l_t)
    cpattn.cp_merge_partials(o_sep, l_sep, o_t, l_t, n, hq, d)
    torch.cuda.synchronize()
    ro_t, rl_t = oracle.attention_partial(q64, k64, v64, oracle.visibility(qpos, kpos, cu), d ** -0.5)
    ro, rl = oracle.merge(o0.astype(np.float64), l0.astype(np.float64), ro_t, rl_t)
    assert np.isneginf(rl_t).any() and np.isfinite(rl_t).any()
    assert_o_close(o_acc.cpu().numpy(), ro, "fused merge O")
    assert_lse_close(l_acc.cpu().numpy(), rl, "fused merge LSE")
    np.testing.assert_allclose(o_acc.cpu().numpy(), o_sep.cpu().numpy(), atol=2e-5, rtol=1e-5)
    got_l, sep_l = l_acc.cpu().numpy(), l_sep.cpu().numpy()
    assert np.array_equal(np.isneginf(got_l), np.isneginf(sep_l))
    np.testing.assert_allclose(got_l[np.isfinite(got_l)], sep_l[np.isfinite(sep_l)], atol=2e-5, rtol=1e-6)
    # rows with nothing visible in this step are bit-identical to the initial state
    dead = np.isneginf(rl_t)
    assert np.array_equal(got_l[dead], l0[dead])
    assert np.array_equal(o_acc.cpu().numpy().transpose(1, 0, 2)[dead], o0.transpose(1, 0, 2)[dead])


RESUME = [
    ("tiny", None),
    ("ragged", None),
    ("packed", np.array([0, 1, 2, 130, 131, 300, 301, 520, 767, 768], dtype=np.int32)),
]


@pytest.mark.parametrize("case,cu", RESUME, ids=[r[0] for r in RESUME])
def test_ring_resumes_from_a_host_copy_of_its_state(case, cu):
    """A ring stopped after step k, its (O, LSE) state copied to host memory and
    the device tensors freed, then resumed from a fresh device copy of that
    state, ends bit-identical to the uninterrupted ring and matches the oracle,
    for every k, on the fused and the separate-merge paths."""
    w = {"tiny": inputs.WORKLOADS["tiny"],
         "ragged": inputs.Workload("resume_ragged", 2 * 4 * 300, 4, 8, 2, 128, backward=False),
         "packed": inputs.Workload("resume_packed", 768, 4, 8, 2, 128, backward=False, packed=True)}[case]
    for rank in sorted({0, w.cp - 1}):
        note(f"resume {w.name} rank={rank}")
        inp = RankInputs(w, rank)
        ring = _ring(w, rank, cu)
        ro, rlse, _ = oracle.rank_forward(inp.q64, inp.qpos, _oracle_blocks(inp, ring), cu, w.scale)
        live = np.isfinite(rlse).T
        for fused in (True, False):
            o_full, l_full, _ = ring.forward(inp.q, inp.kv_of_source, fused=fused)
            torch.cuda.synchronize()
            want_o, want_l = o_full.cpu().numpy(), l_full.cpu().numpy()
            for k in range(1, w.cp):
                o_k, l_k, _ = ring.forward(inp.q, inp.kv_of_source, fused=fused, stop=k)
                host_o, host_l = o_k.cpu().numpy().copy(), l_k.cpu().numpy().copy()
                del o_k, l_k
                torch.cuda.synchronize()
                state = (torch.from_numpy(host_o).cuda(), torch.from_numpy(host_l).cuda())
                o, lse, _ = ring.forward(inp.q, inp.kv_of_source, fused=fused, start=k, state=state)
                torch.cuda.synchronize()
                assert o.data_ptr() == state[0].data_ptr() and lse.data_ptr() == state[1].data_ptr()
                got_o, got_l = o.cpu().numpy(), lse.cpu().numpy()
                assert np.array_equal(got_o, want_o), f"O after resuming at step {k} (fused={fused})"
                assert np.array_equal(got_l, want_l), f"LSE after resuming at step {k} (fused={fused})"
                assert_o_close(got_o, ro, f"resumed O rank {rank} k={k}", live)
                assert_lse_close(got_l, rlse, f"resumed LSE rank {rank} k={k}")


def test_ring_resume_rejects_a_missing_or_misshapen_state():
    w = inputs.WORKLOADS["tiny"]
    inp = RankInputs(w, 0)
    ring = _ring(w, 0)
    rows = 2 * w.chunk
    good = (torch.zeros((rows, w.hq, w.dim), dtype=torch.float32, device="cuda"),
            torch.full((w.hq, rows), float("-inf"), dtype=torch.float32, device="cuda"))
    with pytest.raises(ValueError):
        ring.forward(inp.q, inp.kv_of_source, start=1)
    with pytest.raises(ValueError):
        ring.forward(inp.q, inp.kv_of_source, state=good)
    with pytest.raises(ValueError):
        ring.forward(inp.q, inp.kv_of_source, start=1, state=(good[0][1:], good[1]))
    with pytest.raises(ValueError):
        ring.forward(inp.q, inp.kv_of_source, start=1, state=(good[0], good[1].double()))
    with pytest.raises(ValueError):
        ring.forward(inp.q, inp.kv_of_source, start=2, stop=1, state=good)


def test_clock_probe_records_every_workgroup():
    """cp_debug_clock_probe: each workgroup of a launch records start/end cycle and
    100 MHz tick counters; the implied shader clock is a plausible one."""
    from context_long_attention_amd import cpattn
    w = inputs.Workload("probe", 4096, 2, 8, 2, 128, backward=False)
    inp = RankInputs(w, 0)
    ring = _ring(w, 0)
    p = ring.problem(0)
    o = torch.empty((w.local, w.hq, w.dim), dtype=torch.float32, device="cuda")
    lse = torch.empty((w.hq, w.local), dtype=torch.float32, device="cuda")
    buf = torch.zeros(4 * 4096, dtype=torch.int64, device="cuda")
    cpattn.cp_debug_clock_probe(buf)
    try:
        k, v = inp.kv_of_source(ring.schedule()[0])
        cpattn.cp_attn_fwd_step(p, inp.q, k, v, o, lse)
        torch.cuda.synchronize()
    finally:
        cpattn.cp_debug_clock_probe(None)
    bm, _ = cpattn.cp_tile_shape(w.hq, w.hkv, w.dim)
    n_wg = (w.local // bm) * (w.hq * bm // 256)
    rec = buf.view(-1, 4).cpu().numpy()
    assert (rec[:n_wg] != 0).all() and (rec[n_wg:] == 0).all()
    assert (rec[:, 2] >= rec[:, 0]).all() and (rec[:, 3] >= rec[:, 1]).all()
    busy = rec[:n_wg, 3] - rec[:n_wg, 1] > 100
    mhz = (rec[:n_wg, 2] - rec[:n_wg, 0])[busy] / (rec[:n_wg, 3] - rec[:n_wg, 1])[busy] * 100
    assert busy.any() and 300 < np.median(mhz) < 3000, np.median(mhz)


def test_merge_kernel_matches_oracle():
    from context_long_attention_amd import cpattn
    rng = np.random.default_rng(3)
    rows, hq, d = 300, 6, 64
    o1, o2 = rng.standard_normal((rows, hq, d)), rng.standard_normal((rows, hq, d))
    l1, l2 = rng.standard_normal((hq, rows)) * 5, rng.standard_normal((hq, rows)) * 5
    l1[0, :10] = -np.inf
    l2[0, 5:15] = -np.inf
    o1[:, 0][np.isneginf(l1[0])] = 0
    o2[:, 0][np.isneginf(l2[0])] = 0
    t = lambda x: torch.tensor(x, dtype=torch.float32, device="cuda")
    oa, la, ob, lb = t(o1), t(l1), t(o2), t(l2)
    cpattn.cp_merge_partials(oa, la, ob, lb, rows, hq, d)
    ro, rl = oracle.merge(np.float32(o1), np.float32(l1), np.float32(o2), np.float32(l2))
    np.testing.assert_allclose(oa.cpu().numpy(), ro, atol=1e-5)
    got_l = la.cpu().numpy()
    assert np.array_equal(np.isneginf(got_l), np.isneginf(rl))
    np.testing.assert_allclose(got_l[np.isfinite(rl)], rl[np.isfinite(rl)], atol=1e-5)


@pytest.mark.parametrize("n,d", [(1, 128), (3, 64), (8, 128), (64, 64)])
def test_merge_n_matches_pairwise_oracle(n, d):
    """The N-way merge equals folding the parts one by one with the oracle's
    pairwise merge, including rows that are -inf in some or all parts; the output
    may be the first part's buffers."""
    from context_long_attention_amd import cpattn
    rng = np.random.default_rng(n)
    rows, hq = 257, 3
    os_ = [rng.standard_normal((rows, hq, d)) for _ in range(n)]
    ls = [rng.standard_normal((hq, rows)) * 6 for _ in range(n)]
    for i in range(n):
        dead = rng.random((hq, rows)) < 0.3
        dead[:, :4] = True  # rows 0..3 are -inf in every part
        ls[i][dead] = -np.inf
        os_[i][np.transpose(dead)] = 0.0
    ro = np.zeros((rows, hq, d))
    rl = np.full((hq, rows), -np.inf)
    for o_i, l_i in zip(os_, ls):
        ro, rl = oracle.merge(ro, rl, np.float32(o_i).astype(np.float64), np.float32(l_i).astype(np.float64))
    t = lambda x: torch.tensor(x, dtype=torch.float32, device="cuda")
    o_parts, l_parts = [t(x) for x in os_], [t(x) for x in ls]
    out_o = torch.full((rows, hq, d), 7.0, device="cuda")
    out_l = torch.full((hq, rows), 7.0, device="cuda")
    cpattn.cp_merge_partials_n(out_o, out_l, o_parts, l_parts, rows, hq, d)
    # in place on part 0
    cpattn.cp_merge_partials_n(o_parts[0], l_parts[0], o_parts, l_parts, rows, hq, d)
    torch.cuda.synchronize()
    for go, gl, what in ((out_o, out_l, "out"), (o_parts[0], l_parts[0], "in place")):
        np.testing.assert_allclose(go.cpu().numpy(), ro, atol=2e-5, err_msg=what)
        g = gl.cpu().numpy()
        assert np.array_equal(np.isneginf(g), np.isneginf(rl)), what
        np.testing.assert_allclose(g[np.isfinite(rl)], rl[np.isfinite(rl)], atol=2e-5, err_msg=what)
    assert torch.all(out_o[:4] == 0).item()


def _sampled_rows(local, c, n_extra, seed):
    rng = np.random.default_rng(seed)
    edge = [0, 1, 2, c - 1, c, c + 1, local - 2, local - 1]
    return np.unique(np.concatenate([edge, rng.integers(0, local, n_extra)]))


@pytest.mark.timeout(600)
@pytest.mark.parametrize("rank", [0, 7])
def test_llama3_8b_forward_whole_tensor(rank):
    """Llama-3-8B shape, one rank's share of S=128K at CP=8 (local 16K as two zigzag
    8K chunks, 8 ring steps of 16K-token KV blocks), run as the bench runs it (fused
    merge, staged receive buffers): O and LSE of every local row and every one of the
    32 query heads against the float64 oracle.  Rank 0 holds the first and last
    chunks (half its rows see nothing after step 0); rank 7 the two middle ones."""
    from tests.gpu_common import GroupReference
    w = inputs.WORKLOADS["llama3_8b_fwd"]
    note(f"fwd {w.name} full size rank={rank} whole tensor")
    inp = RankInputs(w, rank)
    ring = _ring(w, rank)
    with GroupReference(inp, ring.schedule(), range(w.hq)) as ref:
        o, lse, _ = ring.forward(inp.q, inp.kv_of_source, stage=True)
        torch.cuda.synchronize()
        got_o, got_l = o.cpu().numpy(), lse.cpu().numpy()
        del o, lse
        ro, rl = ref.forward()
    assert_o_close(got_o, ro, f"O rank {rank}, all rows and heads")
    assert_lse_close(got_l, rl, f"LSE rank {rank}, all rows and heads")
