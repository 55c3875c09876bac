"""Seeded random problems through the step calls of the C ABI (libcpattn.so),
each compared with the float64 oracle: one or two query and KV segments of
arbitrary length (empty and ragged included) at arbitrary rows and global
positions, a random mask class per segment pair, packed documents, sliding
windows, several GQA shapes, both head dims and every dK/dV split.

The expected visibility of a pair comes from the classes' definitions in the
ABI: FULL sees every key whatever the positions, DIAG_CAUSAL sees k <= q inside
the window, DOC additionally only keys of the query's document, SKIP nothing
("Context Parallelism for Scalable Million-Token Inference", section "Ring
Attention Algorithms"; "Announcing Long-Context Training on TPUs with MaxText
Context Parallelism", section "Built on a fast attention kernel" and the
closing section on window layers)."""
import numpy as np
import pytest

import oracle
from tests.gpu_common import assert_lse_close, assert_o_close, device_bf16, note

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

N_CASES = 160
HEADS = [(4, 1), (8, 2), (6, 2), (16, 4), (32, 8), (12, 4), (64, 8), (8, 8), (2, 1)]
LENGTHS = [0, 1, 2, 31, 63, 64, 65, 127, 128, 129, 200, 257, 300]
SENTINEL = 7.25


@pytest.fixture(scope="module", autouse=True)
def _needs_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from context_long_attention_amd import cpattn
    cpattn.lib()


def _segments(rng):
    """One or two runs of rows (row0, pos0, len) with unused rows around them."""
    segs, row = [], int(rng.integers(0, 12))
    for _ in range(int(rng.integers(1, 3))):
        n = int(rng.choice(LENGTHS)) if rng.random() < 0.6 else int(rng.integers(0, 320))
        segs.append((row, int(rng.integers(0, 1500)), n))
        row += n + int(rng.integers(0, 12))
    return segs, row + int(rng.integers(1, 8))


def _case(seed):
    from context_long_attention_amd import cpattn
    rng = np.random.default_rng(1000 + seed)
    hq, hkv = HEADS[int(rng.integers(len(HEADS)))]
    d = int(rng.choice([64, 128]))
    qsegs, q_rows = _segments(rng)
    ksegs, kv_rows = _segments(rng)
    classes = [cpattn.CP_MASK_FULL, cpattn.CP_MASK_DIAG_CAUSAL, cpattn.CP_MASK_DOC, cpattn.CP_MASK_SKIP]
    masks = [[int(rng.choice(classes, p=[0.2, 0.35, 0.3, 0.15])) for _ in range(2)] for _ in range(2)]
    window = int(rng.choice([0, 0, 0, 1, 16, 100, 513]))
    if window:
        # a pair the window cuts must not be marked FULL
        masks = [[cpattn.CP_MASK_DIAG_CAUSAL if m == cpattn.CP_MASK_FULL else m for m in row] for row in masks]
    used = [m for i in range(len(qsegs)) for j, m in enumerate(masks[i]) if j < len(ksegs)]
    cu = None
    if cpattn.CP_MASK_DOC in used:
        top = max(p0 + n for _, p0, n in qsegs + ksegs) + 1
        cuts = np.unique(rng.integers(1, top, int(rng.integers(0, 10))))
        cu = np.concatenate([[0], cuts, [top + int(rng.integers(0, 50))]]).astype(np.int32)
    kv_split = int(rng.choice([0, 0, 1, 2, 3, 5, 8]))
    return dict(hq=hq, hkv=hkv, d=d, qsegs=qsegs, ksegs=ksegs, q_rows=q_rows, kv_rows=kv_rows, masks=masks,
                window=window, cu=cu, kv_split=kv_split, seed=1000 + seed)


def _visibility(c):
    from context_long_attention_amd import cpattn
    vis = np.zeros((c["q_rows"], c["kv_rows"]), dtype=bool)
    w = c["window"] or None
    for i, (qr, qp, qn) in enumerate(c["qsegs"]):
        for j, (kr, kp, kn) in enumerate(c["ksegs"]):
            m = c["masks"][i][j]
            qpos, kpos = qp + np.arange(qn), kp + np.arange(kn)
            if m == cpattn.CP_MASK_FULL:
                block = np.ones((qn, kn), dtype=bool)
            elif m == cpattn.CP_MASK_DIAG_CAUSAL:
                block = oracle.visibility(qpos, kpos, None, w)
            elif m == cpattn.CP_MASK_DOC:
                block = oracle.visibility(qpos, kpos, c["cu"], w)
            else:
                block = np.zeros((qn, kn), dtype=bool)
            vis[qr:qr + qn, kr:kr + kn] = block
    return vis


def _grad_close(got, ref, what):
    """Gradients to 2e-2 of max(1, the largest reference magnitude).  On the
    pages' workloads gradients stay below 1, so this is the plain 2e-2 bound
    there; a few random problems concentrate a gradient (a 2-key segment seen
    by hundreds of query rows gives |dK| of about 8), where the bf16 rounding
    of dS before its product alone exceeds 2e-2 absolute (a reading of the
    tolerance for inputs outside the pages' recipe, as for the adversarial
    numerics cases)."""
    s = max(1.0, float(np.abs(ref).max()) if ref.size else 1.0)
    return assert_o_close(got / s, ref / s, f"{what} (scaled by {s:.3g})")


def _rows(segs):
    return np.concatenate([np.arange(r, r + n) for r, _, n in segs]).astype(np.int64)


@pytest.mark.parametrize("case", range(N_CASES))
def test_random_problem_matches_oracle(case):
    from context_long_attention_amd import cpattn
    c = _case(case)
    hq, hkv, d = c["hq"], c["hkv"], c["d"]
    note(f"random case {case}: seed={c['seed']} Hq={hq} Hkv={hkv} D={d} q={c['qsegs']} kv={c['ksegs']} "
         f"masks={c['masks']} window={c['window']} docs={None if c['cu'] is None else len(c['cu']) - 1} "
         f"split={c['kv_split']}")
    rng = np.random.default_rng(c["seed"] + 7)
    nq, nk = c["q_rows"], c["kv_rows"]
    q64, q = device_bf16(rng.standard_normal((nq, hq, d)).astype(np.float32))
    k64, k = device_bf16(rng.standard_normal((nk, hkv, d)).astype(np.float32))
    v64, v = device_bf16(rng.standard_normal((nk, hkv, d)).astype(np.float32))
    do64, do = device_bf16(rng.standard_normal((nq, hq, d)).astype(np.float32))
    cu_dev = None if c["cu"] is None else torch.from_numpy(c["cu"]).cuda()
    p = cpattn.make_problem(hq, hkv, d, d ** -0.5, nq, nk, c["qsegs"], c["ksegs"], c["masks"],
                            None if cu_dev is None else cu_dev.data_ptr(),
                            0 if c["cu"] is None else len(c["cu"]) - 1, c["window"], c["kv_split"])
    vis = _visibility(c)
    ro, rl = oracle.attention_partial(q64, k64, v64, vis, d ** -0.5)
    qrows, krows = _rows(c["qsegs"]), _rows(c["ksegs"])
    out_q = np.setdiff1d(np.arange(nq), qrows)
    live = vis.any(axis=1)

    # forward: segment rows match the oracle, other rows are not written
    o = torch.full((nq, hq, d), SENTINEL, dtype=torch.float32, device="cuda")
    lse = torch.full((hq, nq), SENTINEL, dtype=torch.float32, device="cuda")
    cpattn.cp_attn_fwd_step(p, q, k, v, o, lse)
    torch.cuda.synchronize()
    go, gl = o.cpu().numpy(), lse.cpu().numpy()
    assert_o_close(go[qrows], ro[qrows], f"case {case}: O", live[qrows])
    assert np.all(go[qrows][~live[qrows]] == 0), f"case {case}: rows with no visible key must hold O = 0"
    assert_lse_close(gl[:, qrows], rl[:, qrows], f"case {case}: LSE")
    assert np.all(go[out_q] == SENTINEL) and np.all(gl[:, out_q] == SENTINEL), f"case {case}: rows outside written"
    # the tile classes the kernel used equal the host's block map of the same problem
    ph = cpattn.make_problem(hq, hkv, d, d ** -0.5, nq, nk, c["qsegs"], c["ksegs"], c["masks"],
                             None if c["cu"] is None else c["cu"].ctypes.data,
                             0 if c["cu"] is None else len(c["cu"]) - 1, c["window"], c["kv_split"])
    n_qt, n_kt = cpattn.cp_block_map_size(ph)
    if n_qt * n_kt:
        tm = torch.full((n_qt, n_kt), 255, dtype=torch.uint8, device="cuda")
        o2 = torch.empty_like(o)
        l2 = torch.empty_like(lse)
        cpattn.cp_attn_fwd_step(p, q, k, v, o2, l2, tile_map=tm)
        torch.cuda.synchronize()
        assert np.array_equal(tm.cpu().numpy(), cpattn.cp_block_map(ph)), f"case {case}: kernel block map"
        assert np.array_equal(o2.cpu().numpy()[qrows], go[qrows]), f"case {case}: O with the block map asked for"

    # fused merge into a random valid state: rows that see nothing keep it bit for bit
    o0 = rng.standard_normal((nq, hq, d)).astype(np.float32)
    l0 = (rng.standard_normal((hq, nq)) * 3).astype(np.float32)
    l0[:, rng.random(nq) < 0.2] = -np.inf
    o0.transpose(1, 0, 2)[np.isneginf(l0)] = 0
    o_acc, l_acc = torch.from_numpy(o0.copy()).cuda(), torch.from_numpy(l0.copy()).cuda()
    cpattn.cp_attn_fwd_step_merge(p, q, k, v, o_acc, l_acc)
    torch.cuda.synchronize()
    mo, ml = oracle.merge(o0.astype(np.float64), l0.astype(np.float64), ro, rl)
    ga, gla = o_acc.cpu().numpy(), l_acc.cpu().numpy()
    merged_live = np.isfinite(ml).T
    assert_o_close(ga[qrows], mo[qrows], f"case {case}: merged O", merged_live[qrows])
    assert_lse_close(gla[:, qrows], ml[:, qrows], f"case {case}: merged LSE")
    still = np.setdiff1d(np.arange(nq), qrows[live[qrows]])
    assert np.array_equal(ga[still], o0[still]) and np.array_equal(gla[:, still], l0[:, still]), \
        f"case {case}: rows with no visible key changed by the merge"

    # backward from this step's own (LSE, delta) as the final ones
    delta = np.ascontiguousarray(oracle.delta_rows(do64, ro))
    rdq, rdk, rdv = oracle.attention_backward_partial(q64, k64, v64, do64, rl, delta, vis, d ** -0.5)
    dq0 = rng.standard_normal((nq, hq, d)).astype(np.float32)
    dq = torch.from_numpy(dq0.copy()).cuda()
    dk = torch.full((nk, hkv, d), SENTINEL, dtype=torch.float32, device="cuda")
    dv = torch.full((nk, hkv, d), SENTINEL, dtype=torch.float32, device="cuda")
    ws = None
    if c["kv_split"] > 1:
        ws = torch.empty(max(16, cpattn.cp_bwd_workspace_size(p, c["kv_split"])), dtype=torch.uint8, device="cuda")
        ws.fill_(0xFF)  # the workspace needs no initial value
    lse_dev = torch.from_numpy(rl.astype(np.float32)).cuda()
    delta_dev = torch.from_numpy(delta.astype(np.float32)).cuda()
    cpattn.cp_attn_bwd_step(p, q, k, v, do, lse_dev, delta_dev, dq, dk, dv, workspace=ws)
    torch.cuda.synchronize()
    gdq, gdk, gdv = dq.cpu().numpy(), dk.cpu().numpy(), dv.cpu().numpy()
    _grad_close(gdq[qrows] - dq0[qrows], rdq[qrows], f"case {case}: dQ")
    assert np.array_equal(gdq[out_q], dq0[out_q]), f"case {case}: dQ rows outside the query segments changed"
    _grad_close(gdk[krows], rdk[krows], f"case {case}: dK")
    _grad_close(gdv[krows], rdv[krows], f"case {case}: dV")
    out_k = np.setdiff1d(np.arange(nk), krows)
    assert np.all(gdk[out_k] == SENTINEL) and np.all(gdv[out_k] == SENTINEL), \
        f"case {case}: dK/dV rows outside the KV segments written"


def test_random_cases_cover_every_feature():
    """The seeded draw exercises every class, documents, windows, empty segments and splits."""
    from context_long_attention_amd import cpattn
    cs = [_case(i) for i in range(N_CASES)]
    used = {m for c in cs for i in range(len(c["qsegs"])) for j, m in enumerate(c["masks"][i]) if j < len(c["ksegs"])}
    assert used == {cpattn.CP_MASK_FULL, cpattn.CP_MASK_DIAG_CAUSAL, cpattn.CP_MASK_DOC, cpattn.CP_MASK_SKIP}
    assert any(c["cu"] is not None for c in cs) and any(c["window"] for c in cs)
    assert any(n == 0 for c in cs for _, _, n in c["qsegs"] + c["ksegs"])
    assert {c["kv_split"] for c in cs} >= {0, 1, 2, 8} and {c["d"] for c in cs} == {64, 128}


N_RINGS = 120


def _ring_case(seed):
    """A random ring: S = 2 R c tokens over R ranks, one rank's share, with or
    without packed documents and a sliding window."""
    from context_long_attention_amd import inputs
    rng = np.random.default_rng(5000 + seed)
    R = int(rng.integers(1, 9))
    c = int(rng.choice([1, 2, 3, 17, 32, 63, 64, 65, 96, 129, 150]))
    S = 2 * R * c
    hq, hkv = HEADS[int(rng.integers(len(HEADS)))]
    d = int(rng.choice([64, 128]))
    cu = None
    if rng.random() < 0.35:
        cuts = np.unique(rng.integers(1, S, int(rng.integers(0, 12)))) if S > 1 else np.zeros(0, dtype=np.int64)
        cu = np.concatenate([[0], cuts, [S]]).astype(np.int32)
    window = int(rng.choice([0, 0, 1, max(1, c // 2 + 1), c, 2 * c + 1, S]))
    w = inputs.Workload(f"ring{seed}", S, R, hq, hkv, d, backward=True, packed=cu is not None, window=window)
    return w, int(rng.integers(0, R)), cu


@pytest.mark.parametrize("case", range(N_RINGS))
def test_random_ring_matches_oracle(case):
    """One rank's whole forward and backward ring (RankRing: live-step skipping,
    the receive double buffer, the fused merge, the library's dK/dV split and its
    workspace) against the oracle's replay of the same ring."""
    from context_long_attention_amd.ring import RankRing
    from tests.gpu_common import RankInputs
    w, rank, cu = _ring_case(case)
    note(f"random ring {case}: S={w.seq_len} R={w.cp} c={w.chunk} Hq={w.hq} Hkv={w.hkv} D={w.dim} rank={rank} "
         f"window={w.window} docs={None if cu is None else len(cu) - 1}")
    inp = RankInputs(w, rank, want_do=True)
    ring = RankRing(w, rank, cu)
    o, lse, _ = ring.forward(inp.q, inp.kv_of_source)
    dq, per_step = ring.backward(inp.q, inp.do, o, lse, inp.kv_of_source)
    torch.cuda.synchronize()
    blocks = [inp.kv64[s] for s in ring.schedule()]
    win = w.window or None
    ro, rl, _ = oracle.rank_forward(inp.q64, inp.qpos, blocks, cu, w.scale, window=win)
    rdq, rsteps, _ = oracle.rank_backward(inp.q64, inp.qpos, inp.do64, ro, rl, blocks, cu, w.scale, window=win)
    assert_o_close(o.cpu().numpy(), ro, f"ring {case}: O", np.isfinite(rl).T)
    assert_lse_close(lse.cpu().numpy(), rl, f"ring {case}: LSE")
    _grad_close(dq.cpu().numpy(), rdq, f"ring {case}: dQ")
    for t, ((src, dk, dv), (rdk, rdv)) in enumerate(zip(per_step, rsteps)):
        assert src == ring.schedule()[t]
        _grad_close(dk.cpu().numpy(), rdk, f"ring {case}: dK step {t}")
        _grad_close(dv.cpu().numpy(), rdv, f"ring {case}: dV step {t}")
