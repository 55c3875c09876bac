"""CPU tests of libcpattn.so: it loads, exports every symbol include/*.h
declares, its host integer logic (partition, ring order, chunk classes, block
map, pair counts) is bit-exact against the oracle's brute force, and bad
arguments are rejected before any launch.  No kernel runs here."""
import ctypes
import os
import re

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
from context_long_attention_amd import cpattn
from context_long_attention_amd.ring import RankRing, RingScheduleError, check_schedule
from context_long_attention_amd import inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "cpattn.h")
HEADERS = sorted(os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include"))
                 if f.endswith(".h"))


@pytest.fixture(scope="module")
def lib():
    return cpattn.lib()


def _declared():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(cp_[a-z_0-9]+)\s*\(", text))
    return sorted(names)


def test_exports_every_declared_symbol(lib):
    declared = _declared()
    assert len(declared) >= 14 and len(HEADERS) >= 2
    assert sorted(cpattn.EXPORTS) == declared
    for name in declared:
        assert hasattr(lib, name), name
    version = int(re.search(r"#define CPATTN_ABI_VERSION (\d+)", open(HEADER).read()).group(1))
    assert cpattn.cp_abi_version() == version
    assert cpattn.cp_status_string(cpattn.CP_ERR_UNSUPPORTED) == "unsupported"


@pytest.mark.parametrize("S,R", [(4, 2), (16, 2), (24, 3), (64, 4), (80, 5), (512, 4), (2048, 16)])
def test_partition_bit_exact(S, R):
    for r in range(R):
        got = cpattn.cp_partition_zigzag(S, R, r)
        assert got.dtype == np.int64
        assert np.array_equal(got, oracle.zigzag_positions(S, R, r))
        for t in range(R):
            assert cpattn.cp_ring_source(R, r, t) == oracle.ring_source(r, t, R)


def test_partition_errors():
    with pytest.raises(cpattn.CpError) as e:
        cpattn.cp_partition_zigzag(10, 3, 0)
    assert e.value.status == cpattn.CP_ERR_INVALID_ARG
    with pytest.raises(cpattn.CpError):
        cpattn.cp_partition_zigzag(16, 2, 2)
    with pytest.raises(cpattn.CpError):
        cpattn.cp_ring_source(4, 0, 4)


@pytest.mark.parametrize("S,R", [(16, 2), (24, 3), (64, 4), (80, 5), (512, 4)])
def test_step_masks_match_brute_force(S, R):
    c = S // (2 * R)
    cu = np.array([0, 3, 3, S // 2 + 1, S], dtype=np.int32)
    for r in range(R):
        qpos = oracle.zigzag_positions(S, R, r)
        for t in range(R):
            kpos = oracle.zigzag_positions(S, R, oracle.ring_source(r, t, R))
            for packed in (False, True):
                got = cpattn.cp_step_masks(R, r, t, packed)
                for i in range(2):
                    for j in range(2):
                        ref = oracle.chunk_pair_class(qpos[i * c:(i + 1) * c], kpos[j * c:(j + 1) * c],
                                                      cu if packed else None)
                        if packed and ref == oracle.CLS_SKIP:
                            # DOC may still be chosen when the chunks are causal-visible but
                            # documents cut them apart; SKIP must be exact in the causal case
                            assert got[i][j] in (oracle.CLS_SKIP, oracle.CLS_DOC)
                        else:
                            assert got[i][j] == ref, (r, t, i, j, packed)


MAP_CASES = [
    # S, R, Hq, Hkv, D, packed
    (400, 2, 8, 2, 128, False),
    (462, 3, 4, 4, 64, False),
    (360, 2, 6, 3, 128, True),
    (264, 4, 16, 1, 64, True),
    (1024, 4, 8, 2, 128, True),
]


@pytest.mark.parametrize("S,R,hq,hkv,d,packed", MAP_CASES)
def test_block_map_and_pairs_match_brute_force(S, R, hq, hkv, d, packed):
    cu = None
    if packed:
        cu = np.array([0, 1, 2, S // 3, S // 3 + 1, S // 2, S - 1, S], dtype=np.int32)
    w = inputs.Workload("case", S, R, hq, hkv, d, backward=False)
    bm, bn = cpattn.cp_tile_shape(hq, hkv, d)
    assert bn == 64 and bm in (64, 128, 256)
    for r in range(R):
        ring = RankRing(w, r, cu, device="cpu")
        for t in range(R):
            p = ring.problem(t, host_docs=True)
            qseg = [(int(p.q_seg[i].pos0), int(p.q_seg[i].len)) for i in range(p.n_q_seg)]
            kseg = [(int(p.kv_seg[j].pos0), int(p.kv_seg[j].len)) for j in range(p.n_kv_seg)]
            ref = oracle.tile_map(qseg, kseg, bm, bn, cu)
            assert np.array_equal(cpattn.cp_block_map(p), ref), (r, t)
            qpos = ring.pos
            kpos = cpattn.cp_partition_zigzag(S, R, ring.schedule()[t])
            assert cpattn.cp_count_pairs(p) == int(oracle.visibility(qpos, kpos, cu).sum())


def test_validation_rejects_bad_problems(lib):
    F = cpattn.CP_MASK_FULL
    good = dict(hq=4, hkv=2, head_dim=128, scale=0.1, q_rows=64, kv_rows=64,
                q_segments=[(0, 0, 64)], kv_segments=[(0, 0, 64)], masks=[[F, F], [F, F]])

    def status(**over):
        kw = dict(good)
        kw.update(over)
        p = cpattn.make_problem(**kw)
        a, b = ctypes.c_int64(), ctypes.c_int64()
        return lib.cp_block_map_size(ctypes.byref(p), ctypes.byref(a), ctypes.byref(b))

    assert status() == cpattn.CP_OK
    assert status(head_dim=96) == cpattn.CP_ERR_UNSUPPORTED
    assert status(hq=6, hkv=4) == cpattn.CP_ERR_INVALID_ARG
    assert status(q_segments=[(0, 0, 65)]) == cpattn.CP_ERR_INVALID_ARG
    assert status(q_segments=[(0, 0, 40), (30, 100, 20)]) == cpattn.CP_ERR_INVALID_ARG
    assert status(kv_segments=[(10, 0, 60)]) == cpattn.CP_ERR_INVALID_ARG
    big = 1 << 62  # row0 + len and pos0 + len would overflow int64
    assert status(q_segments=[(big, 0, big)]) == cpattn.CP_ERR_INVALID_ARG
    assert status(kv_segments=[(0, big, big)]) == cpattn.CP_ERR_INVALID_ARG
    assert status(q_segments=[(0, (1 << 31) - 64, 64)]) == cpattn.CP_OK
    assert status(q_segments=[(0, (1 << 31) - 63, 64)]) == cpattn.CP_ERR_INVALID_ARG
    assert status(masks=[[7, F], [F, F]]) == cpattn.CP_ERR_INVALID_ARG
    assert status(masks=[[cpattn.CP_MASK_DOC, F], [F, F]]) == cpattn.CP_ERR_INVALID_ARG  # no cu_seqlens
    assert status(scale=float("inf")) == cpattn.CP_ERR_INVALID_ARG
    assert status(hq=16384, hkv=8) == cpattn.CP_ERR_UNSUPPORTED
    assert status(hq=8192, hkv=8) == cpattn.CP_OK
    # device entry points validate before any HIP call: these return without launching
    p = cpattn.make_problem(**dict(good, head_dim=80))
    assert lib.cp_attn_fwd_step(ctypes.byref(p), None, None, None, None, None, None, None) == cpattn.CP_ERR_UNSUPPORTED
    assert lib.cp_attn_bwd_step(ctypes.byref(p), None, None, None, None, None, None, None, None, None,
                                None, 0, None) == cpattn.CP_ERR_UNSUPPORTED
    assert lib.cp_merge_partials(None, None, None, None, -1, 4, 128, None) == cpattn.CP_ERR_INVALID_ARG
    assert lib.cp_merge_partials(None, None, None, None, 10, 4, 128, None) == cpattn.CP_ERR_INVALID_ARG
    for n in (0, 65):
        assert lib.cp_merge_partials_n(None, None, None, None, n, 10, 4, 128, None) == cpattn.CP_ERR_INVALID_ARG
    assert lib.cp_merge_partials_n(None, None, None, None, 2, 10, 4, 96, None) == cpattn.CP_ERR_UNSUPPORTED
    assert lib.cp_attn_bwd_prep(None, None, None, 10, 4, 72, None) == cpattn.CP_ERR_UNSUPPORTED
    assert b"head_dim" in lib.cp_last_error()
    # sizes whose element count overflows int64 are refused before any pointer is used
    huge, addr = 1 << 61, 1 << 20
    assert lib.cp_merge_partials(addr, addr, addr, addr, huge, 64, 128, None) == cpattn.CP_ERR_UNSUPPORTED
    assert lib.cp_attn_bwd_prep(addr, addr, addr, huge, 64, 128, None) == cpattn.CP_ERR_UNSUPPORTED
    # misaligned tensor pointers are rejected before any launch (never dereferenced;
    # checked only without a GPU, where a regression could not launch on them)
    import torch
    if torch.cuda.is_available():
        return
    p = cpattn.make_problem(**good)
    ok, bad = 1 << 20, (1 << 20) + 8
    assert lib.cp_attn_fwd_step(ctypes.byref(p), bad, ok, ok, ok, ok, None, None) == cpattn.CP_ERR_INVALID_ARG
    assert b"aligned" in lib.cp_last_error()
    assert lib.cp_attn_fwd_step_merge(ctypes.byref(p), ok, ok, ok, ok, bad, None, None) == cpattn.CP_ERR_INVALID_ARG
    assert lib.cp_attn_bwd_step(ctypes.byref(p), ok, ok, ok, ok, ok, ok, ok, ok, bad,
                                None, 0, None) == cpattn.CP_ERR_INVALID_ARG
    assert lib.cp_attn_bwd_step(ctypes.byref(p), ok, ok, ok, ok, ok, ok, ok, ok, ok,
                                bad, 1 << 20, None) == cpattn.CP_ERR_INVALID_ARG  # misaligned workspace
    assert lib.cp_attn_bwd_step(ctypes.byref(p), ok, ok, ok, ok, ok, ok, ok, ok, ok,
                                None, 64, None) == cpattn.CP_ERR_INVALID_ARG  # bytes without a workspace
    # an explicit split needs its workspace: refused before any launch when it is short
    p.kv_split = 2
    need = cpattn.cp_bwd_workspace_size(p, 2)
    assert need > 0
    assert lib.cp_attn_bwd_step(ctypes.byref(p), ok, ok, ok, ok, ok, ok, ok, ok, ok,
                                ok, need - 16, None) == cpattn.CP_ERR_INVALID_ARG
    assert b"workspace" in lib.cp_last_error()
    p.kv_split = 0
    assert lib.cp_merge_partials(ok, ok, bad, ok, 10, 4, 128, None) == cpattn.CP_ERR_INVALID_ARG
    arr = lambda *a: (ctypes.c_void_p * len(a))(*a)
    assert lib.cp_merge_partials_n(ok, ok, arr(ok, bad), arr(ok, ok), 2, 10, 4, 128, None) == cpattn.CP_ERR_INVALID_ARG
    assert lib.cp_merge_partials_n(ok, ok, arr(ok, None), arr(ok, ok), 2, 10, 4, 128, None) == cpattn.CP_ERR_INVALID_ARG
    assert lib.cp_attn_bwd_prep(ok, ok, bad, 10, 4, 128, None) == cpattn.CP_ERR_INVALID_ARG
    # a KV segment of 1 GiB or more (2^20 keys x 8 heads x 128 dims x 2 bytes) is refused
    big = cpattn.make_problem(32, 8, 128, 0.1, 64, 1 << 20, [(0, 1 << 21, 64)], [(0, 0, 1 << 20)], [[F, F], [F, F]])
    assert lib.cp_attn_fwd_step(ctypes.byref(big), ok, ok, ok, ok, ok, None, None) == cpattn.CP_ERR_UNSUPPORTED
    assert b"1 GiB" in lib.cp_last_error()


def test_clock_probe_arguments(lib):
    """The diagnostics switch only records a pointer: it validates and returns."""
    fake = ctypes.c_void_p(0x1000)
    assert lib.cp_debug_clock_probe(fake, 3) == cpattn.CP_ERR_INVALID_ARG
    assert lib.cp_debug_clock_probe(None, 0) == cpattn.CP_OK
    assert lib.cp_debug_clock_probe(fake, 4) == cpattn.CP_OK
    assert lib.cp_debug_clock_probe(None, 0) == cpattn.CP_OK  # off again


def test_host_cu_seqlens_checked(lib):
    D = cpattn.CP_MASK_DOC
    cu = np.array([0, 10, 5, 64], dtype=np.int32)  # not monotone
    p = cpattn.make_problem(4, 2, 64, 0.1, 64, 64, [(0, 0, 64)], [(0, 0, 64)], [[D, D], [D, D]],
                            cu.ctypes.data, 3)
    with pytest.raises(cpattn.CpError):
        cpattn.cp_block_map(p)
    cu2 = np.array([0, 10, 20], dtype=np.int32)  # does not cover position 63
    p = cpattn.make_problem(4, 2, 64, 0.1, 64, 64, [(0, 0, 64)], [(0, 0, 64)], [[D, D], [D, D]],
                            cu2.ctypes.data, 2)
    with pytest.raises(cpattn.CpError):
        cpattn.cp_count_pairs(p)


def test_schedule_check_rejects_dropped_or_repeated_steps():
    check_schedule(4, [0, 3, 2, 1])
    with pytest.raises(RingScheduleError):
        check_schedule(4, [0, 3, 3, 1])
    with pytest.raises(RingScheduleError):
        check_schedule(4, [0, 3, 2])
    w = inputs.WORKLOADS["tiny"]
    ring = RankRing(w, 1, device="cpu")
    assert ring.schedule() == [oracle.ring_source(1, t, 4) for t in range(4)]
    with pytest.raises(RingScheduleError):
        ring.forward(None, None, schedule=[1, 0, 0, 2])


def test_ring_resume_arguments_checked_before_any_launch():
    """A resumed ring needs the state of the steps before it and a step range
    inside the schedule; both rings refuse otherwise before touching a device."""
    w = inputs.WORKLOADS["tiny"]
    ring = RankRing(w, 2, device="cpu")
    for run in (lambda **kw: ring.forward(None, None, **kw), lambda **kw: ring.backward(None, None, None, None, None, **kw)):
        for kw in (dict(start=1), dict(start=0, state=object()), dict(start=3, stop=2, state=object()),
                   dict(start=0, stop=5), dict(start=-1, state=object())):
            with pytest.raises(ValueError):
                run(**kw)


# ------------------------------------------------------------------ sliding window
@pytest.mark.parametrize("S,R", [(16, 2), (48, 3), (64, 4), (80, 5), (512, 4)])
def test_window_step_masks_match_brute_force(S, R):
    """cp_step_masks_window's closed form against the oracle's brute-force classes for
    windows inside a chunk, across chunks, exactly at chunk multiples and beyond."""
    c = S // (2 * R)
    cu = np.array([0, 3, 3, S // 2 + 1, S], dtype=np.int32)
    windows = sorted({1, 2, c - 1, c, c + 1, 2 * c - 1, 2 * c, 2 * c + 1, 3 * c, S, 0} - {-1})
    for wdw in windows:
        if wdw < 0:
            continue
        for r in range(R):
            qpos = oracle.zigzag_positions(S, R, r)
            for t in range(R):
                kpos = oracle.zigzag_positions(S, R, oracle.ring_source(r, t, R))
                for packed in (False, True):
                    got = cpattn.cp_step_masks_window(S, R, r, t, packed, wdw)
                    for i in range(2):
                        for j in range(2):
                            ref = oracle.chunk_pair_class(qpos[i * c:(i + 1) * c], kpos[j * c:(j + 1) * c],
                                                          cu if packed else None, wdw)
                            if packed and ref == oracle.CLS_SKIP:
                                assert got[i][j] in (oracle.CLS_SKIP, oracle.CLS_DOC)
                            else:
                                assert got[i][j] == ref, (wdw, r, t, i, j, packed)
    # window 0 is the plain causal classification
    for r in range(R):
        for t in range(R):
            assert cpattn.cp_step_masks_window(S, R, r, t, False, 0) == cpattn.cp_step_masks(R, r, t, False)


WINDOW_MAP_CASES = [
    # S, R, Hq, Hkv, D, packed, window
    (400, 2, 8, 2, 128, False, 37),
    (462, 3, 4, 4, 64, False, 77),
    (462, 3, 4, 4, 64, False, 100),
    (360, 2, 6, 3, 128, True, 50),
    (1024, 4, 8, 2, 128, False, 128),
    (1024, 4, 8, 2, 128, True, 300),
]


@pytest.mark.parametrize("S,R,hq,hkv,d,packed,window", WINDOW_MAP_CASES)
def test_window_block_map_and_pairs_match_brute_force(S, R, hq, hkv, d, packed, window):
    cu = None
    if packed:
        cu = np.array([0, 1, 2, S // 3, S // 3 + 1, S // 2, S - 1, S], dtype=np.int32)
    w = inputs.Workload("case", S, R, hq, hkv, d, backward=False, packed=packed, window=window)
    bm, bn = cpattn.cp_tile_shape(hq, hkv, d)
    for r in range(R):
        ring = RankRing(w, r, cu, device="cpu")
        for t in range(R):
            src = ring.schedule()[t]
            p = ring.problem(t, host_docs=True)
            assert p.window == window
            qseg = [(int(p.q_seg[i].pos0), int(p.q_seg[i].len)) for i in range(p.n_q_seg)]
            kseg = [(int(p.kv_seg[j].pos0), int(p.kv_seg[j].len)) for j in range(p.n_kv_seg)]
            ref = oracle.tile_map(qseg, kseg, bm, bn, cu, window)
            assert np.array_equal(cpattn.cp_block_map(p), ref), (r, t)
            kpos = cpattn.cp_partition_zigzag(S, R, src)
            vis = oracle.visibility(ring.pos, kpos, cu, window)
            assert cpattn.cp_count_pairs(p) == int(vis.sum())
            if packed:  # document boundaries are not known to the chunk classes: live is conservative
                assert ring.source_live(src) or not vis.any()
            else:
                assert ring.source_live(src) == bool(vis.any()) or t == 0


def test_window_validation():
    F = cpattn.CP_MASK_FULL
    p = cpattn.make_problem(4, 2, 128, 0.1, 64, 64, [(0, 0, 64)], [(0, 0, 64)], [[F, F], [F, F]], window=-1)
    with pytest.raises(cpattn.CpError) as e:
        cpattn.cp_count_pairs(p)
    assert e.value.status == cpattn.CP_ERR_INVALID_ARG
    with pytest.raises(cpattn.CpError):
        cpattn.cp_step_masks_window(64, 4, 0, 0, False, -5)
    with pytest.raises(cpattn.CpError):
        cpattn.cp_step_masks_window(60, 4, 0, 0, False, 5)


def test_ring_masks_follow_the_block_not_the_step():
    """problem(t, src) classifies against the block actually passed: a permuted but
    complete schedule gets the classes of each block's own arrival step."""
    w = inputs.Workload("perm", 64, 4, 4, 2, 64, backward=False, window=12)
    ring = RankRing(w, 1, device="cpu")
    for src in range(4):
        natural = (1 - src) % 4
        for t in range(4):
            p = ring.problem(t, src, host_docs=True)
            assert [[p.mask[i][j] for j in range(2)] for i in range(2)] == \
                cpattn.cp_step_masks_window(64, 4, 1, natural, False, 12)


def test_kv_split_rule():
    """The dK/dV work split: 1 on the balanced causal steps of the training
    workload, > 1 where a sliding window leaves a triangle of pairs, within
    [1, 8] everywhere."""
    w = inputs.WORKLOADS["llama3_8b_fwdbwd"]
    ring = RankRing(w, 0, device="cpu")
    for t in range(w.cp):
        assert cpattn.cp_bwd_kv_split(ring.problem(t, host_docs=True), 256) == 1
    ww = inputs.WORKLOADS["llama3_8b_window4k"]
    ring = RankRing(ww, 0, device="cpu")
    p7 = ring.problem(ww.cp - 1, host_docs=True)  # the neighbour block: a 4K-wide triangle
    assert cpattn.cp_bwd_kv_split(p7, 256) >= 2
    for t in range(ww.cp):
        assert 1 <= cpattn.cp_bwd_kv_split(ring.problem(t, host_docs=True), 256) <= 8
    wp = inputs.WORKLOADS["llama3_8b_packed"]
    ring = RankRing(wp, 5, wp.cu_seqlens(), device="cpu")
    for t in range(wp.cp):
        assert 1 <= cpattn.cp_bwd_kv_split(ring.problem(t, host_docs=True), 256) <= 8


def test_kv_split_simulated_launch():
    """One 128-key block of one KV head seen by 128 query tiles (FULL): alone it
    takes 128 items plus a fixed cost of 3; split s ways each part takes
    128/s + 3, and the reduction pass reads s + 1 slots at 0.03 each.  With 512
    slots all parts run at once (8 parts: 19.3 against 131); with 2 slots (one
    CU) 2 parts take 67.1, 4 parts 2 x 35 + 0.15 and 8 parts 4 x 19 + 0.27."""
    F, S_ = cpattn.CP_MASK_FULL, cpattn.CP_MASK_SKIP
    p = cpattn.make_problem(1, 1, 128, 0.1, 4096, 128, [(0, 0, 4096)], [(0, 5000, 128)], [[F, S_], [S_, S_]])
    assert cpattn.cp_bwd_kv_split(p, 256) == 8
    assert cpattn.cp_bwd_kv_split(p, 1) == 2
    # 256 equal workgroups (32 blocks x 8 KV heads): two full rounds on 64 CUs are
    # not split; on 256 CUs they fill half of the slots, and halves fill them all
    # (67 per part, plus 0.03 x 3 x 256 for the reduction, against 131)
    p = cpattn.make_problem(8, 8, 128, 0.1, 4096, 4096, [(0, 0, 4096)], [(0, 5000, 4096)], [[F, S_], [S_, S_]])
    assert cpattn.cp_bwd_kv_split(p, 64) == 1
    assert cpattn.cp_bwd_kv_split(p, 256) == 2


def test_bwd_workspace_size():
    """(split - 1) slots of 2 x 128 x D floats per 128-key block of every KV head."""
    F, S_ = cpattn.CP_MASK_FULL, cpattn.CP_MASK_SKIP
    for d in (64, 128):
        p = cpattn.make_problem(8, 2, d, 0.1, 300, 700, [(0, 0, 300)], [(0, 400, 200), (200, 900, 500)],
                                [[F, S_], [S_, S_]])
        blocks = (2 + 4) * 2  # ceil(200/128) + ceil(500/128) key blocks, 2 KV heads
        assert cpattn.cp_bwd_workspace_size(p, 1) == 0
        for split in (2, 3, 8):
            assert cpattn.cp_bwd_workspace_size(p, split) == (split - 1) * blocks * 2 * 128 * d * 4
        for bad in (0, 9, -1):
            with pytest.raises(cpattn.CpError) as e:
                cpattn.cp_bwd_workspace_size(p, bad)
            assert e.value.status == cpattn.CP_ERR_INVALID_ARG


def test_kv_split_validation():
    F = cpattn.CP_MASK_FULL
    p = cpattn.make_problem(4, 2, 128, 0.1, 64, 64, [(0, 0, 64)], [(0, 0, 64)], [[F, F], [F, F]])
    with pytest.raises(cpattn.CpError) as e:
        cpattn.cp_bwd_kv_split(p, 0)
    assert e.value.status == cpattn.CP_ERR_INVALID_ARG
    for bad in (-1, 9):
        p.kv_split = bad
        with pytest.raises(cpattn.CpError) as e:
            cpattn.cp_count_pairs(p)
        assert e.value.status == cpattn.CP_ERR_INVALID_ARG
    p.kv_split = 8
    assert cpattn.cp_count_pairs(p) == 64 * 64


@st.composite
def _random_problem(draw):
    """Arbitrary segments (not ring-shaped): 1-2 query and 1-2 KV segments at random
    positions, DIAG or DOC classes (the ones whose visibility the host derives from
    positions), optional documents and window."""
    hq, hkv = draw(st.sampled_from([(8, 2), (4, 4), (6, 2), (16, 1)]))
    d = draw(st.sampled_from([64, 128]))
    span = 600
    def segs(n_max):
        out, row = [], 0
        for _ in range(draw(st.integers(1, n_max))):
            ln = draw(st.integers(0, 200))
            out.append((row, draw(st.integers(0, span)), ln))
            row += ln
        return out, row
    qs, q_rows = segs(2)
    ks, kv_rows = segs(2)
    docs = draw(st.booleans())
    cu = None
    if docs:
        cuts = sorted(set(draw(st.lists(st.integers(1, span + 200), max_size=6))))
        cu = np.array([0] + cuts + [span + 201], dtype=np.int32)
    m = cpattn.CP_MASK_DOC if docs else cpattn.CP_MASK_DIAG_CAUSAL
    window = draw(st.sampled_from([0, 0, 1, 17, 64, 150]))
    return hq, hkv, d, qs, q_rows, ks, kv_rows, m, cu, window


@settings(max_examples=300, deadline=None)
@given(_random_problem())
def test_block_map_and_pairs_on_arbitrary_segments(prob):
    """The host block map and pair count against the oracle's brute force on
    problems the ring never builds: overlapping position ranges, empty segments,
    segments that start mid-document."""
    hq, hkv, d, qs, q_rows, ks, kv_rows, m, cu, window = prob
    p = cpattn.make_problem(hq, hkv, d, 0.1, max(q_rows, 1), max(kv_rows, 1), qs, ks, [[m, m], [m, m]],
                            None if cu is None else cu.ctypes.data, 0 if cu is None else len(cu) - 1, window)
    bm, bn = cpattn.cp_tile_shape(hq, hkv, d)
    ref = oracle.tile_map([(s[1], s[2]) for s in qs], [(s[1], s[2]) for s in ks], bm, bn, cu, window or None)
    assert np.array_equal(cpattn.cp_block_map(p), ref)
    want = 0
    for _, qp, ql in qs:
        for _, kp, kl in ks:
            want += int(oracle.visibility(np.arange(qp, qp + ql), np.arange(kp, kp + kl), cu, window or None).sum())
    assert cpattn.cp_count_pairs(p) == want


def test_binding_refuses_strided_tensors():
    """The ABI takes dense row-major buffers: the binding passes a contiguous
    tensor's address and refuses a transposed or column-sliced view, whose
    data_ptr would be read with the wrong layout."""
    torch = pytest.importorskip("torch")
    a = torch.zeros((6, 4), dtype=torch.float32)
    assert cpattn._ptr(a).value == a.data_ptr()
    assert cpattn._ptr(a[2:5]).value == a[2:5].data_ptr()  # a run of rows stays dense
    assert cpattn._ptr(None) is None
    for bad in (a.t(), a[:, 1:3], torch.zeros((4, 6)).t().contiguous().t()):
        with pytest.raises(ValueError, match="not contiguous"):
            cpattn._ptr(bad)


class _FakeDeviceTensor:
    """Stands in for a dense GPU tensor: the binding's size checks read only these."""

    def __init__(self, numel, elem, cuda=True):
        self._n, self._e, self.is_cuda = numel, elem, cuda
        self.shape, self.dtype = (numel,), f"{elem}-byte"

    def numel(self):
        return self._n

    def element_size(self):
        return self._e

    def is_contiguous(self):
        return True

    def stride(self):
        return (1,)

    def data_ptr(self):
        return 4096


def test_binding_refuses_buffers_too_small_or_of_the_wrong_kind():
    """The C ABI sees bare pointers, so the binding checks every device buffer
    against the layout the call uses: element size, at least the implied number
    of elements, on the GPU; a refused call never reaches the library."""
    p = cpattn.make_problem(8, 2, 64, 0.125, 100, 70, [(0, 0, 100)], [(0, 0, 70)],
                            [[cpattn.CP_MASK_DIAG_CAUSAL] * 2] * 2)
    nq, nk, nl = 100 * 8 * 64, 70 * 2 * 64, 8 * 100
    good = dict(q=_FakeDeviceTensor(nq, 2), k=_FakeDeviceTensor(nk, 2), v=_FakeDeviceTensor(nk, 2),
                o=_FakeDeviceTensor(nq, 4), lse=_FakeDeviceTensor(nl, 4))
    assert all(x is not None for x in cpattn._fwd_args(p, tile_map=None, **good)[:5])
    for name, bad in [("q", _FakeDeviceTensor(nq - 1, 2)), ("k", _FakeDeviceTensor(nk, 4)),
                      ("o", _FakeDeviceTensor(nq, 2)), ("lse", _FakeDeviceTensor(nl - 8, 4)),
                      ("v", _FakeDeviceTensor(nk, 2, cuda=False))]:
        with pytest.raises(ValueError, match=name):
            cpattn._fwd_args(p, tile_map=None, **dict(good, **{name: bad}))
    bwd = dict(q=good["q"], k=good["k"], v=good["v"], d_o=_FakeDeviceTensor(nq, 2), lse=good["lse"],
               delta=_FakeDeviceTensor(nl, 4), dq=_FakeDeviceTensor(nq, 4), dk=_FakeDeviceTensor(nk, 4),
               dv=_FakeDeviceTensor(nk, 4))
    assert all(x is not None for x in cpattn._bwd_args(p, **bwd))
    for name in ("delta", "dq", "dk"):
        with pytest.raises(ValueError):
            cpattn._bwd_args(p, **dict(bwd, **{name: _FakeDeviceTensor(10, 4)}))
