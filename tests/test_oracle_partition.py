"""Pins of the oracle's partition, ring order, chunk classes and block map (CPU only)."""
import os
import re

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "zigzag_4tokens_2ranks.txt")


def _read_golden():
    rows = {}
    with open(GOLDEN) as f:
        for line in f:
            m = re.match(r"rank (\d+): ([\d ]+)\| blocks (\d+)", line.strip())
            if m:
                rows[int(m.group(1))] = ([int(x) for x in m.group(2).split()], int(m.group(3)))
    return rows


def test_worked_example_from_pages():
    """4 tokens on 2 ranks: rank 0 -> {0, 3}, rank 1 -> {1, 2}, 5 causal blocks each."""
    golden = _read_golden()
    assert sorted(golden) == [0, 1]
    for r, (positions, blocks) in golden.items():
        pos = oracle.zigzag_positions(4, 2, r)
        assert pos.tolist() == positions
        assert int(oracle.visibility(pos, np.arange(4)).sum()) == blocks


@pytest.mark.parametrize("S,R", [(4, 2), (16, 2), (24, 3), (64, 4), (80, 5), (512, 4), (96, 1)])
def test_partition_invariants(S, R):
    c = S // (2 * R)
    allpos = []
    for r in range(R):
        pos = oracle.zigzag_positions(S, R, r)
        assert pos.shape == (S // R,)
        assert pos.dtype == np.int64
        # local order: chunk r first, then chunk 2R-1-r, each contiguous
        assert pos[0] == r * c and pos[c] == (2 * R - 1 - r) * c
        assert np.all(np.diff(pos[:c]) == 1) and np.all(np.diff(pos[c:]) == 1)
        # equal causal work on every rank: 2 R c^2 + c pairs (closed form of the balance claim)
        assert int(oracle.visibility(pos, np.arange(S)).sum()) == 2 * R * c * c + c
        allpos.append(pos)
    allpos = np.concatenate(allpos)
    assert np.array_equal(np.sort(allpos), np.arange(S))
    assert sum(int(oracle.visibility(oracle.zigzag_positions(S, R, r), np.arange(S)).sum())
               for r in range(R)) == S * (S + 1) // 2


def test_partition_rejects_indivisible():
    with pytest.raises(ValueError):
        oracle.zigzag_positions(10, 3, 0)


@pytest.mark.parametrize("R", [1, 2, 3, 4, 8, 16])
def test_ring_visits_every_source_once(R):
    for r in range(R):
        srcs = [oracle.ring_source(r, t, R) for t in range(R)]
        assert srcs[0] == r
        assert sorted(srcs) == list(range(R))
        # the block held at step t+1 is the one the previous rank held at step t
        for t in range(R - 1):
            assert oracle.ring_source(r, t + 1, R) == oracle.ring_source((r - 1) % R, t, R)


def _closed_form_classes(R, r, t):
    """Chunk-pair classes of step t in closed form (query chunk a/b x key chunk s / 2R-1-s)."""
    F, D, S_ = oracle.CLS_FULL, oracle.CLS_DIAG, oracle.CLS_SKIP
    s = (r - t) % R
    if s == r:
        return [[D, S_], [F, D]]
    if s < r:
        return [[F, S_], [F, S_]]
    return [[S_, S_], [F, F]]


@pytest.mark.parametrize("S,R", [(16, 2), (24, 3), (64, 4), (80, 5), (512, 4)])
def test_chunk_classes_closed_form(S, R):
    c = S // (2 * R)
    for r in range(R):
        qpos = oracle.zigzag_positions(S, R, r)
        for t in range(R):
            s = oracle.ring_source(r, t, R)
            kpos = oracle.zigzag_positions(S, R, s)
            got = [[oracle.chunk_pair_class(qpos[i * c:(i + 1) * c], kpos[j * c:(j + 1) * c])
                    for j in range(2)] for i in range(2)]
            assert got == _closed_form_classes(R, r, t)
            # visible pairs per head: 2c^2 + c at step 0, 2c^2 on every other step
            pairs = int(oracle.visibility(qpos, kpos).sum())
            assert pairs == (2 * c * c + c if t == 0 else 2 * c * c)


def test_doc_classes():
    cu = np.array([0, 5, 6, 20, 32])
    qpos = oracle.zigzag_positions(32, 2, 0)
    kpos = oracle.zigzag_positions(32, 2, 1)
    c = 8
    # query chunk 0 (pos 0..7) never sees chunk 1 (8..15) or chunk 2 (16..23): SKIP
    assert oracle.chunk_pair_class(qpos[:c], kpos[:c], cu) == oracle.CLS_SKIP
    # query chunk 3 (24..31) sees part of chunk 2 (doc [20, 32)): DOC
    assert oracle.chunk_pair_class(qpos[c:], kpos[c:], cu) == oracle.CLS_DOC


def _loop_tile_map(q_segments, kv_segments, bm, bn, cu=None):
    """Pure-Python brute force over every (query, key) pair, written with loops."""
    def doc(p):
        if cu is None:
            return 0
        d = 0
        while d + 1 < len(cu) and cu[d + 1] <= p:
            d += 1
        return d
    qt = [(p0 + s, min(bm, n - s)) for p0, n in q_segments for s in range(0, n, bm)]
    kt = [(p0 + s, min(bn, n - s)) for p0, n in kv_segments for s in range(0, n, bn)]
    out = np.zeros((len(qt), len(kt)), np.uint8)
    for i, (q0, ql) in enumerate(qt):
        for j, (k0, kl) in enumerate(kt):
            n_vis = 0
            for qq in range(q0, q0 + ql):
                for kk in range(k0, k0 + kl):
                    if kk <= qq and doc(kk) == doc(qq):
                        n_vis += 1
            out[i, j] = 2 if n_vis == ql * kl else (1 if n_vis else 0)
    return out


@pytest.mark.parametrize("bm,bn", [(4, 4), (3, 5), (8, 2)])
def test_tile_map_against_loops(bm, bn):
    cu = np.array([0, 7, 9, 23, 40])
    q_segments = [(0, 10), (30, 10)]
    kv_segments = [(10, 10), (20, 10)]
    for docs in (None, cu):
        assert np.array_equal(oracle.tile_map(q_segments, kv_segments, bm, bn, docs),
                              _loop_tile_map(q_segments, kv_segments, bm, bn, docs))
    # own block at step 0 of rank 0, S = 40, R = 2: chunks 0 and 3
    own = [(0, 10), (30, 10)]
    assert np.array_equal(oracle.tile_map(own, own, bm, bn), _loop_tile_map(own, own, bm, bn))


def test_tile_map_diagonal_closed_form():
    """A c x c diagonal chunk with tiles dividing c: c/b partial tiles, (c/b)(c/b-1)/2 full."""
    c, b = 64, 8
    tm = oracle.tile_map([(128, c)], [(128, c)], b, b)
    n = c // b
    assert int((tm == oracle.TILE_PARTIAL).sum()) == n
    assert int((tm == oracle.TILE_FULL).sum()) == n * (n - 1) // 2
    assert np.array_equal(tm == oracle.TILE_PARTIAL, np.eye(n, dtype=bool))


def test_tile_map_accounts_for_every_pair():
    """Full-tile areas plus the visible pairs of partial tiles give the step's pair count."""
    S, R, r, t = 96, 3, 1, 0
    bm, bn = 5, 7
    qpos = oracle.zigzag_positions(S, R, r)
    kpos = oracle.zigzag_positions(S, R, oracle.ring_source(r, t, R))
    c = S // (2 * R)
    qseg = [(int(qpos[0]), c), (int(qpos[c]), c)]
    kseg = [(int(kpos[0]), c), (int(kpos[c]), c)]
    tm = oracle.tile_map(qseg, kseg, bm, bn)
    qt = [(p0 + s, min(bm, n - s)) for p0, n in qseg for s in range(0, n, bm)]
    kt = [(p0 + s, min(bn, n - s)) for p0, n in kseg for s in range(0, n, bn)]
    total = 0
    for i, (q0, ql) in enumerate(qt):
        for j, (k0, kl) in enumerate(kt):
            if tm[i, j] == oracle.TILE_FULL:
                total += ql * kl
            elif tm[i, j] == oracle.TILE_PARTIAL:
                total += int(oracle.visibility(np.arange(q0, q0 + ql), np.arange(k0, k0 + kl)).sum())
    assert total == 2 * c * c + c
