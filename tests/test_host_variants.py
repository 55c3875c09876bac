"""CPU tests of the variant schedulers' host logic: every step problem of Pass Q
and of partial prefill is valid, and its visible-pair count (host) equals the
oracle's brute-force visibility between the same positions.  No kernel runs."""
import numpy as np
import pytest

import oracle
from oracle import variants as ov
from context_long_attention_amd import cpattn, inputs
from context_long_attention_amd.variants import PartialPrefillRank, PassQRank


@pytest.mark.parametrize("S,R,packed", [(64, 4, False), (96, 3, True), (512, 8, False), (240, 5, True)])
def test_pass_q_problems_count_the_right_pairs(S, R, packed):
    w = inputs.Workload("pq", S, R, 4, 2, 64, backward=False)
    cu = np.array([0, 3, S // 3, S // 3 + 1, S], dtype=np.int32) if packed else None
    total = 0
    for r in range(R):
        rank = PassQRank(w, r, cu, device="cpu")
        kpos = oracle.zigzag_positions(S, R, r)
        assert rank.schedule() == [oracle.ring_source(r, t, R) for t in range(R)]
        for t, s in enumerate(rank.schedule()):
            p = rank.problem(t, host_docs=True)
            want = int(oracle.visibility(oracle.zigzag_positions(S, R, s), kpos, cu).sum())
            assert cpattn.cp_count_pairs(p) == want, (r, t)
            total += want
    # over all ranks and steps Pass Q covers every visible pair of the sequence once
    assert total == int(oracle.visibility(np.arange(S), np.arange(S), cu).sum())


@pytest.mark.parametrize("P,N,R", [(48, 32, 2), (0, 64, 4), (96, 24, 3)])
def test_partial_prefill_problems_count_the_right_pairs(P, N, R):
    total = 0
    for r in range(R):
        rank = PartialPrefillRank(P, N, R, 4, 2, 64, r, device="cpu")
        _, new_r = ov.partial_prefill_positions(P, N, R, r)
        for t, s in enumerate(rank.schedule()):
            cached_s, new_s = ov.partial_prefill_positions(P, N, R, s)
            probs = rank.problems(t)
            # one call per step, two on the diagonal step (where the new share has causal pairs)
            assert len(probs) == (2 if s == r else 1)
            got = sum(cpattn.cp_count_pairs(p) for p in probs)
            assert got == int(oracle.visibility(new_r, cached_s).sum()) + int(oracle.visibility(new_r, new_s).sum())
            for p in probs:  # every segment lies inside the receive buffer [cached ; new]
                assert p.kv_rows == len(cached_s) + len(new_s)
            total += got
    S = P + N
    assert total == int(oracle.visibility(np.arange(P, S), np.arange(S)).sum())


def test_partial_prefill_rejects_uneven_split():
    with pytest.raises(ValueError):
        PartialPrefillRank(50, 32, 2, 4, 2, 64, 0, device="cpu")
