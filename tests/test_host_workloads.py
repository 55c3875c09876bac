"""CPU checks of the synthetic workloads and of the host pair counts at full size."""
import numpy as np

from context_long_attention_amd import inputs


def test_packed_layout_matches_recipe():
    """The packed workload's documents follow the recipe, and the host's per-(rank, step)
    visible-pair counts add up to the exact total sum over documents of L(L+1)/2: every
    visible pair is computed by exactly one rank at exactly one ring step."""
    from tests.test_gpu_large import _packed_setup
    w, cu, pairs = _packed_setup()
    lens = np.diff(cu.astype(np.int64))
    assert cu[0] == 0 and cu[-1] == w.seq_len
    assert (lens[:-1] >= 256).all() and (lens <= 524288).all()
    assert int(pairs.sum()) == int((lens * (lens + 1) // 2).sum())
    # reproducible from the seed
    assert np.array_equal(cu, w.cu_seqlens())


def test_causal_workloads_are_balanced():
    """Zigzag balance at the configured sizes: 2Rc^2 + c pairs per head on every rank."""
    from context_long_attention_amd.ring import RankRing
    for name in ("llama3_8b_fwd", "llama3_8b_fwdbwd", "llama3_405b_fwd"):
        w = inputs.WORKLOADS[name]
        c = w.chunk
        for r in (0, w.cp // 2, w.cp - 1):
            ring = RankRing(w, r, device="cpu")
            assert sum(ring.step_pairs(t) for t in range(w.cp)) == 2 * w.cp * c * c + c
