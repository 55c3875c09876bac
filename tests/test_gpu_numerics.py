"""GPU numerics of the step kernels on adversarial score ranges, against the float64
oracle, through the C ABI.

The forward kernel keeps no running row maximum: it takes exponentials against the
reference set by a row's first visible tile and falls back to a rescale when a
tile's sum leaves range.  These cases drive that fallback: scores that grow by
hundreds of log2 units from the first tile to the last, huge scores that would
overflow fp32 without the rescale, first tiles far below the rest, and rows whose
first tiles are fully masked (documents, windows).  The backward cases cover empty
and SKIP segments.
"""
import numpy as np
import pytest

import oracle
from context_long_attention_amd import inputs
from tests.gpu_common import assert_lse_close, assert_o_close, device_bf16, note

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _needs_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from context_long_attention_amd import cpattn
    cpattn.lib()


def _inputs(n, m, hq, hkv, d, k_gain, q_gain=1.0, seed=0):
    """Q and V ~ N(0, 1) (Q times q_gain), K ~ N(0, 1) times a per-key gain k_gain[j]."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((n, hq, d)).astype(np.float32) * np.float32(q_gain)
    k = rng.standard_normal((m, hkv, d)).astype(np.float32) * np.asarray(k_gain, np.float32)[:, None, None]
    v = rng.standard_normal((m, hkv, d)).astype(np.float32)
    return device_bf16(q), device_bf16(k), device_bf16(v)


def _run_fwd(p, q, k, v, n, hq, d):
    from context_long_attention_amd import cpattn
    o = torch.zeros((n, hq, d), dtype=torch.float32, device="cuda")
    lse = torch.full((hq, n), float("-inf"), dtype=torch.float32, device="cuda")
    cpattn.cp_attn_fwd_step(p, q, k, v, o, lse)
    torch.cuda.synchronize()
    return o, lse


GROWTH = [
    # name, d, k gain from first to last key, q gain
    ("rising_d128", 128, (0.2, 8.0), 4.0),
    ("rising_d64", 64, (0.2, 8.0), 4.0),
    ("falling_d128", 128, (8.0, 0.2), 4.0),
    ("huge_d128", 128, (6.0, 6.0), 8.0),
]


@pytest.mark.parametrize("name,d,gain,q_gain", GROWTH, ids=[g[0] for g in GROWTH])
@pytest.mark.parametrize("mask", ["full", "causal"])
def test_forward_extreme_score_ranges(name, d, gain, q_gain, mask):
    """Scores spanning hundreds of log2 units across the key tiles of a row: the
    tile-sum check must rescale (rising), keep P tiny but exact (falling), and never
    overflow (huge: scores of several thousand)."""
    from context_long_attention_amd import cpattn
    n, hq, hkv = 640, 4, 2
    note(f"numerics {name} mask={mask}")
    k_gain = np.linspace(gain[0], gain[1], n)
    (q64, q), (k64, k), (v64, v) = _inputs(n, n, hq, hkv, d, k_gain, q_gain)
    m = cpattn.CP_MASK_FULL if mask == "full" else cpattn.CP_MASK_DIAG_CAUSAL
    scale = 1.0 / np.sqrt(d)
    p = cpattn.make_problem(hq, hkv, d, scale, n, n, [(0, 0, n)], [(0, 0, n)], [[m, m], [m, m]])
    o, lse = _run_fwd(p, q, k, v, n, hq, d)
    pos = np.arange(n)
    vis = np.ones((n, n), bool) if mask == "full" else oracle.visibility(pos, pos)
    ro, rl = oracle.attention_partial(q64, k64, v64, vis, scale)
    assert not torch.isnan(o).any().item() and not torch.isinf(o).any().item()
    assert_o_close(o.cpu().numpy(), ro, f"{name} O")
    assert_lse_close(lse.cpu().numpy(), rl, f"{name} LSE")
    # the merging kernel from the empty state gives the same result
    o2 = torch.zeros_like(o)
    l2 = torch.full_like(lse, float("-inf"))
    cpattn.cp_attn_fwd_step_merge(p, q, k, v, o2, l2)
    torch.cuda.synchronize()
    assert_o_close(o2.cpu().numpy(), ro, f"{name} merged O")
    assert_lse_close(l2.cpu().numpy(), rl, f"{name} merged LSE")


def test_forward_first_tiles_masked_with_large_scores():
    """Documents and a window leave the first key tiles of many rows fully masked, so
    those rows have no reference until a later tile; with large scores the first
    visible tile must set it."""
    from context_long_attention_amd import cpattn
    n, hq, hkv, d = 700, 4, 1, 128
    cu = np.array([0, 130, 131, 400, 700], dtype=np.int32)
    cu_dev = torch.from_numpy(cu).cuda()
    k_gain = np.linspace(0.5, 6.0, n)
    (q64, q), (k64, k), (v64, v) = _inputs(n, n, hq, hkv, d, k_gain, 5.0, seed=3)
    pos = np.arange(n)
    for window in (0, 90):
        note(f"numerics masked first tiles window={window}")
        Dm = cpattn.CP_MASK_DOC
        p = cpattn.make_problem(hq, hkv, d, 0.1, n, n, [(0, 0, n)], [(0, 0, n)], [[Dm, Dm], [Dm, Dm]],
                                cu_dev.data_ptr(), len(cu) - 1, window)
        o, lse = _run_fwd(p, q, k, v, n, hq, d)
        ro, rl = oracle.attention_partial(q64, k64, v64, oracle.visibility(pos, pos, cu, window or None), 0.1)
        assert_o_close(o.cpu().numpy(), ro, f"masked-first O w={window}")
        assert_lse_close(lse.cpu().numpy(), rl, f"masked-first LSE w={window}")


def test_backward_extreme_scores_and_empty_segments():
    """The backward step on large, rising scores (exponentials against the final LSE),
    then on an empty KV segment, an empty query segment and an all-SKIP step: dK/dV of
    the KV rows are overwritten (zeros where nothing is visible) and dQ is unchanged."""
    from context_long_attention_amd import cpattn
    n, hq, hkv, d = 384, 4, 2, 128
    k_gain = np.linspace(0.3, 6.0, n)
    (q64, q), (k64, k), (v64, v) = _inputs(n, n, hq, hkv, d, k_gain, 4.0, seed=5)
    do64, do = device_bf16(inputs.chunk_normal(4, 0, n, hq, d))
    D_ = cpattn.CP_MASK_DIAG_CAUSAL
    S_ = cpattn.CP_MASK_SKIP
    scale = 1.0 / np.sqrt(d)
    pos = np.arange(n)
    vis = oracle.visibility(pos, pos)
    p = cpattn.make_problem(hq, hkv, d, scale, n, n, [(0, 0, n)], [(0, 0, n)], [[D_, D_], [D_, D_]])
    o, lse = _run_fwd(p, q, k, v, n, hq, d)
    delta = torch.empty_like(lse)
    cpattn.cp_attn_bwd_prep(do, o, delta, n, hq, d)
    dq = torch.zeros_like(o)
    dk = torch.full((n, hkv, d), 7.0, device="cuda")
    dv = torch.full_like(dk, 7.0)
    cpattn.cp_attn_bwd_step(p, q, k, v, do, lse, delta, dq, dk, dv)
    torch.cuda.synchronize()
    ro, rl = oracle.attention_partial(q64, k64, v64, vis, scale)
    rdq, rdk, rdv = oracle.attention_backward_partial(q64, k64, v64, do64, rl, oracle.delta_rows(do64, ro), vis,
                                                      scale)
    def close(got, ref, what):
        # gradients scale with the scores here; compare relative to their magnitude
        g = got.cpu().numpy()
        assert np.isfinite(g).all(), what
        err = np.abs(g - ref).max() / max(1.0, np.abs(ref).max())
        assert err <= 2e-2, f"{what}: max error {err:.3e} of the largest magnitude"

    for got, ref, what in ((dq, rdq, "dQ"), (dk, rdk, "dK"), (dv, rdv, "dV")):
        close(got, ref, what)
    # empty KV segment and SKIP pairs: only the visible segment contributes
    dq0 = dq.clone()
    dk.fill_(7.0)
    dv.fill_(7.0)
    p = cpattn.make_problem(hq, hkv, d, scale, n, n, [(0, 0, n)], [(0, 0, 0), (0, 0, n)], [[S_, D_], [S_, S_]])
    cpattn.cp_attn_bwd_step(p, q, k, v, do, lse, delta, dq, dk, dv)
    torch.cuda.synchronize()
    close(dq - dq0, rdq, "dQ through the second KV segment")
    close(dk, rdk, "dK through the second KV segment")
    # an all-SKIP step writes zero dK/dV for its KV rows and leaves dQ alone
    dq1 = dq.clone()
    dk.fill_(7.0)
    dv.fill_(7.0)
    p = cpattn.make_problem(hq, hkv, d, scale, n, n, [(0, 0, n)], [(0, 0, n)], [[S_, S_], [S_, S_]])
    cpattn.cp_attn_bwd_step(p, q, k, v, do, lse, delta, dq, dk, dv)
    torch.cuda.synchronize()
    assert torch.all(dq == dq1).item()
    assert torch.all(dk == 0).item() and torch.all(dv == 0).item()
    # an empty query segment: nothing visible, zero dK/dV, dQ untouched
    dk.fill_(7.0)
    p = cpattn.make_problem(hq, hkv, d, scale, n, n, [(0, 0, 0)], [(0, 0, n)], [[D_, D_], [D_, D_]])
    cpattn.cp_attn_bwd_step(p, q, k, v, do, lse, delta, dq, dk, dv)
    torch.cuda.synchronize()
    assert torch.all(dq == dq1).item()
    assert torch.all(dk == 0).item()
