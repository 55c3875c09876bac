"""The allocation-free backward entry point, cp_attn_bwd_step_noalloc, against
cp_attn_bwd_step with a caller-supplied workspace, through the C ABI.  Two
calls in a row on different problems, the second smaller, at explicit dK/dV
splits whose workspace fits the library's fixed scratch and at the library's
own choice: the same bits as the workspace entry point (whose workspace is
pre-filled with NaN) and the oracle's values within the parity tolerance.  A
split whose workspace exceeds the scratch is refused before any launch."""
import ctypes

import numpy as np
import pytest

import oracle
from context_long_attention_amd import inputs
from tests.gpu_common import RankInputs, assert_o_close, note

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _needs_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from context_long_attention_amd import cpattn
    cpattn.lib()


# name, S, R, Hq, Hkv, D, window, rank, step -- the second problem is the smaller one
CASES = [
    ("window_g4_d128", 2 * 4 * 192, 4, 8, 2, 128, 64, 0, 3),
    ("ragged_g2_d64", 2 * 2 * 100, 2, 4, 2, 64, 0, 1, 1),
]


def _setup(name, S, R, hq, hkv, d, window, rank, step):
    """One backward step's problem and inputs, the final LSE/delta from the GPU
    forward ring, and the oracle's dK/dV (and dQ part) of that step."""
    from context_long_attention_amd import cpattn
    from context_long_attention_amd.ring import RankRing
    w = inputs.Workload(name, S, R, hq, hkv, d, backward=True, window=window)
    inp = RankInputs(w, rank, want_do=True)
    ring = RankRing(w, rank)
    o, lse, _ = ring.forward(inp.q, inp.kv_of_source)
    rows = w.local
    delta = torch.empty((w.hq, rows), device="cuda")
    cpattn.cp_attn_bwd_prep(inp.do, o, delta, rows, w.hq, w.dim)
    torch.cuda.synchronize()
    sched = ring.schedule()
    blocks = [inp.kv64[s] for s in sched]
    ro, rl, _ = oracle.rank_forward(inp.q64, inp.qpos, blocks, None, w.scale, window=window or None)
    k64, v64, kpos = inp.kv64[sched[step]]
    vis = oracle.visibility(inp.qpos, kpos, None, window or None)
    rdq, rdk, rdv = oracle.attention_backward_partial(inp.q64, k64, v64, inp.do64, rl,
                                                      oracle.delta_rows(inp.do64, ro), vis, w.scale)
    k, v = inp.kv_of_source(sched[step])
    return w, inp, ring.problem(step, sched[step]), k, v, lse, delta, (rdq, rdk, rdv)


def _outputs(w):
    rows = w.local
    dq = torch.zeros((rows, w.hq, w.dim), device="cuda")
    dk = torch.full((rows, w.hkv, w.dim), 7.0, device="cuda")
    dv = torch.full_like(dk, 7.0)
    return dq, dk, dv


def test_noalloc_matches_workspace_entry_point():
    from context_long_attention_amd import cpattn
    setups = [_setup(*c) for c in CASES]
    for split in (8, 2, 0, 1):
        for (w, inp, p, k, v, lse, delta, ref), case in zip(setups, CASES):
            note(f"no-alloc backward {case[0]} kv_split={split}")
            p.kv_split = split
            # the workspace entry point, with room for any split the library may choose
            ws = torch.full((cpattn.cp_bwd_workspace_size(p, 8) // 4,), float("nan"), device="cuda")
            want = _outputs(w)
            cpattn.cp_attn_bwd_step(p, inp.q, k, v, inp.do, lse, delta, *want, workspace=ws)
            got = _outputs(w)
            cpattn.cp_attn_bwd_step_noalloc(p, inp.q, k, v, inp.do, lse, delta, *got)
            torch.cuda.synchronize()
            for g, x, r, what in zip(got, want, ref, ("dQ", "dK", "dV")):
                assert torch.equal(g, x), f"{what} of {case[0]} differs from the workspace entry point (split {split})"
                assert_o_close(g.cpu().numpy(), r, f"{what} of {case[0]} (split {split})")


def test_noalloc_refuses_a_split_beyond_its_scratch():
    """Split 8 of 80 key blocks of 128 keys (D = 128) needs 7 x 80 x 128 KiB = 70 MiB
    of workspace, more than the 64 MiB scratch: refused, nothing launched."""
    from context_long_attention_amd import cpattn
    F, S_ = cpattn.CP_MASK_FULL, cpattn.CP_MASK_SKIP
    p = cpattn.make_problem(8, 8, 128, 0.1, 64, 1280, [(0, 5000, 64)], [(0, 0, 1280)], [[F, S_], [S_, S_]],
                            kv_split=8)
    assert cpattn.cp_bwd_workspace_size(p, 8) == 70 * (1 << 20)
    # straight through the C entry point with a dummy buffer: the refusal comes
    # before any pointer is used (the Python binding would refuse the dummy first)
    t = torch.empty(16, device="cuda")
    ptr = ctypes.c_void_p(t.data_ptr())
    st = cpattn.lib().cp_attn_bwd_step_noalloc(ctypes.byref(p), *([ptr] * 9),
                                               ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    assert st == cpattn.CP_ERR_INVALID_ARG
    assert "no-alloc" in cpattn.lib().cp_last_error().decode()
    p.kv_split = 4  # 3 x 80 x 128 KiB = 30 MiB fits
    assert cpattn.cp_bwd_workspace_size(p, 4) <= 64 * (1 << 20)
