"""Thin ctypes binding of libcpattn.so (the C ABI declared in include/cpattn.h).

Argument marshalling only: every step of the path runs in the library.  The
same names as the C functions; device tensors are passed as torch tensors (their
``data_ptr()``), streams as torch streams (default: torch's current stream).
A missing library raises: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
# CPATTN_LIB may name another build of the same library (same ABI), e.g. a debug build.
LIB_PATH = os.environ.get("CPATTN_LIB") or os.path.join(_PKG, "libcpattn.so")

CP_OK, CP_ERR_INVALID_ARG, CP_ERR_UNSUPPORTED, CP_ERR_HIP = 0, -1, -2, -3
CP_MASK_FULL, CP_MASK_DIAG_CAUSAL, CP_MASK_DOC, CP_MASK_SKIP = 0, 1, 2, 3
CP_TILE_SKIP, CP_TILE_PARTIAL, CP_TILE_FULL = 0, 1, 2

# Every symbol include/*.h declares (cpattn.h, and cpattn_diag.h for the clock probe).
EXPORTS = (
    "cp_abi_version", "cp_status_string", "cp_last_error", "cp_partition_zigzag", "cp_ring_source",
    "cp_step_masks", "cp_step_masks_window", "cp_tile_shape", "cp_block_map_size", "cp_block_map",
    "cp_count_pairs", "cp_bwd_kv_split", "cp_bwd_workspace_size", "cp_merge_partials_n", "cp_attn_fwd_step",
    "cp_merge_partials", "cp_attn_fwd_step_merge", "cp_attn_bwd_prep", "cp_attn_bwd_step",
    "cp_attn_bwd_step_noalloc", "cp_debug_clock_probe",
)


class CpError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"cpattn status {status}: {msg}")
        self.status = status


class cp_segment(ctypes.Structure):
    _fields_ = [("row0", ctypes.c_int64), ("pos0", ctypes.c_int64), ("len", ctypes.c_int64)]


class cp_attn_problem(ctypes.Structure):
    _fields_ = [
        ("hq", ctypes.c_int32), ("hkv", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("q_rows", ctypes.c_int64), ("kv_rows", ctypes.c_int64),
        ("n_q_seg", ctypes.c_int32), ("n_kv_seg", ctypes.c_int32),
        ("q_seg", cp_segment * 2), ("kv_seg", cp_segment * 2),
        ("mask", (ctypes.c_int32 * 2) * 2),
        ("cu_seqlens", ctypes.c_void_p), ("n_docs", ctypes.c_int32),
        ("window", ctypes.c_int32),
        ("kv_split", ctypes.c_int32),
    ]


_lib = None


def lib():
    """Open libcpattn.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise FileNotFoundError(
                f"{LIB_PATH} is missing: build it with `python -m context_long_attention_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        i32, i64, vp, f32p = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p
        P = ctypes.POINTER(cp_attn_problem)
        sig = {
            "cp_abi_version": ([], i32),
            "cp_status_string": ([i32], ctypes.c_char_p),
            "cp_last_error": ([], ctypes.c_char_p),
            "cp_partition_zigzag": ([i64, i32, i32, vp], i32),
            "cp_ring_source": ([i32, i32, i32, vp], i32),
            "cp_step_masks": ([i32, i32, i32, i32, vp], i32),
            "cp_step_masks_window": ([i64, i32, i32, i32, i32, i64, vp], i32),
            "cp_tile_shape": ([i32, i32, i32, vp, vp], i32),
            "cp_block_map_size": ([P, vp, vp], i32),
            "cp_block_map": ([P, vp], i32),
            "cp_count_pairs": ([P, vp], i32),
            "cp_bwd_kv_split": ([P, i32, vp], i32),
            "cp_bwd_workspace_size": ([P, i32, vp], i32),
            "cp_attn_fwd_step": ([P, vp, vp, vp, f32p, f32p, vp, vp], i32),
            "cp_merge_partials": ([f32p, f32p, f32p, f32p, i64, i32, i32, vp], i32),
            "cp_merge_partials_n": ([f32p, f32p, vp, vp, i32, i64, i32, i32, vp], i32),
            "cp_attn_fwd_step_merge": ([P, vp, vp, vp, f32p, f32p, vp, vp], i32),
            "cp_debug_clock_probe": ([vp, i64], i32),
            "cp_attn_bwd_prep": ([vp, f32p, f32p, i64, i32, i32, vp], i32),
            "cp_attn_bwd_step": ([P, vp, vp, vp, vp, f32p, f32p, f32p, f32p, f32p, vp, i64, vp], i32),
            "cp_attn_bwd_step_noalloc": ([P, vp, vp, vp, vp, f32p, f32p, f32p, f32p, f32p, vp], i32),
        }
        for name, (args, res) in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def _check(status: int):
    if status != CP_OK:
        raise CpError(status, lib().cp_last_error().decode())


def _ptr(t):
    """Device address of a torch tensor (None -> NULL).  The C ABI takes dense
    row-major buffers, so a strided view (a transpose, a column slice) is refused
    rather than passed on as if it were one."""
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError(f"tensor of shape {tuple(t.shape)} and strides {tuple(t.stride())} is not contiguous; "
                         "the C ABI takes dense row-major buffers")
    return ctypes.c_void_p(t.data_ptr())


def _dev(t, elem_bytes, n_elems, what):
    """Address of a device buffer that must hold at least ``n_elems`` elements of
    ``elem_bytes`` bytes (the layout the C ABI reads or writes for this call).
    The ABI receives bare pointers and cannot see sizes, so a tensor that is too
    small, of the wrong element size or not on the GPU is refused here rather
    than read or written out of bounds.  None passes through as NULL."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{what}: a device (GPU) tensor is required")
    if t.element_size() != elem_bytes:
        raise ValueError(f"{what}: {elem_bytes}-byte elements expected, got {t.element_size()}-byte {t.dtype}")
    if t.numel() < n_elems:
        raise ValueError(f"{what}: needs at least {n_elems} elements, got {t.numel()} (shape {tuple(t.shape)})")
    return _ptr(t)


def _stream(stream):
    if stream is None:
        import torch
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


# ------------------------------------------------------------------ host calls
def cp_abi_version() -> int:
    return lib().cp_abi_version()


def cp_status_string(status: int) -> str:
    return lib().cp_status_string(status).decode()


def cp_partition_zigzag(seq_len: int, cp_size: int, rank: int) -> np.ndarray:
    out = np.empty(max(seq_len // max(cp_size, 1), 0), dtype=np.int64)
    _check(lib().cp_partition_zigzag(seq_len, cp_size, rank, out.ctypes.data_as(ctypes.c_void_p)))
    return out


def cp_ring_source(cp_size: int, rank: int, step: int) -> int:
    out = ctypes.c_int32()
    _check(lib().cp_ring_source(cp_size, rank, step, ctypes.byref(out)))
    return out.value


def cp_step_masks(cp_size: int, rank: int, step: int, packed: bool) -> list[list[int]]:
    out = (ctypes.c_int32 * 4)()
    _check(lib().cp_step_masks(cp_size, rank, step, int(bool(packed)), out))
    return [[out[0], out[1]], [out[2], out[3]]]


def cp_step_masks_window(seq_len: int, cp_size: int, rank: int, step: int, packed: bool,
                         window: int) -> list[list[int]]:
    out = (ctypes.c_int32 * 4)()
    _check(lib().cp_step_masks_window(seq_len, cp_size, rank, step, int(bool(packed)), window, out))
    return [[out[0], out[1]], [out[2], out[3]]]


def cp_tile_shape(hq: int, hkv: int, head_dim: int) -> tuple[int, int]:
    bm, bn = ctypes.c_int32(), ctypes.c_int32()
    _check(lib().cp_tile_shape(hq, hkv, head_dim, ctypes.byref(bm), ctypes.byref(bn)))
    return bm.value, bn.value


def make_problem(hq, hkv, head_dim, scale, q_rows, kv_rows, q_segments, kv_segments, masks,
                 cu_seqlens_ptr=None, n_docs=0, window=0, kv_split=0) -> cp_attn_problem:
    """Fill a cp_attn_problem.  Segments are (row0, pos0, len) triples; window is
    the sliding window in tokens (0: none); kv_split the backward's dK/dV work
    split (0: chosen by the library)."""
    p = cp_attn_problem()
    p.hq, p.hkv, p.head_dim, p.scale = hq, hkv, head_dim, scale
    p.q_rows, p.kv_rows = q_rows, kv_rows
    p.n_q_seg, p.n_kv_seg = len(q_segments), len(kv_segments)
    for i, (r0, p0, n) in enumerate(q_segments):
        p.q_seg[i] = cp_segment(r0, p0, n)
    for j, (r0, p0, n) in enumerate(kv_segments):
        p.kv_seg[j] = cp_segment(r0, p0, n)
    for i in range(2):
        for j in range(2):
            p.mask[i][j] = masks[i][j] if (i < len(q_segments) and j < len(kv_segments)) else CP_MASK_SKIP
    p.cu_seqlens = cu_seqlens_ptr
    p.n_docs = n_docs
    p.window = window
    p.kv_split = kv_split
    return p


def cp_block_map_size(p: cp_attn_problem) -> tuple[int, int]:
    a, b = ctypes.c_int64(), ctypes.c_int64()
    _check(lib().cp_block_map_size(ctypes.byref(p), ctypes.byref(a), ctypes.byref(b)))
    return a.value, b.value


def cp_block_map(p: cp_attn_problem) -> np.ndarray:
    """Host block map; p.cu_seqlens must point to host memory here."""
    nq, nk = cp_block_map_size(p)
    out = np.zeros((nq, nk), dtype=np.uint8)
    _check(lib().cp_block_map(ctypes.byref(p), out.ctypes.data_as(ctypes.c_void_p)))
    return out


def cp_bwd_kv_split(p: cp_attn_problem, n_cu: int) -> int:
    """dK/dV work split for p (HOST cu_seqlens) on a GPU with n_cu CUs."""
    out = ctypes.c_int32()
    _check(lib().cp_bwd_kv_split(ctypes.byref(p), n_cu, ctypes.byref(out)))
    return out.value


def cp_bwd_workspace_size(p: cp_attn_problem, kv_split: int) -> int:
    """Workspace bytes cp_attn_bwd_step needs for the dK/dV split kv_split."""
    out = ctypes.c_int64()
    _check(lib().cp_bwd_workspace_size(ctypes.byref(p), kv_split, ctypes.byref(out)))
    return out.value


def cp_count_pairs(p: cp_attn_problem) -> int:
    out = ctypes.c_int64()
    _check(lib().cp_count_pairs(ctypes.byref(p), ctypes.byref(out)))
    return out.value


# ---------------------------------------------------------------- device calls
def _fwd_args(p, q, k, v, o, lse, tile_map):
    nq, nk = p.q_rows * p.hq * p.head_dim, p.kv_rows * p.hkv * p.head_dim
    tm = None
    if tile_map is not None:
        a, b = cp_block_map_size(p)
        tm = _dev(tile_map, 1, a * b, "tile_map")
    return (_dev(q, 2, nq, "q"), _dev(k, 2, nk, "k"), _dev(v, 2, nk, "v"), _dev(o, 4, nq, "o"),
            _dev(lse, 4, p.hq * p.q_rows, "lse"), tm)


def cp_attn_fwd_step(p: cp_attn_problem, q, k, v, o_step, lse_step, tile_map=None, stream=None):
    _check(lib().cp_attn_fwd_step(ctypes.byref(p), *_fwd_args(p, q, k, v, o_step, lse_step, tile_map),
                                  _stream(stream)))


def cp_merge_partials(o_acc, lse_acc, o_step, lse_step, rows, heads, head_dim, stream=None):
    no, nl = rows * heads * head_dim, heads * rows
    _check(lib().cp_merge_partials(_dev(o_acc, 4, no, "o_acc"), _dev(lse_acc, 4, nl, "lse_acc"),
                                   _dev(o_step, 4, no, "o_step"), _dev(lse_step, 4, nl, "lse_step"), rows, heads,
                                   head_dim, _stream(stream)))


def cp_merge_partials_n(o_out, lse_out, o_parts, lse_parts, rows, heads, head_dim, stream=None):
    """Merge the partials in the lists o_parts / lse_parts (same rows, disjoint keys) into o_out / lse_out."""
    n = len(o_parts)
    if len(lse_parts) != n:
        raise ValueError("o_parts and lse_parts differ in length")
    no, nl = rows * heads * head_dim, heads * rows
    op = (ctypes.c_void_p * max(n, 1))(*[_dev(t, 4, no, f"o_parts[{i}]") for i, t in enumerate(o_parts)])
    lp = (ctypes.c_void_p * max(n, 1))(*[_dev(t, 4, nl, f"lse_parts[{i}]") for i, t in enumerate(lse_parts)])
    _check(lib().cp_merge_partials_n(_dev(o_out, 4, no, "o_out"), _dev(lse_out, 4, nl, "lse_out"), op, lp, n, rows,
                                     heads, head_dim, _stream(stream)))


def cp_attn_fwd_step_merge(p: cp_attn_problem, q, k, v, o_acc, lse_acc, tile_map=None, stream=None):
    _check(lib().cp_attn_fwd_step_merge(ctypes.byref(p), *_fwd_args(p, q, k, v, o_acc, lse_acc, tile_map),
                                        _stream(stream)))


def cp_debug_clock_probe(buf=None):
    """Record per-workgroup (cycles, 100 MHz ticks) at start and end of every forward
    step launch into ``buf`` (device int64 tensor, 4 values per workgroup); None stops."""
    _check(lib().cp_debug_clock_probe(_dev(buf, 8, 0, "buf"), 0 if buf is None else buf.numel()))


def cp_attn_bwd_prep(d_o, o, delta, rows, heads, head_dim, stream=None):
    n = rows * heads * head_dim
    _check(lib().cp_attn_bwd_prep(_dev(d_o, 2, n, "d_o"), _dev(o, 4, n, "o"), _dev(delta, 4, heads * rows, "delta"),
                                  rows, heads, head_dim, _stream(stream)))


def _bwd_args(p, q, k, v, d_o, lse, delta, dq, dk, dv):
    nq, nk, nl = p.q_rows * p.hq * p.head_dim, p.kv_rows * p.hkv * p.head_dim, p.hq * p.q_rows
    return (_dev(q, 2, nq, "q"), _dev(k, 2, nk, "k"), _dev(v, 2, nk, "v"), _dev(d_o, 2, nq, "d_o"),
            _dev(lse, 4, nl, "lse"), _dev(delta, 4, nl, "delta"), _dev(dq, 4, nq, "dq_acc"),
            _dev(dk, 4, nk, "dk_out"), _dev(dv, 4, nk, "dv_out"))


def cp_attn_bwd_step(p: cp_attn_problem, q, k, v, d_o, lse, delta, dq_acc, dk_out, dv_out, workspace=None,
                     stream=None):
    """workspace: a device tensor (any dtype) whose bytes serve the dK/dV split, or None."""
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    ws = None if workspace is None else _dev(workspace, workspace.element_size(), 0, "workspace")
    _check(lib().cp_attn_bwd_step(ctypes.byref(p), *_bwd_args(p, q, k, v, d_o, lse, delta, dq_acc, dk_out, dv_out),
                                  ws, ws_bytes, _stream(stream)))


def cp_attn_bwd_step_noalloc(p: cp_attn_problem, q, k, v, d_o, lse, delta, dq_acc, dk_out, dv_out, stream=None):
    """cp_attn_bwd_step with the library's fixed per-device scratch as the workspace."""
    _check(lib().cp_attn_bwd_step_noalloc(ctypes.byref(p),
                                          *_bwd_args(p, q, k, v, d_o, lse, delta, dq_acc, dk_out, dv_out),
                                          _stream(stream)))
