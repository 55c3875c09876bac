"""The host logic of libcpattn (host.cpp: validation, partition, ring order, chunk
classes, block map, pair counts, dK/dV split and workspace sizes) built with
g++ under AddressSanitizer and UndefinedBehaviorSanitizer, every finding fatal,
and driven over a fixed battery of shapes and argument errors and over
hypothesis-generated problems, valid and corrupted; its results must equal the
regular (hipcc) build's on every problem.  CPU only."""
import ctypes
import os
import shutil
import subprocess

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from context_long_attention_amd import cpattn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "context_long_attention_amd", "csrc")


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    out = str(tmp_path_factory.mktemp("sanitized") / "host_driver")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           "-I", "/opt/rocm/include", os.path.join(CSRC, "host.cpp"),
           os.path.join(ROOT, "tests", "host_sanitize_driver.cpp"), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return out


def _run(driver, lines):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([driver], input="".join(l + "\n" for l in lines), capture_output=True, text=True, env=env,
                       timeout=120)
    assert r.returncode == 0 and "runtime error" not in r.stderr and "Sanitizer" not in r.stderr, r.stderr[-4000:]
    return r.stdout.splitlines()


def test_battery_is_clean(driver):
    assert _run(driver, []) == []


@st.composite
def _problem(draw):
    """Fields of one problem in the default line format: mostly valid problems of
    every mask class (segments at arbitrary positions, documents, windows, splits),
    some with one field corrupted."""
    hq, hkv = draw(st.sampled_from([(8, 2), (4, 4), (6, 2), (16, 1), (32, 8)]))
    d = draw(st.sampled_from([64, 128]))
    span = 700

    def segs():
        out, row = [], 0
        for _ in range(draw(st.integers(1, 2))):
            ln = draw(st.integers(0, 300))
            out.append([row, draw(st.integers(0, span)), ln])
            row += ln
        return out, row

    qs, q_rows = segs()
    ks, kv_rows = segs()
    masks = [draw(st.integers(0, 3)) for _ in range(4)]
    docs = draw(st.booleans()) or 2 in masks
    cu = [0] + sorted(set(draw(st.lists(st.integers(1, span + 300), max_size=8)))) + [span + 301] if docs else []
    window = draw(st.sampled_from([0, 0, 1, 17, 64, 150, 1000]))
    split = draw(st.integers(0, 8))
    f = dict(hq=hq, hkv=hkv, d=d, q_rows=max(q_rows, 1), kv_rows=max(kv_rows, 1), qs=qs, ks=ks, masks=masks,
             window=window, split=split, cu=cu)
    bad = draw(st.sampled_from([None] * 6 + ["hq", "d", "rows", "seglen", "mask", "nseg", "window", "split", "cu",
                                             "cu_short", "pos"]))
    if bad == "hq":
        f["hq"] = f["hkv"] + 1 if f["hkv"] > 1 else 0
    elif bad == "d":
        f["d"] = draw(st.sampled_from([0, 96, 256]))
    elif bad == "rows":
        f["q_rows"] = draw(st.sampled_from([-1, 0, 1 << 31]))
    elif bad == "seglen":
        f["ks"][0][2] = draw(st.sampled_from([-5, f["kv_rows"] + 1]))
    elif bad == "mask":
        f["masks"][0] = draw(st.sampled_from([-1, 4, 99]))
    elif bad == "nseg":
        f["nq"] = draw(st.sampled_from([0, 3]))
    elif bad == "window":
        f["window"] = -draw(st.integers(1, 5))
    elif bad == "split":
        f["split"] = draw(st.sampled_from([-1, 9]))
    elif bad == "cu" and cu:
        f["cu"] = cu[::-1]
    elif bad == "cu_short" and cu:
        f["cu"] = cu[:-1] + [1]
    elif bad == "pos":
        f["qs"][0][1] = draw(st.sampled_from([-1, (1 << 31) - 10]))
    return f


def _line(f):
    nq = f.get("nq", len(f["qs"]))
    parts = [f["hq"], f["hkv"], f["d"], f["q_rows"], f["kv_rows"], nq]
    for s in f["qs"][:max(0, min(nq, 2))]:
        parts += s
    parts.append(len(f["ks"]))
    for s in f["ks"]:
        parts += s
    parts += f["masks"] + [f["window"], f["split"], len(f["cu"]) - 1 if f["cu"] else 0] + list(f["cu"])
    return " ".join(str(int(x)) for x in parts)


def _fnv(b: bytes) -> int:
    """FNV-1a of the map bytes, as the driver computes it."""
    h = 1469598103934665603
    for x in b:
        h = ((h ^ x) * 1099511628211) & 0xFFFFFFFFFFFFFFFF
    return h


def _expected(f, cu_keep):
    """The regular build's results on the same problem, in the driver's format."""
    lib = cpattn.lib()
    p = cpattn.cp_attn_problem()
    p.hq, p.hkv, p.head_dim, p.scale = f["hq"], f["hkv"], f["d"], 0.125
    p.q_rows, p.kv_rows = f["q_rows"], f["kv_rows"]
    nq = f.get("nq", len(f["qs"]))
    p.n_q_seg, p.n_kv_seg = nq, len(f["ks"])
    for i, s in enumerate(f["qs"][:max(0, min(nq, 2))]):
        p.q_seg[i] = cpattn.cp_segment(*s)
    for j, s in enumerate(f["ks"]):
        p.kv_seg[j] = cpattn.cp_segment(*s)
    for i in range(2):
        for j in range(2):
            p.mask[i][j] = f["masks"][2 * i + j]
    if f["cu"]:
        arr = np.asarray(f["cu"], dtype=np.int32)
        cu_keep.append(arr)
        p.cu_seqlens, p.n_docs = arr.ctypes.data, len(arr) - 1
    p.window, p.kv_split = f["window"], f["split"]
    a, b = ctypes.c_int64(-1), ctypes.c_int64(-1)
    st_ = lib.cp_block_map_size(ctypes.byref(p), ctypes.byref(a), ctypes.byref(b))
    st_map, h = -100, 0
    if st_ == 0:
        m = np.zeros(a.value * b.value, dtype=np.uint8)
        st_map = lib.cp_block_map(ctypes.byref(p), m.ctypes.data_as(ctypes.c_void_p))
        if st_map == 0:
            h = _fnv(m.tobytes())
    pairs = ctypes.c_int64(-1)
    st_pairs = lib.cp_count_pairs(ctypes.byref(p), ctypes.byref(pairs))
    out = [st_, a.value, b.value, st_map, h, st_pairs, pairs.value]
    for n_cu in (1, 8, 64, 256):
        sp = ctypes.c_int32(-1)
        out.append(sp.value if lib.cp_bwd_kv_split(ctypes.byref(p), n_cu, ctypes.byref(sp)) == 0 else -1)
    for s in range(1, 9):
        by = ctypes.c_int64(-1)
        out.append(by.value if lib.cp_bwd_workspace_size(ctypes.byref(p), s, ctypes.byref(by)) == 0 else -1)
    return " ".join(str(x) for x in out)


@settings(max_examples=12, deadline=None)
@given(st.lists(_problem(), min_size=40, max_size=40))
def test_sanitized_build_matches_on_generated_problems(driver, problems):
    got = _run(driver, [_line(f) for f in problems])
    keep = []
    want = [_expected(f, keep) for f in problems]
    assert len(got) == len(want)
    for g, w_, f in zip(got, want, problems):
        assert g == w_, f"problem {_line(f)}: sanitized build {g} != regular build {w_}"
