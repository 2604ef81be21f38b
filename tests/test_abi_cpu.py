"""CPU tests of the C-ABI library: it loads, exports every function that
include/fa.h declares, reports every argument error on the host before any
launch, and its tile bookkeeping header matches a brute-force mask. No test
here runs a kernel."""

import ctypes
import os
import re
import subprocess
import tempfile

import numpy as np
import pytest

from exact_tiled_attention_28_amd import binding
from exact_tiled_attention_28_amd import build as fa_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB_PATH):
        fa_build.build()
    return binding.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*[a-z_][\w\s\*]*?\b(fa_\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_abi():
    assert declared_functions() == sorted(
        ["fa_bwd", "fa_bwd_atomic", "fa_bwd_noalloc", "fa_bwd_varlen", "fa_bwd_workspace_bytes", "fa_fp8_scales_count",
         "fa_fp8_vt_bytes", "fa_fwd", "fa_fwd_fp8", "fa_fwd_fp8_pv", "fa_fwd_fp8_quantize_q", "fa_fwd_persistent", "fa_fwd_persistent_sched_bytes",
         "fa_fwd_varlen", "fa_last_error", "fa_quantize_fp8", "fa_quantize_vt_fp8", "fa_status_string", "fa_version"])


def test_library_exports_every_declared_function(lib):
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} not exported"
    out = subprocess.run(["nm", "-D", "--defined-only", binding.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (fa_\w+)", out))
    assert set(declared_functions()) <= exported


def test_header_compiles_as_c(tmp_path):
    src = tmp_path / "t.c"
    src.write_text('#include "fa.h"\nint main(void) { return fa_version() == 2 ? 0 : 1; }\n')
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-fsyntax-only", f"-I{os.path.join(ROOT, 'include')}",
                        str(src)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_misc_entry_points(lib):
    assert binding.fa_version() == 2
    assert binding.fa_status_string(0) == "FA_OK"
    assert binding.fa_status_string(1) == "FA_ERR_INVALID_ARGUMENT"
    assert binding.fa_status_string(2) == "FA_ERR_UNSUPPORTED"
    assert binding.fa_status_string(3) == "FA_ERR_HIP"
    assert binding.fa_status_string(99) == "FA_ERR_UNKNOWN"
    assert binding.fa_bwd_workspace_bytes(2, 3, 5) == 4 * 2 * 3 * 5
    assert binding.fa_bwd_workspace_bytes(0, 3, 5) == 0
    assert binding.fa_bwd_workspace_bytes(-1, 3, 5) == 0


# Fake, aligned, never-dereferenced "device" addresses: every call below fails
# validation before anything touches them.
P = 0x10000
MIS = 0x10008  # 8-byte aligned, not 16


def fwd(**kw):
    args = dict(q=P, k=P, v=P, o=P, lse=P, batch=1, n_q_heads=2, n_kv_heads=1, seqlen_q=16, seqlen_k=16,
                head_dim=64, scale=0.125, causal=0, in_dtype=1, out_dtype=1, stream=None)
    args.update(kw)
    return binding.fa_fwd(*args.values())


def bwd(**kw):
    args = dict(q=P, k=P, v=P, o=P, lse=P, dout=P, dq=P, dk=P, dv=P, ws=P, batch=1, n_q_heads=2, n_kv_heads=1,
                seqlen_q=16, seqlen_k=16, head_dim=64, scale=0.125, causal=0, in_dtype=1, o_dtype=1, grad_dtype=1,
                precision=0, stream=None)
    args.update(kw)
    return binding.fa_bwd(*args.values())


INVALID = binding.FA_ERR_INVALID_ARGUMENT
UNSUP = binding.FA_ERR_UNSUPPORTED


@pytest.mark.parametrize("kw,code,text", [
    (dict(q=0), INVALID, "q is NULL"),
    (dict(lse=0), INVALID, "lse is NULL"),
    (dict(v=MIS), INVALID, "v is not 16-byte aligned"),
    (dict(batch=0), INVALID, "sizes must be >= 1"),
    (dict(seqlen_k=-3), INVALID, "sizes must be >= 1"),
    (dict(n_q_heads=3, n_kv_heads=2), INVALID, "multiple of n_kv_heads"),
    (dict(causal=2), INVALID, "causal must be 0 or 1"),
    (dict(scale=float("nan")), INVALID, "scale must be finite"),
    (dict(scale=float("inf")), INVALID, "scale must be finite"),
    (dict(in_dtype=7), INVALID, "FA_DTYPE"),
    (dict(out_dtype=-1), INVALID, "FA_DTYPE"),
    (dict(head_dim=96), UNSUP, "head_dim 96 unsupported"),
    (dict(causal=1, seqlen_q=16, seqlen_k=17), UNSUP, "seqlen_q == seqlen_k"),
    (dict(seqlen_q=1 << 25, head_dim=128), INVALID, "below 2^31"),
])
def test_fwd_argument_errors(lib, kw, code, text):
    assert fwd(**kw) == code
    assert text in binding.fa_last_error()


@pytest.mark.parametrize("kw,code,text", [
    (dict(dout=0), INVALID, "dout is NULL"),
    (dict(ws=0), INVALID, "workspace is NULL"),
    (dict(dq=MIS), INVALID, "dq is not 16-byte aligned"),
    (dict(n_kv_heads=0), INVALID, "sizes must be >= 1"),
    (dict(grad_dtype=5), INVALID, "FA_DTYPE"),
    (dict(in_dtype=0), UNSUP, "bf16"),
    (dict(head_dim=32), UNSUP, "head_dim 32"),
    (dict(causal=1, seqlen_k=15), UNSUP, "seqlen_q == seqlen_k"),
    (dict(precision=2), INVALID, "FA_PRECISION"),
    (dict(precision=-1), INVALID, "FA_PRECISION"),
])
def test_bwd_argument_errors(lib, kw, code, text):
    assert bwd(**kw) == code
    assert text in binding.fa_last_error()
    args = dict(q=P, k=P, v=P, o=P, lse=P, dout=P, dq=P, dk=P, dv=P, ws=P, batch=1, n_q_heads=2, n_kv_heads=1,
                seqlen_q=16, seqlen_k=16, head_dim=64, scale=0.125, causal=0, in_dtype=1, o_dtype=1, grad_dtype=1,
                precision=0, stream=None)
    args.update(kw)
    assert binding.fa_bwd_atomic(*args.values()) == code
    assert text in binding.fa_last_error()


def bwd_noalloc(**kw):
    args = dict(q=P, k=P, v=P, o=P, lse=P, dout=P, dq=P, dk=P, dv=P, batch=1, n_q_heads=2, n_kv_heads=1,
                seqlen_q=16, seqlen_k=16, head_dim=64, scale=0.125, causal=0, in_dtype=1, o_dtype=1, grad_dtype=1,
                precision=0, stream=None)
    args.update(kw)
    return binding.fa_bwd_noalloc(*args.values())


@pytest.mark.parametrize("kw,code,text", [
    (dict(dq=0), INVALID, "dq is NULL"),
    (dict(dv=MIS), INVALID, "dv is not 16-byte aligned"),
    (dict(head_dim=96), UNSUP, "head_dim 96"),
    (dict(precision=3), INVALID, "FA_PRECISION"),
    # more rows than the static scratch holds: rejected before any device call
    (dict(n_q_heads=2, seqlen_q=(1 << 21) + 1, seqlen_k=16), INVALID, "exceeds its scratch"),
    (dict(batch=4, n_q_heads=8, n_kv_heads=8, seqlen_q=131073, seqlen_k=131073), INVALID, "exceeds its scratch"),
])
def test_bwd_noalloc_argument_errors(lib, kw, code, text):
    assert bwd_noalloc(**kw) == code
    assert text in binding.fa_last_error()


def test_bwd_noalloc_limit_matches_header():
    text = open(HEADER).read()
    assert re.search(r"#define FA_BWD_NOALLOC_MAX_ROWS 4194304\b", text)
    assert 4194304 == 1 << 22


def test_bwd_atomic_rejects_hilo(lib):
    args = dict(q=P, k=P, v=P, o=P, lse=P, dout=P, dq=P, dk=P, dv=P, ws=P, batch=1, n_q_heads=2, n_kv_heads=1,
                seqlen_q=16, seqlen_k=16, head_dim=64, scale=0.125, causal=0, in_dtype=1, o_dtype=1, grad_dtype=1,
                precision=binding.FA_PRECISION_HILO, stream=None)
    assert binding.fa_bwd_atomic(*args.values()) == UNSUP
    assert "FA_PRECISION_BF16 only" in binding.fa_last_error()


CU = 0x20000       # fake 4-byte-aligned offset arrays
CU2 = 0x20010
CU_MIS = 0x20002


def fwd_varlen(**kw):
    args = dict(q=P, k=P, v=P, o=P, lse=P, cu_q=CU, cu_k=CU, batch=2, max_q=16, max_k=16, total_q=20, total_k=20,
                n_q_heads=2, n_kv_heads=1, head_dim=64, scale=0.125, causal=0, in_dtype=1, out_dtype=1, stream=None)
    args.update(kw)
    return binding.fa_fwd_varlen(*args.values())


def bwd_varlen(**kw):
    args = dict(q=P, k=P, v=P, o=P, lse=P, dout=P, dq=P, dk=P, dv=P, ws=P, cu_q=CU, cu_k=CU, batch=2, max_q=16,
                max_k=16, total_q=20, total_k=20, n_q_heads=2, n_kv_heads=1, head_dim=64, scale=0.125, causal=0,
                in_dtype=1, o_dtype=1, grad_dtype=1, precision=0, stream=None)
    if "out_dtype" in kw:
        kw = dict(kw)
        kw["grad_dtype"] = kw.pop("out_dtype")
    args.update(kw)
    return binding.fa_bwd_varlen(*args.values())


@pytest.mark.parametrize("kw,code,text", [
    (dict(q=0), INVALID, "q is NULL"),
    (dict(cu_q=0), INVALID, "cu_seqlens_q is NULL"),
    (dict(cu_k=0), INVALID, "cu_seqlens_k is NULL"),
    (dict(cu_k=CU_MIS), INVALID, "4-byte aligned"),
    (dict(batch=0), INVALID, "must be >= 1"),
    (dict(max_q=-1), INVALID, "max_seqlen <= total"),
    (dict(max_k=21), INVALID, "max_seqlen <= total"),
    (dict(n_q_heads=3, n_kv_heads=2), INVALID, "multiple of n_kv_heads"),
    (dict(causal=3), INVALID, "causal must be 0 or 1"),
    (dict(scale=float("nan")), INVALID, "scale must be finite"),
    (dict(head_dim=80), UNSUP, "head_dim 80"),
    (dict(in_dtype=0), UNSUP, "bf16"),
    (dict(out_dtype=4), INVALID, "FA_DTYPE"),
    (dict(causal=1, cu_k=CU2), UNSUP, "same sequences"),
    (dict(causal=1, max_k=15), UNSUP, "same sequences"),
    (dict(total_q=1 << 25, max_q=16, head_dim=128), INVALID, "below 2^31"),
])
def test_varlen_argument_errors(lib, kw, code, text):
    assert fwd_varlen(**kw) == code
    assert text in binding.fa_last_error()
    assert bwd_varlen(**kw) == code
    assert text in binding.fa_last_error()


def test_varlen_backward_pointer_errors(lib):
    assert bwd_varlen(dout=0) == INVALID and "dout is NULL" in binding.fa_last_error()
    assert bwd_varlen(ws=0) == INVALID and "workspace is NULL" in binding.fa_last_error()
    assert bwd_varlen(dq=MIS) == INVALID and "dq is not 16-byte aligned" in binding.fa_last_error()


def test_varlen_without_query_rows_launches_nothing(lib):
    # max_seqlen_q == 0: nothing to compute; the call succeeds without a GPU
    # launch (the fake pointers are never touched).
    assert fwd_varlen(max_q=0, total_q=0) == 0


def fwd_persistent(**kw):
    args = dict(q=P, k=P, v=P, o=P, lse=P, sched=CU, batch=1, n_q_heads=2, n_kv_heads=1, seqlen_q=16, seqlen_k=16,
                head_dim=64, scale=0.125, causal=0, in_dtype=1, out_dtype=1, stream=None)
    args.update(kw)
    return binding.fa_fwd_persistent(*args.values())


@pytest.mark.parametrize("kw,code,text", [
    (dict(q=0), INVALID, "q is NULL"),
    (dict(o=MIS), INVALID, "o is not 16-byte aligned"),
    (dict(sched=0), INVALID, "sched is NULL"),
    (dict(sched=CU_MIS), INVALID, "sched is not 4-byte aligned"),
    (dict(batch=0), INVALID, "sizes must be >= 1"),
    (dict(n_q_heads=3, n_kv_heads=2), INVALID, "multiple of n_kv_heads"),
    (dict(causal=1, seqlen_k=17), UNSUP, "seqlen_q == seqlen_k"),
    (dict(in_dtype=0), UNSUP, "bf16"),
    (dict(out_dtype=5), INVALID, "FA_DTYPE"),
    (dict(head_dim=96), UNSUP, "head_dim 96"),
])
def test_fwd_persistent_argument_errors(lib, kw, code, text):
    assert fwd_persistent(**kw) == code
    assert text in binding.fa_last_error()


def test_fwd_persistent_sched_bytes(lib):
    assert binding.fa_fwd_persistent_sched_bytes() == 36


def quantize_fp8(**kw):
    args = dict(x=P, codes=P, scales=CU, signs=None, batch=1, n_heads=2, seqlen=100, head_dim=128, in_dtype=1,
                stream=None)
    args.update(kw)
    return binding.fa_quantize_fp8(*args.values())


def fwd_fp8(**kw):
    args = dict(q=P, qs=CU, k=P, ks=CU, v=P, o=P, lse=P, batch=1, n_q_heads=2, n_kv_heads=1, seqlen_q=16,
                seqlen_k=16, head_dim=128, scale=0.125, causal=0, out_dtype=1, stream=None)
    args.update(kw)
    return binding.fa_fwd_fp8(*args.values())


@pytest.mark.parametrize("kw,code,text", [
    (dict(x=0), INVALID, "x is NULL"),
    (dict(codes=MIS), INVALID, "codes is not 16-byte aligned"),
    (dict(scales=0), INVALID, "block_scales is NULL"),
    (dict(scales=CU_MIS), INVALID, "4-byte aligned"),
    (dict(seqlen=0), INVALID, "sizes must be >= 1"),
    (dict(in_dtype=3), INVALID, "FA_DTYPE"),
    (dict(in_dtype=0), UNSUP, "bf16"),
    (dict(head_dim=96), UNSUP, "head_dim 96"),
    (dict(seqlen=1 << 24), INVALID, "below 2^31"),
])
def test_quantize_fp8_argument_errors(lib, kw, code, text):
    assert quantize_fp8(**kw) == code
    assert text in binding.fa_last_error()


@pytest.mark.parametrize("kw,code,text", [
    (dict(q=0), INVALID, "q is NULL"),
    (dict(v=MIS), INVALID, "v is not 16-byte aligned"),
    (dict(qs=0), INVALID, "q_scales is NULL"),
    (dict(ks=0), INVALID, "k_scales is NULL"),
    (dict(ks=CU_MIS), INVALID, "4-byte aligned"),
    (dict(n_q_heads=3, n_kv_heads=2), INVALID, "multiple of n_kv_heads"),
    (dict(causal=1, seqlen_k=17), UNSUP, "seqlen_q == seqlen_k"),
    (dict(out_dtype=9), INVALID, "FA_DTYPE"),
    (dict(scale=float("inf")), INVALID, "scale must be finite"),
    (dict(head_dim=96), UNSUP, "head_dim 96"),
])
def test_fwd_fp8_argument_errors(lib, kw, code, text):
    assert fwd_fp8(**kw) == code
    assert text in binding.fa_last_error()


def quantize_vt_fp8(**kw):
    args = dict(v=P, codes=P, scales=CU, batch=1, n_heads=2, seqlen=100, head_dim=128, in_dtype=1, stream=None)
    args.update(kw)
    return binding.fa_quantize_vt_fp8(*args.values())


def fwd_fp8_pv(**kw):
    args = dict(q=P, qs=CU, k=P, ks=CU, vt=P, vs=CU, o=P, lse=P, batch=1, n_q_heads=2, n_kv_heads=1, seqlen_q=16,
                seqlen_k=16, head_dim=128, scale=0.125, causal=0, out_dtype=1, stream=None)
    args.update(kw)
    return binding.fa_fwd_fp8_pv(*args.values())


@pytest.mark.parametrize("kw,code,text", [
    (dict(v=0), INVALID, "v is NULL"),
    (dict(codes=MIS), INVALID, "vt_codes is not 16-byte aligned"),
    (dict(scales=0), INVALID, "block_scales is NULL"),
    (dict(scales=CU_MIS), INVALID, "4-byte aligned"),
    (dict(seqlen=0), INVALID, "sizes must be >= 1"),
    (dict(in_dtype=0), UNSUP, "bf16"),
    (dict(head_dim=96), UNSUP, "head_dim 96"),
    (dict(seqlen=1 << 24), INVALID, "below 2^31"),
])
def test_quantize_vt_fp8_argument_errors(lib, kw, code, text):
    assert quantize_vt_fp8(**kw) == code
    assert text in binding.fa_last_error()


@pytest.mark.parametrize("kw,code,text", [
    (dict(q=0), INVALID, "q is NULL"),
    (dict(vt=MIS), INVALID, "v is not 16-byte aligned"),
    (dict(qs=0), INVALID, "q_scales is NULL"),
    (dict(vs=0), INVALID, "v_scales is NULL"),
    (dict(vs=CU_MIS), INVALID, "4-byte aligned"),
    (dict(n_q_heads=3, n_kv_heads=2), INVALID, "multiple of n_kv_heads"),
    (dict(causal=1, seqlen_k=17), UNSUP, "seqlen_q == seqlen_k"),
    (dict(head_dim=96), UNSUP, "head_dim 96"),
])
def test_fwd_fp8_pv_argument_errors(lib, kw, code, text):
    assert fwd_fp8_pv(**kw) == code
    assert text in binding.fa_last_error()


def test_fp8_vt_bytes(lib):
    assert binding.fa_fp8_vt_bytes(2, 3, 64, 128) == 2 * 3 * 64 * 128
    assert binding.fa_fp8_vt_bytes(2, 3, 65, 64) == 2 * 3 * 128 * 64
    assert binding.fa_fp8_vt_bytes(1, 1, 1, 128) == 64 * 128
    assert binding.fa_fp8_vt_bytes(0, 3, 5, 64) == 0
    assert binding.fa_fp8_vt_bytes(1, 1, -5, 64) == 0


def test_fp8_scales_count(lib):
    assert binding.fa_fp8_scales_count(2, 3, 64) == 6
    assert binding.fa_fp8_scales_count(2, 3, 65) == 12
    assert binding.fa_fp8_scales_count(1, 1, 1) == 1
    assert binding.fa_fp8_scales_count(0, 3, 5) == 0
    assert binding.fa_fp8_scales_count(1, 1, -5) == 0


def test_errors_are_thread_local(lib):
    import threading
    assert fwd(q=0) == INVALID
    seen = {}

    def other():
        seen["before"] = binding.fa_last_error()
        fwd(head_dim=48)
        seen["after"] = binding.fa_last_error()

    t = threading.Thread(target=other)
    t.start()
    t.join()
    assert seen["before"] == ""
    assert "head_dim 48" in seen["after"]
    assert binding.fa_last_error() == "q is NULL"


TILE_PROBE = r"""
#include <cstdio>
#include "fa_tiles.h"
int main() {
  for (int q0 = 0; q0 < 40; q0 += 3)
    for (int nq = 1; nq <= 9; nq += 4)
      for (int k0 = 0; k0 < 40; k0 += 5)
        for (int nk = 1; nk <= 9; nk += 4)
          std::printf("%d %d %d %d %d\n", q0, nq, k0, nk, (int)fa::causal_tile_class(q0, nq, k0, nk));
  for (int n = 1; n <= 300; n += 7)
    for (int br = 16; br <= 128; br *= 2)
      for (int bc = 16; bc <= 128; bc *= 2)
        for (int q0 = 0; q0 < n; q0 += br)
          std::printf("K %d %d %d %d %d %d %d\n", n, br, bc, q0, fa::kv_tiles_for(q0, br, n, bc, true),
                      fa::kv_tiles_for(q0, br, n, bc, false), fa::first_q_tile_for(q0, br, true));
  for (int lo = -3; lo <= 12; ++lo)
    for (int hi = -3; hi <= 12; ++hi)
      for (int total = 0; total <= 9; total += 3)
        for (int mx = 0; mx <= 10; mx += 5) {
          fa::SeqSpan sp = fa::clamp_span(lo, hi, total, mx);
          std::printf("S %d %d %d %d %d %d\n", lo, hi, total, mx, sp.off, sp.len);
        }
  for (int units = 1; units <= 48; units += 1)
    for (int items = 1; items <= 9; items += 4)
      for (int L = 0; L < units * items; ++L) {
        fa::UnitItem u = fa::xcd_decode(L, units);
        std::printf("X %d %d %d %d %d\n", units, items, L, u.unit, u.item);
      }
  return 0;
}
"""


def test_tile_bookkeeping_matches_brute_force():
    with tempfile.TemporaryDirectory() as tmp:
        src = os.path.join(tmp, "probe.cpp")
        exe = os.path.join(tmp, "probe")
        open(src, "w").write(TILE_PROBE)
        r = subprocess.run(["g++", "-std=c++17", "-O1", f"-I{os.path.join(ROOT, 'exact_tiled_attention_28_amd', 'csrc')}",
                            src, "-o", exe], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
        lines = subprocess.run([exe], capture_output=True, text=True, check=True).stdout.splitlines()
    n_cls = n_trip = 0
    seen = {}
    for ln in lines:
        f = ln.split()
        if f[0] == "S":
            lo, hi, total, mx, off, ln = map(int, f[1:])
            # the span is inside [0, total], no longer than mx, and equals
            # [lo, hi) whenever that is a well-formed range of length <= mx
            assert 0 <= off <= total and 0 <= ln <= mx and off + ln <= total
            if 0 <= lo <= hi <= total and hi - lo <= mx:
                assert (off, ln) == (lo, hi - lo)
            continue
        if f[0] == "X":
            units, items, L, unit, item = map(int, f[1:])
            assert 0 <= unit < units and 0 <= item < items
            seen.setdefault((units, items), set()).add((unit, item))
            if units % 8 == 0:
                assert unit % 8 == L % 8, "a unit must stay on one XCD (L % 8)"
            continue
        if f[0] == "K":
            n, br, bc, q0, trips_c, trips_n, first = map(int, f[1:])
            rows = range(q0, min(n, q0 + br))
            # brute force: the last key any row of the tile may see (key <= row)
            last_c = max(rows)
            assert trips_c == (min(n, q0 + br) + bc - 1) // bc and trips_c * bc > last_c
            assert trips_n == (n + bc - 1) // bc
            # first Q tile of height br that sees key k0 = q0 (k0 is a multiple of br here)
            assert first == q0 // br
            n_trip += 1
            continue
        q0, nq, k0, nk, cls = map(int, f)
        vis = np.array([[c <= r for c in range(k0, k0 + nk)] for r in range(q0, q0 + nq)])
        expect = 0 if vis.all() else (2 if not vis.any() else 1)
        assert cls == expect, (q0, nq, k0, nk)
        n_cls += 1
    assert n_cls > 500 and n_trip > 500
    for (units, items), pairs in seen.items():
        assert len(pairs) == units * items, "xcd_decode must be a bijection"


def test_abi_under_host_sanitizers(tmp_path):
    """The C ABI (fa_api.cpp with fa_args.h) built by g++ with the address and
    undefined-behaviour sanitizers, the kernel launchers replaced by stubs
    (tests/host/launch_stubs.cpp), driven through valid and invalid calls at
    the edges of the 32-bit sizes (tests/host/abi_driver.cpp): it must run to
    the end with every expectation met and no sanitizer report."""
    import shutil
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = tmp_path / "abi_driver"
    csrc = os.path.join(ROOT, "exact_tiled_attention_28_amd", "csrc")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           f"-I{os.path.join(ROOT, 'include')}", f"-I{csrc}", os.path.join(csrc, "fa_api.cpp"),
           os.path.join(ROOT, "tests", "host", "launch_stubs.cpp"),
           os.path.join(ROOT, "tests", "host", "abi_driver.cpp"), "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1", UBSAN_OPTIONS="halt_on_error=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "abi driver ok" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr


def fwd_fp8_quantize_q(**kw):
    args = dict(q=P, signs=None, k=P, ks=CU, v=P, vs=None, o=P, lse=P, batch=1, n_q_heads=2, n_kv_heads=1,
                seqlen_q=16, seqlen_k=16, head_dim=128, scale=0.125, causal=0, out_dtype=1, stream=None)
    args.update(kw)
    return binding.fa_fwd_fp8_quantize_q(*args.values())


@pytest.mark.parametrize("kw,code,text", [
    (dict(q=0), INVALID, "q is NULL"),
    (dict(q=MIS), INVALID, "q is not 16-byte aligned"),
    (dict(v=MIS), INVALID, "v is not 16-byte aligned"),
    (dict(ks=0), INVALID, "k_scales is NULL"),
    (dict(ks=CU_MIS), INVALID, "4-byte aligned"),
    (dict(vs=CU_MIS), INVALID, "4-byte aligned"),
    (dict(n_q_heads=3, n_kv_heads=2), INVALID, "multiple of n_kv_heads"),
    (dict(causal=1, seqlen_k=17), UNSUP, "seqlen_q == seqlen_k"),
    (dict(out_dtype=9), INVALID, "FA_DTYPE"),
    (dict(scale=float("nan")), INVALID, "scale must be finite"),
    (dict(head_dim=96), UNSUP, "head_dim 96"),
])
def test_fwd_fp8_quantize_q_argument_errors(lib, kw, code, text):
    assert fwd_fp8_quantize_q(**kw) == code
    assert text in binding.fa_last_error()
