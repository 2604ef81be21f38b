"""ctypes binding of libfa.so (include/fa.h). Argument marshalling only:
every step of the attention computation runs in the library's HIP kernels.

Two levels:

* ``fa_fwd`` / ``fa_bwd`` / ``fa_bwd_atomic`` / ``fa_bwd_noalloc`` / ``fa_fwd_varlen`` /
  ``fa_bwd_varlen`` / ``fa_bwd_workspace_bytes`` / ``fa_status_string`` /
  ``fa_last_error`` / ``fa_version`` mirror the C functions one to one
  (pointers and streams as Python ints);
* ``forward`` / ``backward`` / ``forward_varlen`` / ``backward_varlen`` take
  torch tensors on the GPU, allocate the outputs with torch, call the C
  functions on torch's current stream and raise ``FAError`` on a non-zero
  status.

There is no fallback: if the library is missing, loading it raises.
"""

from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "lib", "libfa.so")

FA_OK = 0
FA_ERR_INVALID_ARGUMENT = 1
FA_ERR_UNSUPPORTED = 2
FA_ERR_HIP = 3
FA_DTYPE_F32 = 0
FA_DTYPE_BF16 = 1
FA_PRECISION_BF16 = 0
FA_PRECISION_HILO = 1

_lib = None

_c_int = ctypes.c_int
_c_ptr = ctypes.c_void_p
_c_float = ctypes.c_float


class FAError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: {fa_status_string(status)}: {detail}")
        self.status = status


def load_library(path: str | None = None) -> ctypes.CDLL:
    """Load libfa.so once; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(
            f"{p} not found: build it with `python -m exact_tiled_attention_28_amd.build` "
            "(there is no fallback implementation)")
    lib = ctypes.CDLL(p)
    lib.fa_fwd.restype = _c_int
    lib.fa_fwd.argtypes = [_c_ptr] * 5 + [_c_int] * 6 + [_c_float] + [_c_int] * 3 + [_c_ptr]
    for fn in (lib.fa_bwd, lib.fa_bwd_atomic):
        fn.restype = _c_int
        fn.argtypes = [_c_ptr] * 10 + [_c_int] * 6 + [_c_float] + [_c_int] * 5 + [_c_ptr]
    if hasattr(lib, "fa_bwd_noalloc"):
        lib.fa_bwd_noalloc.restype = _c_int
        lib.fa_bwd_noalloc.argtypes = [_c_ptr] * 9 + [_c_int] * 6 + [_c_float] + [_c_int] * 5 + [_c_ptr]
    # (looked up only if present, so that an older build still loads for the
    # fixed-length calls; calling a missing function raises AttributeError)
    if hasattr(lib, "fa_fwd_varlen"):
        lib.fa_fwd_varlen.restype = _c_int
        lib.fa_fwd_varlen.argtypes = [_c_ptr] * 7 + [_c_int] * 8 + [_c_float] + [_c_int] * 3 + [_c_ptr]
    if hasattr(lib, "fa_bwd_varlen"):
        lib.fa_bwd_varlen.restype = _c_int
        lib.fa_bwd_varlen.argtypes = [_c_ptr] * 12 + [_c_int] * 8 + [_c_float] + [_c_int] * 5 + [_c_ptr]
    if hasattr(lib, "fa_fwd_persistent"):
        lib.fa_fwd_persistent.restype = _c_int
        lib.fa_fwd_persistent.argtypes = [_c_ptr] * 6 + [_c_int] * 6 + [_c_float] + [_c_int] * 3 + [_c_ptr]
        lib.fa_fwd_persistent_sched_bytes.restype = ctypes.c_size_t
        lib.fa_fwd_persistent_sched_bytes.argtypes = []
    if hasattr(lib, "fa_quantize_fp8"):
        lib.fa_quantize_fp8.restype = _c_int
        lib.fa_quantize_fp8.argtypes = [_c_ptr] * 4 + [_c_int] * 5 + [_c_ptr]
        lib.fa_fp8_scales_count.restype = ctypes.c_size_t
        lib.fa_fp8_scales_count.argtypes = [_c_int] * 3
        lib.fa_fwd_fp8.restype = _c_int
        lib.fa_fwd_fp8.argtypes = [_c_ptr] * 7 + [_c_int] * 6 + [_c_float] + [_c_int] * 2 + [_c_ptr]
    if hasattr(lib, "fa_quantize_vt_fp8"):
        lib.fa_quantize_vt_fp8.restype = _c_int
        lib.fa_quantize_vt_fp8.argtypes = [_c_ptr] * 3 + [_c_int] * 5 + [_c_ptr]
        lib.fa_fp8_vt_bytes.restype = ctypes.c_size_t
        lib.fa_fp8_vt_bytes.argtypes = [_c_int] * 4
        lib.fa_fwd_fp8_pv.restype = _c_int
        lib.fa_fwd_fp8_pv.argtypes = [_c_ptr] * 8 + [_c_int] * 6 + [_c_float] + [_c_int] * 2 + [_c_ptr]
    if hasattr(lib, "fa_fwd_fp8_quantize_q"):
        lib.fa_fwd_fp8_quantize_q.restype = _c_int
        lib.fa_fwd_fp8_quantize_q.argtypes = [_c_ptr] * 8 + [_c_int] * 6 + [_c_float] + [_c_int] * 2 + [_c_ptr]
    lib.fa_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.fa_bwd_workspace_bytes.argtypes = [_c_int] * 3
    lib.fa_status_string.restype = ctypes.c_char_p
    lib.fa_status_string.argtypes = [_c_int]
    lib.fa_last_error.restype = ctypes.c_char_p
    lib.fa_last_error.argtypes = []
    lib.fa_version.restype = _c_int
    lib.fa_version.argtypes = []
    _lib = lib
    return lib


# ---------------------------------------------------------------------------
# one-to-one wrappers of the C functions
# ---------------------------------------------------------------------------

def fa_fwd(q, k, v, o, lse, batch, n_q_heads, n_kv_heads, seqlen_q, seqlen_k, head_dim, scale, causal,
           in_dtype, out_dtype, stream) -> int:
    return load_library().fa_fwd(q, k, v, o, lse, batch, n_q_heads, n_kv_heads, seqlen_q, seqlen_k, head_dim,
                                 scale, causal, in_dtype, out_dtype, stream)


def fa_bwd(q, k, v, o, lse, dout, dq, dk, dv, workspace, batch, n_q_heads, n_kv_heads, seqlen_q, seqlen_k,
           head_dim, scale, causal, in_dtype, o_dtype, grad_dtype, precision, stream) -> int:
    return load_library().fa_bwd(q, k, v, o, lse, dout, dq, dk, dv, workspace, batch, n_q_heads, n_kv_heads,
                                 seqlen_q, seqlen_k, head_dim, scale, causal, in_dtype, o_dtype, grad_dtype,
                                 precision, stream)


def fa_bwd_atomic(q, k, v, o, lse, dout, dq, dk, dv, workspace, batch, n_q_heads, n_kv_heads, seqlen_q, seqlen_k,
                  head_dim, scale, causal, in_dtype, o_dtype, grad_dtype, precision, stream) -> int:
    return load_library().fa_bwd_atomic(q, k, v, o, lse, dout, dq, dk, dv, workspace, batch, n_q_heads, n_kv_heads,
                                        seqlen_q, seqlen_k, head_dim, scale, causal, in_dtype, o_dtype, grad_dtype,
                                        precision, stream)


def fa_bwd_noalloc(q, k, v, o, lse, dout, dq, dk, dv, batch, n_q_heads, n_kv_heads, seqlen_q, seqlen_k, head_dim,
                   scale, causal, in_dtype, o_dtype, grad_dtype, precision, stream) -> int:
    return load_library().fa_bwd_noalloc(q, k, v, o, lse, dout, dq, dk, dv, batch, n_q_heads, n_kv_heads, seqlen_q,
                                         seqlen_k, head_dim, scale, causal, in_dtype, o_dtype, grad_dtype, precision,
                                         stream)


def fa_fwd_varlen(q, k, v, o, lse, cu_q, cu_k, batch, max_seqlen_q, max_seqlen_k, total_q, total_k, n_q_heads,
                  n_kv_heads, head_dim, scale, causal, in_dtype, out_dtype, stream) -> int:
    return load_library().fa_fwd_varlen(q, k, v, o, lse, cu_q, cu_k, batch, max_seqlen_q, max_seqlen_k, total_q,
                                        total_k, n_q_heads, n_kv_heads, head_dim, scale, causal, in_dtype, out_dtype,
                                        stream)


def fa_bwd_varlen(q, k, v, o, lse, dout, dq, dk, dv, workspace, cu_q, cu_k, batch, max_seqlen_q, max_seqlen_k,
                  total_q, total_k, n_q_heads, n_kv_heads, head_dim, scale, causal, in_dtype, o_dtype, grad_dtype,
                  precision, stream) -> int:
    return load_library().fa_bwd_varlen(q, k, v, o, lse, dout, dq, dk, dv, workspace, cu_q, cu_k, batch,
                                        max_seqlen_q, max_seqlen_k, total_q, total_k, n_q_heads, n_kv_heads, head_dim,
                                        scale, causal, in_dtype, o_dtype, grad_dtype, precision, stream)


def fa_fwd_persistent(q, k, v, o, lse, sched, batch, n_q_heads, n_kv_heads, seqlen_q, seqlen_k, head_dim, scale,
                      causal, in_dtype, out_dtype, stream) -> int:
    return load_library().fa_fwd_persistent(q, k, v, o, lse, sched, batch, n_q_heads, n_kv_heads, seqlen_q, seqlen_k,
                                            head_dim, scale, causal, in_dtype, out_dtype, stream)


def fa_fwd_persistent_sched_bytes() -> int:
    return load_library().fa_fwd_persistent_sched_bytes()


def fa_quantize_fp8(x, codes, block_scales, signs, batch, n_heads, seqlen, head_dim, in_dtype, stream) -> int:
    return load_library().fa_quantize_fp8(x, codes, block_scales, signs, batch, n_heads, seqlen, head_dim, in_dtype,
                                          stream)


def fa_fp8_scales_count(batch, n_heads, seqlen) -> int:
    return load_library().fa_fp8_scales_count(batch, n_heads, seqlen)


def fa_fwd_fp8(q_codes, q_scales, k_codes, k_scales, v, o, lse, batch, n_q_heads, n_kv_heads, seqlen_q, seqlen_k,
               head_dim, scale, causal, out_dtype, stream) -> int:
    return load_library().fa_fwd_fp8(q_codes, q_scales, k_codes, k_scales, v, o, lse, batch, n_q_heads, n_kv_heads,
                                     seqlen_q, seqlen_k, head_dim, scale, causal, out_dtype, stream)


def fa_quantize_vt_fp8(v, vt_codes, block_scales, batch, n_heads, seqlen, head_dim, in_dtype, stream) -> int:
    return load_library().fa_quantize_vt_fp8(v, vt_codes, block_scales, batch, n_heads, seqlen, head_dim, in_dtype,
                                             stream)


def fa_fp8_vt_bytes(batch, n_heads, seqlen, head_dim) -> int:
    return load_library().fa_fp8_vt_bytes(batch, n_heads, seqlen, head_dim)


def fa_fwd_fp8_quantize_q(q, q_signs, k_codes, k_scales, v, v_scales, o, lse, batch, n_q_heads, n_kv_heads, seqlen_q,
                          seqlen_k, head_dim, scale, causal, out_dtype, stream) -> int:
    return load_library().fa_fwd_fp8_quantize_q(q, q_signs, k_codes, k_scales, v, v_scales, o, lse, batch, n_q_heads,
                                                n_kv_heads, seqlen_q, seqlen_k, head_dim, scale, causal, out_dtype,
                                                stream)


def fa_fwd_fp8_pv(q_codes, q_scales, k_codes, k_scales, vt_codes, v_scales, o, lse, batch, n_q_heads, n_kv_heads,
                  seqlen_q, seqlen_k, head_dim, scale, causal, out_dtype, stream) -> int:
    return load_library().fa_fwd_fp8_pv(q_codes, q_scales, k_codes, k_scales, vt_codes, v_scales, o, lse, batch,
                                        n_q_heads, n_kv_heads, seqlen_q, seqlen_k, head_dim, scale, causal, out_dtype,
                                        stream)


def fa_bwd_workspace_bytes(batch, n_q_heads, seqlen_q) -> int:
    return load_library().fa_bwd_workspace_bytes(batch, n_q_heads, seqlen_q)


def fa_status_string(status: int) -> str:
    return load_library().fa_status_string(status).decode()


def fa_last_error() -> str:
    return load_library().fa_last_error().decode()


def fa_version() -> int:
    return load_library().fa_version()


# ---------------------------------------------------------------------------
# torch-tensor convenience layer (allocation and marshalling only)
# ---------------------------------------------------------------------------

def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return FA_DTYPE_BF16
    if t.dtype == torch.float32:
        return FA_DTYPE_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _torch_dtype(code):
    import torch
    return torch.float32 if code == FA_DTYPE_F32 else torch.bfloat16


def _stream_handle(stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _check(rc, where):
    if rc != FA_OK:
        raise FAError(rc, where, fa_last_error())


def forward(q, k, v, scale, causal, out_dtype=None, o=None, lse=None, stream=None):
    """O, L = attention(q, k, v). q: [B,Hq,Nq,d]; k, v: [B,Hkv,Nk,d]
    (contiguous, bf16 or fp32, on the GPU). Returns (o, lse)."""
    import torch
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    oc = _dtype_code(q) if out_dtype is None else (FA_DTYPE_F32 if out_dtype == torch.float32 else FA_DTYPE_BF16)
    if o is None:
        o = torch.empty((B, Hq, Nq, d), dtype=_torch_dtype(oc), device=q.device)
    else:
        oc = _dtype_code(o)
    if lse is None:
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    for t in (q, k, v, o, lse):
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")
    rc = fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, Hq, Hkv, Nq, Nk, d,
                float(scale), int(bool(causal)), _dtype_code(q), oc, _stream_handle(stream))
    _check(rc, "fa_fwd")
    return o, lse


def backward(q, k, v, o, lse, do, scale, causal, grad_dtype=None, stream=None, atomic_dq=False, hilo=False):
    """dQ (fp32), dK, dV (grad_dtype, default the input dtype) and the
    workspace holding D. Returns (dq, dk, dv, dvec). atomic_dq selects
    fa_bwd_atomic instead of fa_bwd; hilo selects FA_PRECISION_HILO."""
    import torch
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    gc = _dtype_code(q) if grad_dtype is None else (FA_DTYPE_F32 if grad_dtype == torch.float32 else FA_DTYPE_BF16)
    dq = torch.empty((B, Hq, Nq, d), dtype=torch.float32, device=q.device)
    dk = torch.empty((B, Hkv, Nk, d), dtype=_torch_dtype(gc), device=q.device)
    dv = torch.empty((B, Hkv, Nk, d), dtype=_torch_dtype(gc), device=q.device)
    ws = torch.empty(max(1, fa_bwd_workspace_bytes(B, Hq, Nq) // 4), dtype=torch.float32, device=q.device)
    for t in (q, k, v, o, lse, do):
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")
    fn = fa_bwd_atomic if atomic_dq else fa_bwd
    rc = fn(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), do.data_ptr(),
            dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), ws.data_ptr(), B, Hq, Hkv, Nq, Nk, d, float(scale),
            int(bool(causal)), _dtype_code(q), _dtype_code(o), gc,
            FA_PRECISION_HILO if hilo else FA_PRECISION_BF16, _stream_handle(stream))
    _check(rc, fn.__name__)
    return dq, dk, dv, ws[:B * Hq * Nq].view(B, Hq, Nq)


def forward_varlen(q, k, v, cu_q, cu_k, max_seqlen_q, max_seqlen_k, scale, causal, out_dtype=None, stream=None):
    """Packed variable-length forward. q: [Hq, total_q, d]; k, v: [Hkv, total_k, d]
    (contiguous bf16 on the GPU); cu_q, cu_k: int32 device tensors of batch + 1
    offsets (pass the same tensor twice for causal). Returns (o, lse) with
    o [Hq, total_q, d] and lse [Hq, total_q]."""
    import torch
    Hq, total_q, d = q.shape
    Hkv, total_k = k.shape[0], k.shape[1]
    oc = _dtype_code(q) if out_dtype is None else (FA_DTYPE_F32 if out_dtype == torch.float32 else FA_DTYPE_BF16)
    o = torch.empty((Hq, total_q, d), dtype=_torch_dtype(oc), device=q.device)
    lse = torch.empty((Hq, total_q), dtype=torch.float32, device=q.device)
    for t in (q, k, v, cu_q, cu_k):
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")
    if cu_q.dtype != torch.int32 or cu_k.dtype != torch.int32:
        raise TypeError("cu_seqlens must be int32")
    rc = fa_fwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), cu_q.data_ptr(),
                       cu_k.data_ptr(), cu_q.numel() - 1, int(max_seqlen_q), int(max_seqlen_k), total_q, total_k, Hq,
                       Hkv, d, float(scale), int(bool(causal)), _dtype_code(q), oc, _stream_handle(stream))
    _check(rc, "fa_fwd_varlen")
    return o, lse


def backward_varlen(q, k, v, o, lse, do, cu_q, cu_k, max_seqlen_q, max_seqlen_k, scale, causal, grad_dtype=None,
                    stream=None, hilo=False):
    """Packed variable-length backward (layouts as in forward_varlen; hilo
    selects FA_PRECISION_HILO). Returns (dq fp32 [Hq, total_q, d], dk, dv
    [Hkv, total_k, d], D [Hq, total_q])."""
    import torch
    Hq, total_q, d = q.shape
    Hkv, total_k = k.shape[0], k.shape[1]
    gc = _dtype_code(q) if grad_dtype is None else (FA_DTYPE_F32 if grad_dtype == torch.float32 else FA_DTYPE_BF16)
    dq = torch.empty((Hq, total_q, d), dtype=torch.float32, device=q.device)
    dk = torch.empty((Hkv, total_k, d), dtype=_torch_dtype(gc), device=q.device)
    dv = torch.empty((Hkv, total_k, d), dtype=_torch_dtype(gc), device=q.device)
    ws = torch.empty(max(1, fa_bwd_workspace_bytes(1, Hq, total_q) // 4), dtype=torch.float32, device=q.device)
    for t in (q, k, v, o, lse, do, cu_q, cu_k):
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")
    rc = fa_bwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), do.data_ptr(),
                       dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), ws.data_ptr(), cu_q.data_ptr(), cu_k.data_ptr(),
                       cu_q.numel() - 1, int(max_seqlen_q), int(max_seqlen_k), total_q, total_k, Hq, Hkv, d,
                       float(scale), int(bool(causal)), _dtype_code(q), _dtype_code(o), gc,
                       FA_PRECISION_HILO if hilo else FA_PRECISION_BF16, _stream_handle(stream))
    _check(rc, "fa_bwd_varlen")
    return dq, dk, dv, ws[:Hq * total_q].view(Hq, total_q)


def quantize_fp8(x, signs=None, codes=None, scales=None, stream=None):
    """FP8 codes (uint8 [B,H,N,d]) and power-of-two block scales (fp32
    [B,H,ceil(N/64)]) of x [B,H,N,d] (contiguous bf16 on the GPU); signs is an
    int8 [d] tensor of +1/-1 (random-sign Hadamard transform) or None."""
    import torch
    B, H, N, d = x.shape
    if codes is None:
        codes = torch.empty((B, H, N, d), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((B, H, -(-N // 64)), dtype=torch.float32, device=x.device)
    for t in (x, codes, scales) + ((signs,) if signs is not None else ()):
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")
    if signs is not None and (signs.dtype != torch.int8 or signs.numel() != d):
        raise TypeError("signs must be an int8 tensor of head_dim entries")
    rc = fa_quantize_fp8(x.data_ptr(), codes.data_ptr(), scales.data_ptr(),
                         signs.data_ptr() if signs is not None else None, B, H, N, d, _dtype_code(x),
                         _stream_handle(stream))
    _check(rc, "fa_quantize_fp8")
    return codes, scales


def forward_fp8(q_codes, q_scales, k_codes, k_scales, v, scale, causal, out_dtype=None, o=None, lse=None,
                stream=None):
    """O, L of the FP8 forward from codes and block scales written by
    quantize_fp8 (same signs for Q and K); v [B,Hkv,Nk,d] bf16, d = 64 or 128."""
    import torch
    B, Hq, Nq, d = q_codes.shape
    Hkv, Nk = k_codes.shape[1], k_codes.shape[2]
    oc = FA_DTYPE_BF16 if out_dtype in (None, torch.bfloat16) else FA_DTYPE_F32
    if o is None:
        o = torch.empty((B, Hq, Nq, d), dtype=_torch_dtype(oc), device=q_codes.device)
    else:
        oc = _dtype_code(o)
    if lse is None:
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q_codes.device)
    for t in (q_codes, q_scales, k_codes, k_scales, v, o, lse):
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")
    rc = fa_fwd_fp8(q_codes.data_ptr(), q_scales.data_ptr(), k_codes.data_ptr(), k_scales.data_ptr(), v.data_ptr(),
                    o.data_ptr(), lse.data_ptr(), B, Hq, Hkv, Nq, Nk, d, float(scale), int(bool(causal)), oc,
                    _stream_handle(stream))
    _check(rc, "fa_fwd_fp8")
    return o, lse


def new_sched(device=None):
    """A zeroed work-queue counter array for forward_persistent."""
    import torch
    return torch.zeros(fa_fwd_persistent_sched_bytes() // 4, dtype=torch.int32, device=device or "cuda")


def forward_persistent(q, k, v, scale, causal, sched, out_dtype=None, o=None, lse=None, stream=None):
    """forward() on the persistent work-queue grid; sched from new_sched()."""
    import torch
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    oc = _dtype_code(q) if out_dtype is None else (FA_DTYPE_F32 if out_dtype == torch.float32 else FA_DTYPE_BF16)
    if o is None:
        o = torch.empty((B, Hq, Nq, d), dtype=_torch_dtype(oc), device=q.device)
    else:
        oc = _dtype_code(o)
    if lse is None:
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    for t in (q, k, v, o, lse, sched):
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")
    if sched.dtype != torch.int32 or sched.numel() * 4 < fa_fwd_persistent_sched_bytes():
        raise TypeError("sched must be an int32 tensor from new_sched()")
    rc = fa_fwd_persistent(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), sched.data_ptr(),
                           B, Hq, Hkv, Nq, Nk, d, float(scale), int(bool(causal)), _dtype_code(q), oc,
                           _stream_handle(stream))
    _check(rc, "fa_fwd_persistent")
    return o, lse


def quantize_vt_fp8(v, codes=None, scales=None, stream=None):
    """Transposed FP8 codes of V for forward_fp8_pv (uint8
    [B,H,ceil(N/64),d,64], see fa_quantize_vt_fp8 for the key order within a
    block) and the power-of-two block scales (fp32 [B,H,ceil(N/64)]) of
    v [B,H,N,d] (contiguous bf16 on the GPU)."""
    import torch
    B, H, N, d = v.shape
    nb = -(-N // 64)
    if codes is None:
        codes = torch.empty((B, H, nb, d, 64), dtype=torch.uint8, device=v.device)
    if scales is None:
        scales = torch.empty((B, H, nb), dtype=torch.float32, device=v.device)
    for t in (v, codes, scales):
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")
    if codes.numel() != fa_fp8_vt_bytes(B, H, N, d):
        raise ValueError("codes must hold fa_fp8_vt_bytes(B, H, N, d) bytes")
    rc = fa_quantize_vt_fp8(v.data_ptr(), codes.data_ptr(), scales.data_ptr(), B, H, N, d, _dtype_code(v),
                            _stream_handle(stream))
    _check(rc, "fa_quantize_vt_fp8")
    return codes, scales


def forward_fp8_pv(q_codes, q_scales, k_codes, k_scales, vt_codes, v_scales, scale, causal, out_dtype=None, o=None,
                   lse=None, stream=None):
    """O, L of the FP8 forward with P V in FP8 as well: Q, K codes and scales
    from quantize_fp8, V from quantize_vt_fp8."""
    import torch
    B, Hq, Nq, d = q_codes.shape
    Hkv, Nk = k_codes.shape[1], k_codes.shape[2]
    oc = FA_DTYPE_BF16 if out_dtype in (None, torch.bfloat16) else FA_DTYPE_F32
    if o is None:
        o = torch.empty((B, Hq, Nq, d), dtype=_torch_dtype(oc), device=q_codes.device)
    else:
        oc = _dtype_code(o)
    if lse is None:
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q_codes.device)
    for t in (q_codes, q_scales, k_codes, k_scales, vt_codes, v_scales, o, lse):
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")
    if vt_codes.numel() != fa_fp8_vt_bytes(B, Hkv, Nk, d):
        raise ValueError("vt_codes must hold fa_fp8_vt_bytes(B, Hkv, Nk, d) bytes")
    rc = fa_fwd_fp8_pv(q_codes.data_ptr(), q_scales.data_ptr(), k_codes.data_ptr(), k_scales.data_ptr(),
                       vt_codes.data_ptr(), v_scales.data_ptr(), o.data_ptr(), lse.data_ptr(), B, Hq, Hkv, Nq, Nk, d,
                       float(scale), int(bool(causal)), oc, _stream_handle(stream))
    _check(rc, "fa_fwd_fp8_pv")
    return o, lse


def forward_fp8_quantize_q(q, k_codes, k_scales, v, scale, causal, signs=None, v_scales=None, out_dtype=None, o=None,
                           lse=None, stream=None):
    """O, L of the FP8 forward with Q quantized inside the kernel: q is bf16
    [B,Hq,Nq,d], k_codes / k_scales from quantize_fp8 (with the same signs),
    v bf16 [B,Hkv,Nk,d] (v_scales None) or the transposed codes and scales of
    quantize_vt_fp8. Equal bit for bit to quantize_fp8(q, signs) followed by
    forward_fp8 / forward_fp8_pv."""
    import torch
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k_codes.shape[1], k_codes.shape[2]
    oc = FA_DTYPE_BF16 if out_dtype in (None, torch.bfloat16) else FA_DTYPE_F32
    if o is None:
        o = torch.empty((B, Hq, Nq, d), dtype=_torch_dtype(oc), device=q.device)
    else:
        oc = _dtype_code(o)
    if lse is None:
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    tensors = (q, k_codes, k_scales, v, o, lse) + tuple(t for t in (signs, v_scales) if t is not None)
    for t in tensors:
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")
    if v_scales is not None and v.numel() != fa_fp8_vt_bytes(B, Hkv, Nk, d):
        raise ValueError("the V codes must hold fa_fp8_vt_bytes(B, Hkv, Nk, d) bytes")
    rc = fa_fwd_fp8_quantize_q(q.data_ptr(), signs.data_ptr() if signs is not None else None, k_codes.data_ptr(),
                               k_scales.data_ptr(), v.data_ptr(), v_scales.data_ptr() if v_scales is not None else None,
                               o.data_ptr(), lse.data_ptr(), B, Hq, Hkv, Nq, Nk, d, float(scale), int(bool(causal)), oc,
                               _stream_handle(stream))
    _check(rc, "fa_fwd_fp8_quantize_q")
    return o, lse
