// fa_args.h — host-side argument validation for the C ABI (plain C++, no HIP
// calls), so that every error is reported before anything is enqueued.
#pragma once

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <string>

#include "../../include/fa.h"

namespace fa {

struct Shape {
  int batch, n_q_heads, n_kv_heads, seqlen_q, seqlen_k, head_dim;
};

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline bool valid_dtype(int t) { return t == FA_DTYPE_F32 || t == FA_DTYPE_BF16; }

// Checks common to the forward and backward entry points. On failure, writes
// a message to `err` and returns the status code.
inline int check_shape(const Shape& s, float scale, int causal, std::string& err) {
  char buf[256];
  if (s.batch < 1 || s.n_q_heads < 1 || s.n_kv_heads < 1 || s.seqlen_q < 1 || s.seqlen_k < 1) {
    std::snprintf(buf, sizeof buf, "sizes must be >= 1 (batch=%d n_q_heads=%d n_kv_heads=%d seqlen_q=%d seqlen_k=%d)",
                  s.batch, s.n_q_heads, s.n_kv_heads, s.seqlen_q, s.seqlen_k);
    err = buf;
    return FA_ERR_INVALID_ARGUMENT;
  }
  if (s.n_q_heads % s.n_kv_heads != 0) {
    std::snprintf(buf, sizeof buf, "n_q_heads (%d) must be a multiple of n_kv_heads (%d)", s.n_q_heads, s.n_kv_heads);
    err = buf;
    return FA_ERR_INVALID_ARGUMENT;
  }
  if (causal != 0 && causal != 1) {
    err = "causal must be 0 or 1";
    return FA_ERR_INVALID_ARGUMENT;
  }
  if (!std::isfinite(scale)) {
    err = "scale must be finite";
    return FA_ERR_INVALID_ARGUMENT;
  }
  if (s.head_dim != 64 && s.head_dim != 128) {
    std::snprintf(buf, sizeof buf, "head_dim %d unsupported (64 or 128)", s.head_dim);
    err = buf;
    return FA_ERR_UNSUPPORTED;
  }
  if (causal && s.seqlen_q != s.seqlen_k) {
    std::snprintf(buf, sizeof buf, "causal attention needs seqlen_q == seqlen_k (got %d and %d)", s.seqlen_q, s.seqlen_k);
    err = buf;
    return FA_ERR_UNSUPPORTED;
  }
  // Element offsets inside one head use 32-bit arithmetic in the kernels; the
  // per-head base offset is 64-bit.
  if ((long long)s.seqlen_q * s.head_dim >= (1LL << 31) || (long long)s.seqlen_k * s.head_dim >= (1LL << 31)) {
    err = "seqlen * head_dim must be below 2^31";
    return FA_ERR_INVALID_ARGUMENT;
  }
  if ((long long)s.batch * s.n_q_heads >= (1LL << 31) / 1024) {
    err = "batch * n_q_heads too large";
    return FA_ERR_INVALID_ARGUMENT;
  }
  return FA_OK;
}

inline int check_ptr(const void* p, const char* name, std::string& err) {
  if (p == nullptr) {
    err = std::string(name) + " is NULL";
    return FA_ERR_INVALID_ARGUMENT;
  }
  if (!aligned16(p)) {
    err = std::string(name) + " is not 16-byte aligned";
    return FA_ERR_INVALID_ARGUMENT;
  }
  return FA_OK;
}

inline int check_fwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const Shape& s,
                     float scale, int causal, int in_dtype, int out_dtype, std::string& err) {
  int rc;
  if ((rc = check_ptr(q, "q", err)) || (rc = check_ptr(k, "k", err)) || (rc = check_ptr(v, "v", err)) ||
      (rc = check_ptr(o, "o", err)) || (rc = check_ptr(lse, "lse", err)))
    return rc;
  if (!valid_dtype(in_dtype) || !valid_dtype(out_dtype)) {
    err = "in_dtype and out_dtype must be FA_DTYPE_F32 or FA_DTYPE_BF16";
    return FA_ERR_INVALID_ARGUMENT;
  }
  return check_shape(s, scale, causal, err);
}

inline int check_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
                     const float* dq, const void* dk, const void* dv, const float* workspace, const Shape& s,
                     float scale, int causal, int in_dtype, int o_dtype, int grad_dtype, std::string& err,
                     bool need_workspace = true) {
  int rc;
  // (workspace == nullptr is accepted only by the caller that passes no
  // workspace at all, fa_bwd_noalloc, which checks the other pointers here
  // with need_workspace = false)
  if ((rc = check_ptr(q, "q", err)) || (rc = check_ptr(k, "k", err)) || (rc = check_ptr(v, "v", err)) ||
      (rc = check_ptr(o, "o", err)) || (rc = check_ptr(lse, "lse", err)) || (rc = check_ptr(dout, "dout", err)) ||
      (rc = check_ptr(dq, "dq", err)) || (rc = check_ptr(dk, "dk", err)) || (rc = check_ptr(dv, "dv", err)) ||
      (need_workspace && (rc = check_ptr(workspace, "workspace", err))))
    return rc;
  if (!valid_dtype(in_dtype) || !valid_dtype(o_dtype) || !valid_dtype(grad_dtype)) {
    err = "dtypes must be FA_DTYPE_F32 or FA_DTYPE_BF16";
    return FA_ERR_INVALID_ARGUMENT;
  }
  if ((rc = check_shape(s, scale, causal, err))) return rc;
  if (in_dtype != FA_DTYPE_BF16) {
    err = "the backward pass takes bf16 q, k, v, dout";
    return FA_ERR_UNSUPPORTED;
  }
  return FA_OK;
}

// The backward's precision argument (enum fa_precision); the atomic scheme
// takes FA_PRECISION_BF16 only.
inline int check_precision(int precision, bool atomic_dq, std::string& err) {
  if (precision != FA_PRECISION_BF16 && precision != FA_PRECISION_HILO) {
    err = "precision must be FA_PRECISION_BF16 or FA_PRECISION_HILO";
    return FA_ERR_INVALID_ARGUMENT;
  }
  if (atomic_dq && precision != FA_PRECISION_BF16) {
    err = "fa_bwd_atomic supports FA_PRECISION_BF16 only";
    return FA_ERR_UNSUPPORTED;
  }
  return FA_OK;
}

// Packed variable-length batch (fa_fwd_varlen / fa_bwd_varlen).
struct VarlenShape {
  int batch, max_seqlen_q, max_seqlen_k, total_q, total_k, n_q_heads, n_kv_heads, head_dim;
};

inline int check_varlen(const void* cu_q, const void* cu_k, const VarlenShape& s, float scale, int causal,
                        std::string& err) {
  char buf[256];
  if (cu_q == nullptr || cu_k == nullptr) {
    err = cu_q == nullptr ? "cu_seqlens_q is NULL" : "cu_seqlens_k is NULL";
    return FA_ERR_INVALID_ARGUMENT;
  }
  if ((reinterpret_cast<uintptr_t>(cu_q) & 3u) || (reinterpret_cast<uintptr_t>(cu_k) & 3u)) {
    err = "cu_seqlens_q / cu_seqlens_k must be 4-byte aligned";
    return FA_ERR_INVALID_ARGUMENT;
  }
  if (s.batch < 1 || s.n_q_heads < 1 || s.n_kv_heads < 1) {
    std::snprintf(buf, sizeof buf, "batch, n_q_heads and n_kv_heads must be >= 1 (got %d, %d, %d)", s.batch,
                  s.n_q_heads, s.n_kv_heads);
    err = buf;
    return FA_ERR_INVALID_ARGUMENT;
  }
  if (s.max_seqlen_q < 0 || s.max_seqlen_k < 0 || s.total_q < 0 || s.total_k < 0 || s.max_seqlen_q > s.total_q ||
      s.max_seqlen_k > s.total_k) {
    std::snprintf(buf, sizeof buf,
                  "need 0 <= max_seqlen <= total (got max_seqlen_q=%d total_q=%d max_seqlen_k=%d total_k=%d)",
                  s.max_seqlen_q, s.total_q, s.max_seqlen_k, s.total_k);
    err = buf;
    return FA_ERR_INVALID_ARGUMENT;
  }
  if (s.n_q_heads % s.n_kv_heads != 0) {
    std::snprintf(buf, sizeof buf, "n_q_heads (%d) must be a multiple of n_kv_heads (%d)", s.n_q_heads, s.n_kv_heads);
    err = buf;
    return FA_ERR_INVALID_ARGUMENT;
  }
  if (causal != 0 && causal != 1) {
    err = "causal must be 0 or 1";
    return FA_ERR_INVALID_ARGUMENT;
  }
  if (!std::isfinite(scale)) {
    err = "scale must be finite";
    return FA_ERR_INVALID_ARGUMENT;
  }
  if (s.head_dim != 64 && s.head_dim != 128) {
    std::snprintf(buf, sizeof buf, "head_dim %d unsupported (64 or 128)", s.head_dim);
    err = buf;
    return FA_ERR_UNSUPPORTED;
  }
  if (causal && (cu_q != cu_k || s.max_seqlen_q != s.max_seqlen_k || s.total_q != s.total_k)) {
    err = "causal attention needs the same sequences for queries and keys (cu_seqlens_q == cu_seqlens_k, equal "
          "max_seqlen and total)";
    return FA_ERR_UNSUPPORTED;
  }
  if ((long long)s.total_q * s.head_dim >= (1LL << 31) || (long long)s.total_k * s.head_dim >= (1LL << 31)) {
    err = "total * head_dim must be below 2^31";
    return FA_ERR_INVALID_ARGUMENT;
  }
  if ((long long)s.batch * s.n_q_heads >= (1LL << 31) / 1024) {
    err = "batch * n_q_heads too large";
    return FA_ERR_INVALID_ARGUMENT;
  }
  return FA_OK;
}

}  // namespace fa
