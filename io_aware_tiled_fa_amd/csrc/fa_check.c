/*
 * fa_check.c - host-side argument validation of fa_fwd (no HIP dependency).
 *
 * Compiled with the host C compiler so that it can be unit-tested and run
 * under a host sanitizer without a GPU.  fa_fwd calls fa_check_args first and
 * launches nothing unless it returns FA_OK.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include "fa.h"

#define FA_BLOCK_M 128 /* query rows per workgroup (must match the kernels) */

static int aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

/* Any finite scale, of either sign or zero, whose product with log2(e),
 * rounded to fp32 as the kernels fold it into their exponentials, is finite
 * (|scale| below about 2.36e38). */
static int scale_ok(float scale) {
  return isfinite(scale) && isfinite((float)((double)scale * 1.4426950408889634074));
}

int fa_check_args(const void* q, const void* k, const void* v, const void* o,
                  const float* lse, int64_t B, int64_t H, int64_t M, int64_t N,
                  int64_t D, float scale, int causal, int dtype) {
  if (dtype != FA_DTYPE_F32 && dtype != FA_DTYPE_F16 && dtype != FA_DTYPE_BF16)
    return FA_ERR_BAD_DTYPE;
  if (B < 0 || H < 0 || M < 0 || N < 0) return FA_ERR_BAD_SHAPE;
  if (causal != 0 && causal != 1) return FA_ERR_BAD_SHAPE;
  if (D < 1 || D > 128) return FA_ERR_UNSUPPORTED_D;
  if (!scale_ok(scale)) return FA_ERR_BAD_SCALE;
  if (B == 0 || H == 0 || M == 0) return FA_OK; /* nothing to compute */
  if (q == NULL || o == NULL || lse == NULL) return FA_ERR_NULL_PTR;
  if (N > 0 && (k == NULL || v == NULL)) return FA_ERR_NULL_PTR;
  if (!aligned(q, 16) || !aligned(o, 16) || !aligned(lse, 4)) return FA_ERR_MISALIGNED;
  if (N > 0 && (!aligned(k, 16) || !aligned(v, 16))) return FA_ERR_MISALIGNED;
  {
    /* Every product below is formed only once its factors are known to keep
     * it within int64 (M * D >= 2^31 is tested as M > (2^31 - 1) / D). */
    const int64_t lim = (int64_t)1 << 31;
    if (M > (lim - 1) / D || N > (lim - 1) / D) return FA_ERR_TOO_LARGE;
    if (B > lim / H) return FA_ERR_TOO_LARGE;
    const int64_t tiles = (M + FA_BLOCK_M - 1) / FA_BLOCK_M;
    if (B * H >= lim / tiles) return FA_ERR_TOO_LARGE;
  }
  return FA_OK;
}

int fa_bwd_check_args(const void* q, const void* k, const void* v, const void* o,
                      const float* lse, const void* dout, const void* dq, const void* dk,
                      const void* dv, const float* delta, int64_t B, int64_t H, int64_t M,
                      int64_t N, int64_t D, float scale, int causal, int dtype) {
  if (dtype != FA_DTYPE_F32 && dtype != FA_DTYPE_F16 && dtype != FA_DTYPE_BF16)
    return FA_ERR_BAD_DTYPE;
  if (B < 0 || H < 0 || M < 0 || N < 0) return FA_ERR_BAD_SHAPE;
  if (causal != 0 && causal != 1) return FA_ERR_BAD_SHAPE;
  if (D < 1 || D > 128) return FA_ERR_UNSUPPORTED_D;
  if (!scale_ok(scale)) return FA_ERR_BAD_SCALE;
  if (B == 0 || H == 0 || (M == 0 && N == 0)) return FA_OK; /* nothing to compute */
  if (M > 0 && (q == NULL || o == NULL || lse == NULL || dout == NULL || dq == NULL ||
                delta == NULL))
    return FA_ERR_NULL_PTR;
  if (N > 0 && (k == NULL || v == NULL || dk == NULL || dv == NULL)) return FA_ERR_NULL_PTR;
  if (M > 0 && (!aligned(q, 16) || !aligned(o, 16) || !aligned(dout, 16) || !aligned(dq, 16) ||
                !aligned(lse, 4) || !aligned(delta, 4)))
    return FA_ERR_MISALIGNED;
  if (N > 0 && (!aligned(k, 16) || !aligned(v, 16) || !aligned(dk, 16) || !aligned(dv, 16)))
    return FA_ERR_MISALIGNED;
  {
    const int64_t lim = (int64_t)1 << 31;
    if (M > (lim - 1) / D || N > (lim - 1) / D) return FA_ERR_TOO_LARGE;
    if (B > lim / H) return FA_ERR_TOO_LARGE;
    const int64_t qt = (M + FA_BLOCK_M - 1) / FA_BLOCK_M;
    const int64_t kt = (N + FA_BLOCK_M - 1) / FA_BLOCK_M;
    if (qt > 0 && B * H >= lim / qt) return FA_ERR_TOO_LARGE;
    if (kt > 0 && B * H >= lim / kt) return FA_ERR_TOO_LARGE;
  }
  return FA_OK;
}

int fa_splitkv_check_args(const void* q, const void* k, const void* v, const void* o,
                          const float* lse, int64_t B, int64_t H, int64_t M, int64_t N,
                          int64_t D, float scale, int causal, int dtype, int splits,
                          const void* workspace, int64_t workspace_bytes) {
  const int st = fa_check_args(q, k, v, o, lse, B, H, M, N, D, scale, causal, dtype);
  if (st != FA_OK) return st;
  if (splits < 1 || splits > FA_MAX_SPLITS) return FA_ERR_BAD_SHAPE;
  if (B == 0 || H == 0 || M == 0 || N == 0) return FA_OK; /* no chunk is computed */
  if (workspace == NULL || !aligned(workspace, 16)) return FA_ERR_WORKSPACE;
  {
    const int64_t rows = B * H * M;
    const int64_t lim = (int64_t)1 << 62;
    if (rows > lim / ((D + 1) * 4 * (int64_t)splits)) return FA_ERR_TOO_LARGE;
    if (workspace_bytes < rows * (D + 1) * 4 * (int64_t)splits) return FA_ERR_WORKSPACE;
  }
  return FA_OK;
}

const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "FA_OK";
    case FA_ERR_NULL_PTR: return "FA_ERR_NULL_PTR: a required pointer is NULL";
    case FA_ERR_BAD_SHAPE:
      return "FA_ERR_BAD_SHAPE: B, H, M, N must be >= 0, causal 0 or 1, and splits 1..FA_MAX_SPLITS";
    case FA_ERR_BAD_DTYPE: return "FA_ERR_BAD_DTYPE: dtype must be F32, F16 or BF16";
    case FA_ERR_UNSUPPORTED_D: return "FA_ERR_UNSUPPORTED_D: head dim must be in 1..128";
    case FA_ERR_BAD_SCALE:
      return "FA_ERR_BAD_SCALE: scale must be finite, with scale*log2(e) finite in fp32";
    case FA_ERR_MISALIGNED: return "FA_ERR_MISALIGNED: q/k/v/o need 16-byte, lse 4-byte alignment";
    case FA_ERR_TOO_LARGE: return "FA_ERR_TOO_LARGE: per-head extent or grid beyond 32-bit limits";
    case FA_ERR_HIP: return "FA_ERR_HIP: the HIP runtime reported an error";
    case FA_ERR_WORKSPACE:
      return "FA_ERR_WORKSPACE: workspace NULL, not 16-byte aligned, or smaller than required";
    case FA_ERR_SCRATCH_LIMIT:
      return "FA_ERR_SCRATCH_LIMIT: split-KV partials exceed the static scratch FA_NOALLOC_MAX_BYTES";
    default: return "unknown fa status";
  }
}

int fa_abi_version(void) { return 6; }
