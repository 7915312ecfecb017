/*
 * fa.h - C ABI of the MI355X (gfx950) FlashAttention library (libfa_fwd.so):
 * the forward pass and its gradients.
 *
 * The operation is exact scaled dot-product attention with one log-sum-exp per
 * query row, computed tile by tile with the online-softmax recurrence so that no
 * M x N score or probability matrix exists in memory:
 *
 *   S = scale * Q K^T,   P = row-softmax(S),   O = P V,   LSE_i = m_i + ln(sum_j exp(S_ij - m_i))
 *
 * Definition: "Module 08: FlashAttention and Memory-Efficient Kernels"
 * (backend-roadmap), sections "Where the time goes in standard attention",
 * "Tiling and the online softmax" and "The backward pass: recompute instead of
 * store" (the per-row L = m + log(l)); problem statement and shapes (Q is M x D,
 * K and V are N x D, O is M x D): "FlashAttention in Triton: A Tile-by-Tile
 * Walkthrough", section "First, what does attention actually do?"; the caller
 * pre-allocates the output the kernel writes into, as that page's launcher does.
 *
 * Causal masking is aligned to the bottom-right corner: key j is visible to
 * query i iff j <= i + (N - M) (the pages' lower-triangular mask when M == N).
 * A query row with no visible key (causal with M > N, or N == 0) gets O = 0 and
 * LSE = -inf.
 */
#ifndef FA_H
#define FA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of q, k, v and o.  lse is always fp32. */
typedef enum {
  FA_DTYPE_F32 = 0,  /* IEEE fp32 in and out; P stays fp32 for the PV product   */
  FA_DTYPE_F16 = 1,  /* IEEE half; fp32 accumulation, P rounded to half for PV  */
  FA_DTYPE_BF16 = 2  /* bfloat16; fp32 accumulation, P rounded to bf16 for PV   */
} fa_dtype_t;

typedef enum {
  FA_OK = 0,
  FA_ERR_NULL_PTR = 1,       /* a required pointer is NULL                               */
  FA_ERR_BAD_SHAPE = 2,      /* B, H, M or N negative, causal not 0/1, splits out of range */
  FA_ERR_BAD_DTYPE = 3,      /* dtype is not one of fa_dtype_t                            */
  FA_ERR_UNSUPPORTED_D = 4,  /* D outside 1..128                                          */
  FA_ERR_BAD_SCALE = 5,      /* scale not finite, or scale*log2(e) overflows fp32         */
  FA_ERR_MISALIGNED = 6,     /* q, k, v or o not 16-byte aligned, or lse not 4-byte       */
  FA_ERR_TOO_LARGE = 7,      /* a per-head extent or the grid exceeds the 32-bit limits   */
  FA_ERR_HIP = 8,            /* the HIP runtime reported an error at launch               */
  FA_ERR_WORKSPACE = 9,      /* fa_fwd_splitkv: workspace NULL, misaligned or too small   */
  FA_ERR_SCRATCH_LIMIT = 10  /* fa_fwd_splitkv_noalloc: partials exceed FA_NOALLOC_MAX_BYTES */
} fa_status_t;

/* Largest number of key chunks fa_fwd_splitkv accepts. */
#define FA_MAX_SPLITS 64

/*
 * fa_fwd - enqueue the attention forward pass on `stream`.
 *
 * Arguments (all pointers are DEVICE pointers owned by the caller; the library
 * allocates nothing, keeps no per-call state and never synchronises):
 *   q    [B, H, M, D]  contiguous row-major, element type `dtype`
 *   k    [B, H, N, D]  contiguous row-major, element type `dtype`
 *   v    [B, H, N, D]  contiguous row-major, element type `dtype`
 *   o    [B, H, M, D]  contiguous row-major, element type `dtype` (written)
 *   lse  [B, H, M]     contiguous fp32, natural-log units (written)
 *   scale              the multiplier of Q K^T (typically 1/sqrt(D)); any finite value
 *                      with |scale * log2(e)| finite in fp32 (|scale| < 2.36e38):
 *                      negative scales weight small scores up, and scale 0 gives
 *                      uniform weights over the visible keys (LSE = ln #visible)
 *   causal             0: every key visible; 1: bottom-right causal mask
 *   dtype              an fa_dtype_t value
 *   stream             a hipStream_t, or NULL for the default stream
 * o and lse must not overlap q, k or v.  Output rounding to f16/bf16 is
 * round-to-nearest-even.
 *
 * Returns FA_OK once the work is enqueued.  Every argument error is detected on
 * the host before any HIP call; then nothing is launched and o and lse are not
 * touched.  Empty problems (B, H or M zero) return FA_OK without a launch, and
 * pointers may then be NULL.  N == 0 is valid (k and v may be NULL): every row
 * is empty.  A device-side fault shows at the caller's next synchronisation.
 * Limits: 1 <= D <= 128; M*D and N*D below 2^31; B*H*ceil(M/128) below 2^31.
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int64_t B, int64_t H, int64_t M, int64_t N, int64_t D,
           float scale, int causal, int dtype, void* stream);

/*
 * fa_fwd_general - the same operation, arguments, ownership and errors as
 * fa_fwd, always executed by the general kernel (K/V tiles staged through
 * registers, any D in 1..128) instead of the direct-to-LDS fast path fa_fwd
 * picks for fp16/bf16 with D in {64, 96, 128} (and, zero-padded to the next
 * of those sizes, for the other multiples of 8 except 32).  Results agree
 * with fa_fwd within the accuracy stated for the dtype (the summation order
 * is the same, so they are usually bit-identical); it exists to cross-check
 * the two paths.
 */
int fa_fwd_general(const void* q, const void* k, const void* v, void* o, float* lse,
                   int64_t B, int64_t H, int64_t M, int64_t N, int64_t D,
                   float scale, int causal, int dtype, void* stream);

/*
 * fa_check_args - the host-side validation fa_fwd performs, with the same
 * arguments and return codes, and no HIP call (usable without a GPU).
 */
int fa_check_args(const void* q, const void* k, const void* v, const void* o,
                  const float* lse, int64_t B, int64_t H, int64_t M, int64_t N,
                  int64_t D, float scale, int causal, int dtype);

/*
 * fa_fwd_splitkv - the same operation and results as fa_fwd (O and LSE within
 * the same accuracy; the summation order differs), computed over key chunks:
 * the N keys are cut into at most `splits` chunks of whole 64-key tiles, one
 * launch computes the partial (O_g, LSE_g) of every chunk (normalised over the
 * chunk's keys, fp32) for every query tile, and a second merges them with the
 * concatenation algebra ("Module 08: FlashAttention and Memory-Efficient
 * Kernels", "Tiling and the online softmax": the softmax of a concatenation
 * follows from the maxima and sums of its pieces):
 *
 *   LSE = log sum_g exp(LSE_g),   O = sum_g exp(LSE_g - LSE) O_g.
 *
 * It exposes `splits` times more workgroups when B * H * ceil(M/128) alone
 * cannot fill the GPU (few heads, short query runs, long key runs) -- the
 * under-filled grid "FlashAttention in Triton" names in "What the H100 run
 * showed".  The causal mask is the global one (key j visible to row i iff
 * j <= i + N - M), whichever chunk holds the key.
 *
 * Arguments as fa_fwd, plus:
 *   splits           1 .. FA_MAX_SPLITS
 *   workspace        device memory owned by the caller, 16-byte aligned, at
 *                    least fa_splitkv_workspace_bytes(B, H, M, D, splits)
 *                    bytes (fp32 partials; contents on return unspecified)
 *   workspace_bytes  its size
 * Errors as fa_fwd, plus FA_ERR_BAD_SHAPE for `splits` out of range and
 * FA_ERR_WORKSPACE for a NULL, misaligned or too small workspace (not checked
 * when nothing is computed: B, H, M or N zero).  Calls that share a workspace
 * must be ordered (same stream or explicit dependencies).
 */
int fa_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                   int64_t B, int64_t H, int64_t M, int64_t N, int64_t D,
                   float scale, int causal, int dtype, int splits, void* workspace,
                   int64_t workspace_bytes, void* stream);

/*
 * fa_splitkv_workspace_bytes - bytes of workspace fa_fwd_splitkv needs for
 * these sizes: splits * B * H * M * (D + 1) * 4.  Returns -1 for negative
 * sizes, D outside 1..128, splits < 1, or a size beyond int64.
 */
int64_t fa_splitkv_workspace_bytes(int64_t B, int64_t H, int64_t M, int64_t D, int splits);

/* Size of the static device scratch behind fa_fwd_splitkv_noalloc (64 MiB). */
#define FA_NOALLOC_MAX_BYTES ((int64_t)64 << 20)

/*
 * fa_fwd_splitkv_noalloc - fa_fwd_splitkv for callers that cannot allocate
 * device memory or pass a workspace (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation).
 *
 * Arguments, results and errors as fa_fwd_splitkv without `workspace` and
 * `workspace_bytes`: the fp32 partials go to a file-scope device array of
 * FA_NOALLOC_MAX_BYTES bytes that each GPU the library runs on holds until the
 * process ends; its address is looked up once per device, on the first call
 * that runs there (with that device made current for the lookup).  The call
 * makes no hipMalloc, hipFree or other allocation.  A problem whose partials,
 * fa_splitkv_workspace_bytes(B, H, M, D, splits), exceed FA_NOALLOC_MAX_BYTES
 * returns FA_ERR_SCRATCH_LIMIT and launches nothing.  Every call on one GPU
 * shares that array and leaves its contents behind (nothing in it needs to
 * start at zero): calls that may overlap on one GPU, on different streams or
 * from different threads, race on it and must be ordered by the caller.
 */
int fa_fwd_splitkv_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                           int64_t B, int64_t H, int64_t M, int64_t N, int64_t D,
                           float scale, int causal, int dtype, int splits, void* stream);

/*
 * fa_splitkv_check_args - the host-side validation fa_fwd_splitkv performs,
 * with its arguments (no stream) and return codes, and no HIP call.
 */
int fa_splitkv_check_args(const void* q, const void* k, const void* v, const void* o,
                          const float* lse, int64_t B, int64_t H, int64_t M, int64_t N,
                          int64_t D, float scale, int causal, int dtype, int splits,
                          const void* workspace, int64_t workspace_bytes);

/*
 * fa_bwd - enqueue the gradients of fa_fwd's output o with respect to q, k, v.
 *
 * The backward pass by recomputation ("Module 08: FlashAttention and
 * Memory-Efficient Kernels", section "The backward pass: recompute instead of
 * store"): only o and lse are kept from the forward pass; every tile of P is
 * rebuilt on chip as exp(S - LSE) from q and k, and no M x N matrix is stored.
 * With dO = dout, the chain rule of the definition above (the pages give the
 * rebuild, not the gradient formulas):
 *
 *   dV = P^T dO,  dP = dO V^T,  Delta_i = sum_d dO_id O_id,
 *   dS = P * (dP - Delta),  dQ = scale dS K,  dK = scale dS^T Q.
 *
 * Arguments (all DEVICE pointers owned by the caller; the library allocates
 * nothing and never synchronises):
 *   q, k, v      as for fa_fwd (read)
 *   o, lse       fa_fwd's outputs for the same q, k, v, scale, causal (read)
 *   dout [B, H, M, D]  element type `dtype`: dLoss/dO (read)
 *   dq   [B, H, M, D], dk [B, H, N, D], dv [B, H, N, D]  element type `dtype` (written)
 *   delta [2, B, H, M] fp32 workspace (written; on return delta[0] holds
 *                      -Delta_i and delta[1] holds -LSE_i / |scale| (-LSE_i
 *                      for scale 0), 0 where LSE_i = -inf: per-row terms the
 *                      kernels fold into their accumulators)
 *   scale, causal, stream  as for fa_fwd
 *   dtype        FA_DTYPE_F32, FA_DTYPE_F16 or FA_DTYPE_BF16
 * P and dS are rounded to `dtype` for their matrix products (fp32 inputs keep
 * them in fp32); accumulation is fp32; Delta uses the o passed in.  Written buffers must not overlap each
 * other or any read buffer.
 *
 * Returns FA_OK once the work is enqueued.  Argument errors are detected on the
 * host before any HIP call; then nothing is launched and no output is touched.
 * B or H zero, or M and N both zero: FA_OK without a launch (pointers may be
 * NULL).  M == 0 (N > 0): dk and dv are written with zeros (q, o, lse, dout,
 * dq, delta may be NULL).  N == 0 (M > 0): dq is written with zeros (k, v, dk,
 * dv may be NULL).  Limits as fa_fwd, plus B*H*ceil(N/128) below 2^31.
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
           const void* dout, void* dq, void* dk, void* dv, float* delta,
           int64_t B, int64_t H, int64_t M, int64_t N, int64_t D,
           float scale, int causal, int dtype, void* stream);

/*
 * fa_bwd_check_args - the host-side validation fa_bwd performs, with the same
 * arguments (no stream) and return codes, and no HIP call.
 */
int fa_bwd_check_args(const void* q, const void* k, const void* v, const void* o,
                      const float* lse, const void* dout, const void* dq, const void* dk,
                      const void* dv, const float* delta, int64_t B, int64_t H, int64_t M,
                      int64_t N, int64_t D, float scale, int causal, int dtype);

/* fa_status_string - a static, human-readable name for a status code. */
const char* fa_status_string(int status);

/* fa_abi_version - the ABI revision of this header (currently 6: 3 added fa_bwd
 * and fa_fwd_splitkv; 4 doubled fa_bwd's workspace to [2, B, H, M]; 5 accepts
 * zero and negative scales; 6 added fa_fwd_splitkv_noalloc). */
int fa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
