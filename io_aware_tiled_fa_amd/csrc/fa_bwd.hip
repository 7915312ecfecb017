// fa_bwd.hip - FlashAttention backward for CDNA4 (gfx950): kernels and the C-ABI entry.
//
// The backward pass by recomputation ("Module 08: FlashAttention and
// Memory-Efficient Kernels", section "The backward pass: recompute instead of
// store"): the forward pass keeps O and one number per query row, the
// log-sum-exp L; here every tile of P is rebuilt on chip as exp(S - L) from Q
// and K, and no M x N matrix exists in memory.  With dO the incoming gradient,
// the gradients are the chain rule of the attention definition (the pages give
// the rebuild, not the formulas):
//
//   dV = P^T dO,   dP = dO V^T,   Delta_i = sum_d dO_id O_id,
//   dS = P * (dP - Delta),   dQ = scale dS K,   dK = scale dS^T Q.
//
// Three kernels:
//  * delta: Delta per query row from O and dO (one pass, bandwidth-bound).
//  * dkdv:  one workgroup per (batch*head, 128-key tile); each wave owns 32 keys,
//           whose K and V rows stay in registers, and accumulates dK^T and dV^T
//           over 64-query tiles of Q and dO staged through LDS.  S = Q K^T and
//           dP = dO V^T read the Q and dO rows in a permuted order (bits 2 and 3
//           of the row index swapped) so that P and dS come out of the MFMA
//           already in the B-operand layout of dV^T += dO^T P and
//           dK^T += Q^T dS, whose A operands are transposing LDS reads
//           (ds_read_b64_tr_b16) of the row-major dO and Q tiles.
//  * dq:    one workgroup per (batch*head, 128-query tile), the forward's
//           shape: S^T = K Q^T and dP^T = V dO^T with permuted K and V rows, so
//           dS^T is the B operand of dQ^T += K^T dS^T (K^T by transposing reads).
// P and dS are rounded to the input type for their MFMAs; everything else
// accumulates in fp32.  The MFMA work is seven M x N x D products (dkdv
// recomputes S and dP beside dV and dK, dq recomputes them again) against the
// five of a backward pass with one recomputation; the two extra products buy a
// dQ with neither atomics nor an fp32 scratch copy.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "fa.h"
#include "fa_device.h"

namespace {

constexpr int BT = 256;          // threads per workgroup (4 waves)
constexpr int BK = 128;          // keys per dkdv workgroup
constexpr int BQ = 64;           // queries per dkdv step
constexpr int BMQ = 128;         // queries per dq workgroup
constexpr int BNK = 64;          // keys per dq step
constexpr float LOG2E = 1.44269504088896340736f;
#ifndef DKDV_NBUF
#define DKDV_NBUF 3  // query-tile buffers of the fast dK/dV kernel (copies run NBUF - 2 tiles ahead)
#endif
#ifndef DKDV_LA1
#define DKDV_LA1 4   // fast dK/dV: MFMAs whose row reads are issued ahead (stage 1)
#endif
#ifndef DKDV_LA2
#define DKDV_LA2 4   // fast dK/dV: MFMAs whose transposing reads are issued ahead (stage 2)
#endif

typedef float f32x4 __attribute__((ext_vector_type(4)));

// Per query row, into the two halves of the workspace:
//   ws[row]        = -Delta_i, Delta_i = sum_d dO[i, d] * O[i, d] in fp32;
//   ws[rows + row] = -L_i / s (0 where L_i = -inf: the row sees no key), s the
//   positive scale of the score product (|scale|, or 1 for scale 0: fold_scale).
// The fast dK/dV kernel loads them as the initial values of the dP and S
// accumulators, so that the MFMAs leave dP - Delta and S - L / scale, and
// P = exp2(c * acc) with c = scale * log2(e).  LPR lanes per row (4 at
// D <= 32, 8 at D <= 64, else 16), so that a row's 16-byte chunks keep every
// lane busy.
template <class T, int LPR>
__global__ __launch_bounds__(BT) void fa_bwd_delta_kernel(const typename T::elt* __restrict__ o,
                                                          const typename T::elt* __restrict__ dout,
                                                          const float* __restrict__ lse,
                                                          float* __restrict__ ws, int64_t rows,
                                                          int D, float scale) {
  using elt = typename T::elt;
  using vec8 = typename T::vec8;
  constexpr int RPB = BT / LPR;  // rows per block and pass
  const int sub = threadIdx.x / LPR;
  const int l16 = threadIdx.x % LPR;
  for (int64_t row0 = (int64_t)blockIdx.x * RPB; row0 < rows; row0 += (int64_t)gridDim.x * RPB) {
    const int64_t row = row0 + sub;
    float acc = 0.0f;
    if (row < rows) {
      const elt* orow = o + row * D;
      const elt* grow = dout + row * D;
      if ((D & 7) == 0) {
        for (int c8 = l16; 8 * c8 < D; c8 += LPR) {
          const vec8 a = __builtin_bit_cast(vec8, *reinterpret_cast<const u32x4*>(orow + 8 * c8));
          const vec8 b = __builtin_bit_cast(vec8, *reinterpret_cast<const u32x4*>(grow + 8 * c8));
#pragma unroll
          for (int e = 0; e < 8; ++e) acc = __builtin_fmaf((float)a[e], (float)b[e], acc);
        }
      } else {
        for (int d = l16; d < D; d += LPR) acc = __builtin_fmaf((float)orow[d], (float)grow[d], acc);
      }
    }
#pragma unroll
    for (int m = LPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, LPR);
    if (row < rows && l16 == 0) {
      ws[row] = -acc;
      const float x = lse[row];
      ws[rows + row] = x == -INFINITY ? 0.0f : -(x / scale);
    }
  }
}

// Eight features of row `row` starting at column d0 as an MFMA operand (zero
// outside [0, rows) x [0, D)).
template <class T, bool DFULL>
__device__ __forceinline__ typename T::vec8 load_row8(const typename T::elt* base, int row,
                                                      int rows, int D, int d0) {
  using elt = typename T::elt;
  using vec8 = typename T::vec8;
  if (DFULL) {
    u32x4 raw = {0u, 0u, 0u, 0u};
    if (row < rows) raw = *reinterpret_cast<const u32x4*>(base + (int64_t)row * D + d0);
    return __builtin_bit_cast(vec8, raw);
  }
  vec8 x;
#pragma unroll
  for (int e = 0; e < 8; ++e)
    x[e] = (row < rows && d0 + e < D) ? base[(int64_t)row * D + d0 + e] : (elt)0.0f;
  return x;
}

// Store 4 consecutive features (fp32 values times `mul`) of row `row` at column d0.
template <class T, bool DFULL>
__device__ __forceinline__ void store_row4(typename T::elt* base, int row, int D, int d0,
                                           const f32x16& acc, int g, float mul) {
  using elt = typename T::elt;
  elt y[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) y[e] = (elt)(acc[4 * g + e] * mul);
  if (DFULL) {
    *reinterpret_cast<u32x2*>(base + (int64_t)row * D + d0) = __builtin_bit_cast(u32x2, y);
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (d0 + e < D) base[(int64_t)row * D + d0 + e] = y[e];
  }
}

// The A operand of a transposed product from a row-major LDS tile with row
// stride STR (elements): lane l receives column (col0 + l % 32) of the 8 rows
// row0 + 8 * (l / 32) + e, e = 0..7 -- two transposing reads of 4 rows each.
// Lane j of each 16-lane group addresses row row0 + 8h + j/4 (and 4 further) at
// column col0 + 16 * ((l / 16) % 2) + 4 * (j % 4).
template <class T, int STR>
__device__ __forceinline__ typename T::vec8 load_tr8(const typename T::elt* tile, int row0,
                                                     int col0, int lane) {
  using vec8 = typename T::vec8;
  const int h = lane >> 5;
  const int j16 = lane & 15;
  const int row = row0 + 8 * h + (j16 >> 2);
  const int col = col0 + 16 * ((lane >> 4) & 1) + 4 * (j16 & 3);
  const auto* p = reinterpret_cast<const char*>(tile) + 2 * (row * STR + col);
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + 2 * 4 * STR));
  return __builtin_bit_cast(vec8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Register staging of ROWS x DP elements of a row-major [rows, D] matrix into
// an LDS tile with row stride DP + 8 (16-byte chunks, zero-filled outside).
template <class T, int DP, int ROWS, bool DFULL>
struct Stager {
  using elt = typename T::elt;
  static constexpr int STR = DP + 8;
  static constexpr int CH = DP / 8;
  static constexpr int LD = ROWS * CH / BT;
  static_assert(ROWS * CH % BT == 0, "staging plan");
  u32x4 r[LD];
  __device__ __forceinline__ void load(const elt* base, int row0, int rows, int D, int tid) {
#pragma unroll
    for (int i = 0; i < LD; ++i) {
      const int ci = tid + BT * i;
      const int row = ci / CH;
      const int col = (ci - row * CH) * 8;
      const int gr = row0 + row;
      if (DFULL) {
        u32x4 raw = {0u, 0u, 0u, 0u};
        if (gr < rows) raw = *reinterpret_cast<const u32x4*>(base + (int64_t)gr * D + col);
        r[i] = raw;
      } else {
        typename T::vec8 x;
#pragma unroll
        for (int e = 0; e < 8; ++e)
          x[e] = (gr < rows && col + e < D) ? base[(int64_t)gr * D + col + e] : (elt)0.0f;
        r[i] = __builtin_bit_cast(u32x4, x);
      }
    }
  }
  __device__ __forceinline__ void store(elt* tile, int tid) const {
#pragma unroll
    for (int i = 0; i < LD; ++i) {
      const int ci = tid + BT * i;
      const int row = ci / CH;
      const int col = (ci - row * CH) * 8;
      *reinterpret_cast<u32x4*>(tile + row * STR + col) = r[i];
    }
  }
};

// Rounds 16 fp32 values to two 8-element MFMA operands (values 8t..8t+7 -> t).
template <class T>
__device__ __forceinline__ void pack16(const f32x16& x, typename T::vec8 (&out)[2]) {
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    f32x8 f;
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = x[8 * t + e];
    out[t] = __builtin_convertvector(f, typename T::vec8);
  }
}

// ---------------------------------------------------------------------------
// dK and dV.  DP: head dim padded to a multiple of 32; DFULL: D == DP.
template <class T, int DP, bool CAUSAL, bool DFULL>
__global__ __launch_bounds__(BT, 1) void fa_bwd_dkdv_kernel(
    const typename T::elt* __restrict__ q, const typename T::elt* __restrict__ k,
    const typename T::elt* __restrict__ v, const typename T::elt* __restrict__ dout,
    const float* __restrict__ lse, const float* __restrict__ delta, typename T::elt* __restrict__ dk,
    typename T::elt* __restrict__ dv, int M, int N, int D, int ktiles, float c, float scale,
    QFold qf) {
  using elt = typename T::elt;
  using vec8 = typename T::vec8;
  using St = Stager<T, DP, BQ, DFULL>;
  constexpr int STR = St::STR;
  constexpr int TILE = BQ * STR;
  constexpr int KK = DP / 16;
  constexpr int DT = DP / 32;

  __shared__ __attribute__((aligned(16))) elt smem[2 * 2 * TILE];  // [stage][Q, dO]
  __shared__ __attribute__((aligned(16))) float stat[2][2][BQ];    // [stage][L*log2e, Delta]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int h = lane >> 5;
  const int l32 = lane & 31;

  // Key tiles in natural order: under the causal mask the first tiles see the
  // most queries, so the heaviest workgroups start first.
  const TileCoord tc = tile_coord<false, BK>(ktiles);
  const int k0 = tc.q0;
  const elt* Qh = q + (int64_t)tc.bh * M * D;
  const elt* Kh = k + (int64_t)tc.bh * N * D;
  const elt* Vh = v + (int64_t)tc.bh * N * D;
  const elt* Gh = dout + (int64_t)tc.bh * M * D;
  const float* Lh = lse + (int64_t)tc.bh * M;
  const float* Dh = delta + (int64_t)tc.bh * M;  // -Delta per row (the workspace's first half)
  elt* dKh = dk + (int64_t)tc.bh * N * D;
  elt* dVh = dv + (int64_t)tc.bh * N * D;

  const int off = N - M;  // causal: key j visible to query i iff j <= i + off
  const int kw0 = k0 + 32 * w;
  const int key = kw0 + l32;

  // K and V rows of this lane's key: B operands of S = Q K^T and dP = dO V^T.
  vec8 kb[KK], vb[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    kb[kk] = fold_vec(load_row8<T, DFULL>(Kh, key, N, D, 16 * kk + 8 * h), qf);
    vb[kk] = load_row8<T, DFULL>(Vh, key, N, D, 16 * kk + 8 * h);
  }
  f32x16 dka[DT], dva[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    dka[dt] = f32x16{};
    dva[dt] = f32x16{};
  }

  // Query tiles: under the causal mask, key k0 is first seen by query k0 - off.
  const int qstart = CAUSAL ? max(0, k0 - off) : 0;
  const int qt0 = qstart / BQ;
  const int nqt = (M + BQ - 1) / BQ;

  St sq, sg;
  float st_val = 0.0f;
  auto load_tile = [&](int q0) {
    sq.load(Qh, q0, M, D, tid);
    sg.load(Gh, q0, M, D, tid);
    if (tid < 2 * BQ) {
      const int r = q0 + (tid & (BQ - 1));
      // Rows past M (and rows with no visible key, LSE = -inf) are masked before
      // their statistics are used; keep them finite here.
      float x = 0.0f;
      if (r < M) x = tid < BQ ? Lh[r] * LOG2E : -Dh[r];
      st_val = (x == -INFINITY) ? 0.0f : x;
    }
  };
  auto store_tile = [&](int stage) {
    sq.store(smem + stage * 2 * TILE, tid);
    sg.store(smem + stage * 2 * TILE + TILE, tid);
    if (tid < 2 * BQ) stat[stage][tid >> 6][tid & (BQ - 1)] = st_val;
  };

  if (qt0 < nqt) {
    load_tile(qt0 * BQ);
    store_tile(0);
  }
  __syncthreads();

  for (int qt = qt0; qt < nqt; ++qt) {
    const int q0 = qt * BQ;
    const int stage = (qt - qt0) & 1;
    const bool more = qt + 1 < nqt;
    if (more) load_tile(q0 + BQ);
    const elt* Qs = smem + stage * 2 * TILE;
    const elt* Gs = Qs + TILE;
    const float* L2s = stat[stage][0];
    const float* Ds = stat[stage][1];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int qb = q0 + 32 * t;
      // Wave-uniform skip: no query of this half sees any key of this wave.
      if (kw0 >= N || (CAUSAL && qb + 31 + off < kw0) || qb >= M) continue;
      f32x16 s = f32x16{}, dp = f32x16{};
      const int arow = 32 * t + swap23(l32);
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const vec8 aq = *reinterpret_cast<const vec8*>(Qs + arow * STR + 16 * kk + 8 * h);
        const vec8 ag = *reinterpret_cast<const vec8*>(Gs + arow * STR + 16 * kk + 8 * h);
        s = T::mfma(aq, kb[kk], s);
        dp = T::mfma(ag, vb[kk], dp);
      }
      // Accumulator register r holds query qb + 16 (r >> 3) + 8h + (r & 7) of
      // this lane's key: two runs of 8 consecutive queries.
      const f32x4 la = *reinterpret_cast<const f32x4*>(L2s + 32 * t + 8 * h);
      const f32x4 lb = *reinterpret_cast<const f32x4*>(L2s + 32 * t + 8 * h + 4);
      const f32x4 lc = *reinterpret_cast<const f32x4*>(L2s + 32 * t + 16 + 8 * h);
      const f32x4 ld = *reinterpret_cast<const f32x4*>(L2s + 32 * t + 16 + 8 * h + 4);
      const f32x4 da = *reinterpret_cast<const f32x4*>(Ds + 32 * t + 8 * h);
      const f32x4 db = *reinterpret_cast<const f32x4*>(Ds + 32 * t + 8 * h + 4);
      const f32x4 dc = *reinterpret_cast<const f32x4*>(Ds + 32 * t + 16 + 8 * h);
      const f32x4 dd = *reinterpret_cast<const f32x4*>(Ds + 32 * t + 16 + 8 * h + 4);
      const float l2[16] = {la[0], la[1], la[2], la[3], lb[0], lb[1], lb[2], lb[3],
                            lc[0], lc[1], lc[2], lc[3], ld[0], ld[1], ld[2], ld[3]};
      const float dl[16] = {da[0], da[1], da[2], da[3], db[0], db[1], db[2], db[3],
                            dc[0], dc[1], dc[2], dc[3], dd[0], dd[1], dd[2], dd[3]};
      const bool need_mask = (qb + 31 >= M) || (kw0 + 31 >= N) || (CAUSAL && kw0 + 31 > qb + off);
      f32x16 p, ds;
#pragma unroll
      for (int r = 0; r < 16; ++r) p[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c, -l2[r]));
      if (need_mask) {  // rare: a real branch (P is pinned first so the selects stay in it);
        pin(p);         // rows with L = -inf have no visible key and are masked here
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int qi = qb + key_of_reg(r, h);
          const bool vis = qi < M && key < N && (!CAUSAL || key <= qi + off);
          p[r] = vis ? p[r] : 0.0f;
        }
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) ds[r] = p[r] * (dp[r] - dl[r]);
      vec8 pb[2], dsb[2];
      pack16<T>(p, pb);
      pack16<T>(ds, dsb);
      // dV^T += dO^T P and dK^T += Q^T dS over the 32 queries of this half.
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const vec8 ag = load_tr8<T, STR>(Gs, 32 * t + 16 * t2, 32 * dt, lane);
          dva[dt] = T::mfma(ag, pb[t2], dva[dt]);
          const vec8 aq = load_tr8<T, STR>(Qs, 32 * t + 16 * t2, 32 * dt, lane);
          dka[dt] = T::mfma(aq, dsb[t2], dka[dt]);
        }
      }
    }
    if (more) store_tile(stage ^ 1);
    __syncthreads();
  }

  // Accumulator register 4g + e of tile dt holds feature 32dt + 8g + 4h + e of
  // this lane's key.
  if (key < N) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * dt + 8 * g + 4 * h;
        store_row4<T, DFULL>(dVh, key, D, d0, dva[dt], g, 1.0f);
        store_row4<T, DFULL>(dKh, key, D, d0, dka[dt], g, scale);
      }
  }
}

// ---------------------------------------------------------------------------
// dK and dV on the fast path (fp16/bf16, D in {64, 96, 128}).
//
// The work split of fa_bwd_dkdv_kernel (4 waves of 32 keys, K and V rows in
// registers, dK^T and dV^T accumulated over 64-query tiles), with:
//  * Q, dO, L and Delta of a query tile copied HBM -> LDS directly
//    (global_load_lds) into one of NBUF rotating buffers, NBUF - 2 query tiles
//    ahead; the tiles use the forward's K-tile swizzle, which keeps both the
//    row reads and the transposing reads free of bank conflicts.
//  * A two-stage pipeline over 32-query halves u: while the MFMA unit computes
//    S and dP of half u+1, the VALU forms dS of half u and rounds P and dS to
//    16 bits; while it computes dV and dK of half u, the VALU exponentiates the
//    scores of half u+1.
//  * One barrier per query tile, between its two halves.  Waves do not skip
//    halves that none of their keys sees: such a half is computed and masked
//    to zero, which costs nothing since the wave would wait at the barrier.

// The direct-to-LDS copy through inline assembly.  The compiler does not track
// it, so it adds no conservative wait before LDS reads of other buffers; the
// kernel owns every s_waitcnt vmcnt and barrier that orders a copy against its
// readers.  M0 holds the LDS address of the copy (one wait state before the
// load reads it) and is restored afterwards.  Lane l writes bytes
// [4 l, 4 l + 4) after that address (lds_copy_tile below: the 16-byte form).
__device__ __forceinline__ void lds_copy4(const void* g, unsigned lds_addr) {
  unsigned saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(g), "s"(lds_addr)
      : "memory");
}

// The 2*NB direct-to-LDS copies of one query tile in one statement: for copy
// i, NB-row blocks of Q (base qb) and dO (base gb) at the lane's byte offset
// off[i] go to LDS addresses m0 + i*STRIDE and m0 + i*STRIDE + GOFF.  M0 is
// saved once, stepped between copies (one wait state after each write) and
// restored at the end.
template <int NB, int STRIDE, int GOFF>
__device__ __forceinline__ void lds_copy_tile(const void* qb, const void* gb, const unsigned (&off)[NB],
                                              unsigned m0) {
  unsigned saved;
  if constexpr (NB == 4) {
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\ts_nop 0\n\t"
        "global_load_lds_dwordx4 %4, %2\n\t"
        "s_add_u32 m0, m0, %8\n\ts_nop 0\n\t"
        "global_load_lds_dwordx4 %4, %3\n\t"
        "s_add_u32 m0, m0, %9\n\ts_nop 0\n\t"
        "global_load_lds_dwordx4 %5, %2\n\t"
        "s_add_u32 m0, m0, %8\n\ts_nop 0\n\t"
        "global_load_lds_dwordx4 %5, %3\n\t"
        "s_add_u32 m0, m0, %9\n\ts_nop 0\n\t"
        "global_load_lds_dwordx4 %6, %2\n\t"
        "s_add_u32 m0, m0, %8\n\ts_nop 0\n\t"
        "global_load_lds_dwordx4 %6, %3\n\t"
        "s_add_u32 m0, m0, %9\n\ts_nop 0\n\t"
        "global_load_lds_dwordx4 %7, %2\n\t"
        "s_add_u32 m0, m0, %8\n\ts_nop 0\n\t"
        "global_load_lds_dwordx4 %7, %3\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(m0), "s"(qb), "s"(gb), "v"(off[0]), "v"(off[1]), "v"(off[2]), "v"(off[3]),
          "i"(GOFF), "i"(STRIDE - GOFF)
        : "memory", "scc");
  } else {
    static_assert(NB == 2, "copies per wave");
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\ts_nop 0\n\t"
        "global_load_lds_dwordx4 %4, %2\n\t"
        "s_add_u32 m0, m0, %6\n\ts_nop 0\n\t"
        "global_load_lds_dwordx4 %4, %3\n\t"
        "s_add_u32 m0, m0, %7\n\ts_nop 0\n\t"
        "global_load_lds_dwordx4 %5, %2\n\t"
        "s_add_u32 m0, m0, %6\n\ts_nop 0\n\t"
        "global_load_lds_dwordx4 %5, %3\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(m0), "s"(qb), "s"(gb), "v"(off[0]), "v"(off[1]), "i"(GOFF), "i"(STRIDE - GOFF)
        : "memory", "scc");
  }
}

//
// PAD: the rows hold Drow < DP features, Drow a multiple of 8 (whole 16-byte
// chunks, 16-byte aligned rows).  Chunks at or past Drow are neither loaded nor
// copied: K's and V's are zero in registers, Q's and dO's stay zero in LDS
// (cleared once at the start), so they add nothing to S and dP and only fill
// gradient columns that are not stored.
template <class T, int DP, int NBUF, bool PAD>
__global__ __launch_bounds__(BT, 1) void fa_bwd_dkdv_fast_kernel(
    const typename T::elt* __restrict__ q, const typename T::elt* __restrict__ k,
    const typename T::elt* __restrict__ v, const typename T::elt* __restrict__ dout,
    const float* __restrict__ lse, const float* __restrict__ delta, typename T::elt* __restrict__ dk,
    typename T::elt* __restrict__ dv, int M, int N, int ktiles, int items, float c, float scale,
    int causal, QFold qf, int Drow) {
  // lse is unused here: `delta` points at the workspace [2, B*H*M], whose
  // second half holds -L / scale per row (see fa_bwd_delta_kernel).
  using elt = typename T::elt;
  using vec8 = typename T::vec8;
  using L = FastLayout<DP>;
  const int D = PAD ? Drow : DP;  // features per row in HBM
  constexpr int KK = DP / 16;
  constexpr int DT = DP / 32;
  constexpr int NW = BT / 64;
  constexpr int BPW = L::NBLK / NW;  // 1 KB copies per wave per 64-row tile
  constexpr int TB = L::TILEB;       // bytes of one 64-row tile
  constexpr int BUFB = 2 * TB;       // Q and dO tiles of one query tile
  constexpr int STB = 2 * BQ * 4;    // L and Delta of one query tile
  constexpr int VMT = 2 * BPW + 1;   // copy instructions per wave per query tile
  constexpr int BSTEP = NW * L::RPB; // rows between a lane's consecutive copies
  static_assert(L::NBLK % NW == 0 && BSTEP % 16 == 0, "copy plan");
  static_assert(NBUF == 3 || NBUF == 4, "pipeline depth");
  static_assert(VMT < 16 && 2 * VMT < 64, "vmcnt range");

  __shared__ __attribute__((aligned(1024))) char lds[NBUF * (BUFB + STB)];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int h = lane >> 5;
  const int l32 = lane & 31;

  if constexpr (PAD) {  // padding chunks of the Q and dO buffers read as zeros
    const u32x4 z = {0u, 0u, 0u, 0u};
    for (int i = tid; i < NBUF * BUFB / 16; i += BT) *reinterpret_cast<u32x4*>(lds + 16 * i) = z;
    __syncthreads();
  }

  // Persistent loop at D >= 96 (one workgroup per CU): items are
  // (batch*head, key tile), key tiles in natural order (under the causal mask
  // the first see the most queries), taken in the snake order of
  // persistent_item.  At D = 64 (two workgroups per CU) one item each.
  constexpr bool PERSIST = DP >= 96;
  auto work = [&](const TileCoord tc) {
  const int k0 = tc.q0;
  const elt* Qh = q + (int64_t)tc.bh * M * D;
  const elt* Kh = k + (int64_t)tc.bh * N * D;
  const elt* Vh = v + (int64_t)tc.bh * N * D;
  const elt* Gh = dout + (int64_t)tc.bh * M * D;
  const int64_t nrows = (int64_t)(items / ktiles) * M;  // B*H*M
  const float* Sh = delta + nrows + (int64_t)tc.bh * M;     // -L / scale per row
  const float* Dh = delta + (int64_t)tc.bh * M;             // -Delta per row
  elt* dKh = dk + (int64_t)tc.bh * N * D;
  elt* dVh = dv + (int64_t)tc.bh * N * D;
  (void)lse;

  // Key j visible to query i iff j <= i + off; without the mask off = N (no
  // query reaches it, so only the N tail is masked).
  const int off = causal ? N - M : N;
  const int kw0 = k0 + 32 * w;
  const int key = kw0 + l32;

  vec8 kb[KK], vb[KK];
  f32x16 dka[DT], dva[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    dka[dt] = f32x16{};
    dva[dt] = f32x16{};
  }

  // Query tiles from the one holding the first query that sees key k0.
  const int qt0 = max(0, k0 - off) / BQ;
  const int nqt = (M + BQ - 1) / BQ;

  // Copy plan (the forward's): wave w issues the 1 KB copies w + NW*i of each
  // tile; lane l fills slot l % SLOTS of row (w + NW*i)*RPB + l / SLOTS.  Rows
  // past M copy row M - 1 (their P is masked to 0).  Row statistics: wave w
  // copies rows 32*(w % 2) .. +31 of -L/scale (w < 2) or -Delta (w >= 2), one
  // dword per lane.
  const int cp_sub = lane / L::SLOTS;
  const int cp_slot = lane % L::SLOTS;
  const int cp_row = w * L::RPB + cp_sub;
  const int chunk = cp_slot ^ L::swz_k(cp_row);
  const unsigned lds0 = (unsigned)(uintptr_t)(__attribute__((address_space(3))) char*)lds;
  const unsigned lds_w = __builtin_amdgcn_readfirstlane(lds0 + (unsigned)w * 1024u);
  const unsigned lds_st =
      __builtin_amdgcn_readfirstlane(lds0 + NBUF * BUFB + (unsigned)(w >> 1) * (BQ * 4));
  const float* st_src = (w >> 1) ? Dh : Sh;
  auto issue = [&](int qt) {
    const int b = qt % NBUF;
    const int q0 = qt * BQ;
    const unsigned dst = lds_w + (unsigned)(b * BUFB);
    // D = 96: slots 12..15 of a row hold no data; padding chunks stay zero
    if (chunk < L::CPR && (!PAD || 8 * chunk < D)) {
      // Byte offsets within the head: M * D < 2^31 elements, so at two bytes
      // each they fit 32 unsigned bits (formed in unsigned arithmetic).
      const unsigned rowb = 2u * (unsigned)D;
      unsigned off[BPW];
      const unsigned off0 = (unsigned)(q0 + cp_row) * rowb + 16u * (unsigned)chunk;
      if (q0 + BQ <= M) {
#pragma unroll
        for (int i = 0; i < BPW; ++i) off[i] = off0 + (unsigned)(i * BSTEP) * rowb;
      } else {
#pragma unroll
        for (int i = 0; i < BPW; ++i)
          off[i] = (unsigned)min(q0 + cp_row + i * BSTEP, M - 1) * rowb + 16u * (unsigned)chunk;
      }
      lds_copy_tile<BPW, NW * 1024, TB>(Qh, Gh, off, dst);
    }
    if (h == (w & 1)) lds_copy4(st_src + min(q0 + lane, M - 1), lds_st + (unsigned)(b * STB));
  };
  auto wait_copies = [&](int pending_tiles) {  // all but the last `pending_tiles` tiles landed
    if (pending_tiles <= 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    else if (pending_tiles == 1) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(VMT) : "memory");
    else asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * VMT) : "memory");
  };
  auto barrier = [&]() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); };

  // Row reads (A operands of S and dP, query rows in swap-2-3 order).
  const int krow = swap23(l32);
  int koff[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) koff[kk] = krow * L::ROWB + 16 * ((2 * kk + h) ^ L::swz_k(krow));
  // Transposing reads (A operands of dV^T and dK^T): lane j of a 16-lane group
  // addresses row 8h + j/4 (+4 for the second read) of a 16-query chunk and 4
  // features at 32dt + 16*dhalf + 4*(j%4); the swizzle repeats every 16 rows.
  const int dhalf = (lane >> 4) & 1;
  const int j16 = lane & 15;
  int toff[DT][2];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int hi = 0; hi < 2; ++hi) {
      const int row = 8 * h + (j16 >> 2) + 4 * hi;
      const int ch = 4 * dt + 2 * dhalf + ((j16 & 3) >> 1);
      toff[dt][hi] = row * L::ROWB + 16 * (ch ^ L::swz_k(row)) + 8 * (j16 & 1);
    }

  // Row statistics (which = 0: -L/scale, 1: -Delta) of half t of buffer b in
  // the accumulator order (register r <-> query 16 (r >> 3) + 8h + (r & 7)):
  // the initial value of the S or dP accumulator.
  auto read_stats = [&](int b, int which, int t, f32x16& x) {
    const char* base = lds + NBUF * BUFB + b * STB + which * (BQ * 4) + 4 * (32 * t + 8 * h);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x4 y = *reinterpret_cast<const f32x4*>(base + 16 * ((g & 1) + 4 * (g >> 1)));
#pragma unroll
      for (int e = 0; e < 4; ++e) x[4 * g + e] = y[e];
    }
  };

  f32x16 p;         // P of the current half (masked)
  f32x16 dpA, dpB;  // dP of the current / next half, alternating roles

  // One pipeline step: CUR = dS, dV, dK of half (bc, tcur) from p and dp_cur
  // (which holds dP - Delta); NEXT = S - L/scale, dP - Delta (into dp_next) and
  // P (into p) of half (bn, tn).
  //
  // With both, the step is issued in a fixed order, one chunk per MFMA with
  // scheduling fences between chunks: stage 1 runs the 2*KK S / dP MFMAs (row
  // reads issued LA1 MFMAs ahead) beside the VALU work of dS and the 16-bit
  // rounding of P and dS; stage 2 runs the 4*DT dV / dK MFMAs (transposing
  // reads issued LA2 MFMAs ahead, the first ones during stage 1) beside the
  // exponentials of the next half.
  auto row_read = [&](int b, int t, int m) -> vec8 {  // A operand of stage-1 MFMA m
    const char* base = lds + b * BUFB + 32 * t * L::ROWB + ((m & 1) ? TB : 0);
    return *reinterpret_cast<const vec8*>(base + koff[m >> 1]);
  };
  auto tr_read = [&](int b, int t, int m) -> vec8 {  // A operand of stage-2 MFMA m
    const int t2 = m / (2 * DT), dt = (m >> 1) % DT;
    const char* base = lds + b * BUFB + 32 * t * L::ROWB + 16 * t2 * L::ROWB + ((m & 1) ? 0 : TB);
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + toff[dt][0]));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + toff[dt][1]));
    return __builtin_bit_cast(vec8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  auto step = [&](auto cur_tag, auto next_tag, int bc, int tcur, int bn, int tn, f32x16& dp_cur,
                  f32x16& dp_next) {
    constexpr bool CUR = decltype(cur_tag)::value;
    constexpr bool NEXT = decltype(next_tag)::value;
    constexpr int NM1 = 2 * KK, NM2 = 4 * DT;
    f32x16 s;
    vec8 pb[2], dsb[2];
    if constexpr (CUR && NEXT) {
      f32x16 ds;
      vec8 ra[NM1], ta[NM2];
      read_stats(bn, 0, tn, s);
      read_stats(bn, 1, tn, dp_next);
#pragma unroll
      for (int m = 0; m < DKDV_LA1; ++m) ra[m] = row_read(bn, tn, m);
      // Stage 1.  VALU units: 16 products dS = P * (dP - Delta), then the
      // rounding of P (units 16, 17) and dS (18, 19).
#pragma unroll
      for (int m = 0; m < NM1; ++m) {
        __builtin_amdgcn_sched_barrier(0);
        if (m + DKDV_LA1 < NM1) ra[m + DKDV_LA1] = row_read(bn, tn, m + DKDV_LA1);
        const int pre = m - (NM1 - DKDV_LA2);  // first stage-2 reads, spread over the last MFMAs
        if (pre >= 0) ta[pre] = tr_read(bc, tcur, pre);
        if (m & 1) dp_next = T::mfma(ra[m], vb[m >> 1], dp_next);
        else s = T::mfma(ra[m], kb[m >> 1], s);
#pragma unroll
        for (int u = 20 * m / NM1; u < 20 * (m + 1) / NM1; ++u) {
          if (u < 16) {
            float x = p[u] * dp_cur[u];
            pin(x);
            ds[u] = x;
          } else {
            f32x8 f;
#pragma unroll
            for (int e = 0; e < 8; ++e) f[e] = u < 18 ? p[8 * (u & 1) + e] : ds[8 * (u & 1) + e];
            vec8 y = __builtin_convertvector(f, vec8);
            pin(y);
            if (u < 18) pb[u & 1] = y;
            else dsb[u & 1] = y;
          }
        }
      }
      // Stage 2.  VALU units: the 16 exponentials of the next half.
#pragma unroll
      for (int m = 0; m < NM2; ++m) {
        __builtin_amdgcn_sched_barrier(0);
        if (m + DKDV_LA2 < NM2) ta[m + DKDV_LA2] = tr_read(bc, tcur, m + DKDV_LA2);
        const int t2 = m / (2 * DT), dt = (m >> 1) % DT;
        if (m & 1) dka[dt] = T::mfma(ta[m], dsb[t2], dka[dt]);
        else dva[dt] = T::mfma(ta[m], pb[t2], dva[dt]);
#pragma unroll
        for (int r = 16 * m / NM2; r < 16 * (m + 1) / NM2; ++r) {
          float x = __builtin_amdgcn_exp2f(s[r] * c);
          pin(x);
          p[r] = x;
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    } else {
      // Pipeline head (S, dP, P only) or tail (dS, dV, dK only).
      if (NEXT) {
        read_stats(bn, 0, tn, s);
        read_stats(bn, 1, tn, dp_next);
#pragma unroll
        for (int m = 0; m < NM1; ++m) {
          const vec8 a = row_read(bn, tn, m);
          if (m & 1) dp_next = T::mfma(a, vb[m >> 1], dp_next);
          else s = T::mfma(a, kb[m >> 1], s);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) p[r] = __builtin_amdgcn_exp2f(s[r] * c);
      }
      if (CUR) {
        f32x16 ds;
#pragma unroll
        for (int r = 0; r < 16; ++r) ds[r] = p[r] * dp_cur[r];
        pack16<T>(p, pb);
        pack16<T>(ds, dsb);
#pragma unroll
        for (int m = 0; m < NM2; ++m) {
          const int t2 = m / (2 * DT), dt = (m >> 1) % DT;
          const vec8 a = tr_read(bc, tcur, m);
          if (m & 1) dka[dt] = T::mfma(a, dsb[t2], dka[dt]);
          else dva[dt] = T::mfma(a, pb[t2], dva[dt]);
        }
      }
    }
#if defined(__HIP_DEVICE_COMPILE__)
    // Keep P's exponentials in this step: without the use below they would be
    // sunk past the mask's branch, away from the MFMAs they should overlap.
    if (NEXT) asm volatile("" ::"v"(p));
#endif
  };

  // Zero P where query qb + key_of_reg(r, h) does not see this lane's key
  // (causal mask, M and N tails); rows with L = -inf are always masked here.
  auto mask = [&](int u) {
    const int qb = 32 * u;
    if (qb + 31 >= M || kw0 + 31 >= N || kw0 + 31 > qb + off) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qi = qb + key_of_reg(r, h);
        p[r] = (qi < M && key < N && key <= qi + off) ? p[r] : 0.0f;
      }
    }
  };

  using F = std::integral_constant<bool, false>;
  using Tr = std::integral_constant<bool, true>;
  // The first copies go out before the K and V loads, so that their latencies
  // overlap.
#pragma unroll
  for (int i = 0; i < NBUF - 1; ++i)
    if (qt0 + i < nqt) issue(qt0 + i);
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    const bool in_d = !PAD || 16 * kk + 8 * h < D;  // padding chunks: zero
    kb[kk] = fold_vec(load_row8<T, true>(Kh, in_d ? key : N, N, D, 16 * kk + 8 * h), qf);
    vb[kk] = load_row8<T, true>(Vh, in_d ? key : N, N, D, 16 * kk + 8 * h);
  }
  if (qt0 < nqt) {
    wait_copies(min(NBUF - 2, nqt - 1 - qt0));
    barrier();
    step(F{}, Tr{}, 0, 0, qt0 % NBUF, 0, dpB, dpA);
    mask(2 * qt0);
    int b = qt0 % NBUF;
    for (int j = qt0; j < nqt - 1; ++j) {
      const int bn = b + 1 == NBUF ? 0 : b + 1;
      step(Tr{}, Tr{}, b, 0, b, 1, dpA, dpB);
      mask(2 * j + 1);
      wait_copies(min(NBUF - 3, nqt - 2 - j));
      barrier();
      if (j + NBUF - 1 < nqt) issue(j + NBUF - 1);
      step(Tr{}, Tr{}, b, 1, bn, 0, dpB, dpA);
      mask(2 * j + 2);
      b = bn;
    }
    // Last query tile: its second half has no successor.
    step(Tr{}, Tr{}, b, 0, b, 1, dpA, dpB);
    mask(2 * nqt - 1);
    step(Tr{}, F{}, b, 1, 0, 0, dpB, dpA);
  }

  // Accumulator register 4g + e of tile dt holds feature 32dt + 8g + 4h + e of
  // this lane's key.
  if (key < N) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * dt + 8 * g + 4 * h;
        if (PAD && d0 >= D) continue;  // padding columns
        store_row4<T, true>(dVh, key, D, d0, dva[dt], g, 1.0f);
        store_row4<T, true>(dKh, key, D, d0, dka[dt], g, scale);
      }
  }
  };  // work

  if constexpr (PERSIST) {
    for (int round = 0;; ++round) {
      const int item = persistent_item(round, items);
      if (item < 0) break;
      // The previous item's last reads of the LDS buffers precede this item's
      // first copies into them.
      if (round > 0) asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      work(item_coord<false, BK>(item, ktiles));
    }
  } else {
    work(tile_coord<false, BK>(ktiles));
  }
}

// ---------------------------------------------------------------------------
// dQ.  DP: head dim padded to a multiple of 32; DFULL: D == DP.
template <class T, int DP, bool CAUSAL, bool DFULL>
__global__ __launch_bounds__(BT, 1) void fa_bwd_dq_kernel(
    const typename T::elt* __restrict__ q, const typename T::elt* __restrict__ k,
    const typename T::elt* __restrict__ v, const typename T::elt* __restrict__ dout,
    const float* __restrict__ lse, const float* __restrict__ delta, typename T::elt* __restrict__ dq,
    int M, int N, int D, int qtiles, float c, float scale, QFold qf) {
  using elt = typename T::elt;
  using vec8 = typename T::vec8;
  using St = Stager<T, DP, BNK, DFULL>;
  constexpr int STR = St::STR;
  constexpr int TILE = BNK * STR;
  constexpr int KK = DP / 16;
  constexpr int DT = DP / 32;

  __shared__ __attribute__((aligned(16))) elt smem[2 * 2 * TILE];  // [stage][K, V]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int h = lane >> 5;
  const int l32 = lane & 31;

  const TileCoord tc = tile_coord<CAUSAL, BMQ>(qtiles);
  const int q0 = tc.q0;
  const elt* Qh = q + (int64_t)tc.bh * M * D;
  const elt* Kh = k + (int64_t)tc.bh * N * D;
  const elt* Vh = v + (int64_t)tc.bh * N * D;
  const elt* Gh = dout + (int64_t)tc.bh * M * D;
  const float* Lh = lse + (int64_t)tc.bh * M;
  const float* Dh = delta + (int64_t)tc.bh * M;  // -Delta per row (the workspace's first half)
  elt* dQh = dq + (int64_t)tc.bh * M * D;

  const int off = N - M;
  const int qrow = q0 + 32 * w + l32;
  const int wq_first = q0 + 32 * w;
  const int wq_last = min(wq_first + 31, M - 1);
  const int n_end = CAUSAL ? min(N, q0 + BMQ + off) : N;
  const int ntiles = n_end > 0 ? (n_end + BNK - 1) / BNK : 0;
  int w_end = CAUSAL ? min(N, wq_last + 1 + off) : N;
  if (wq_first >= M) w_end = 0;
  const int lim = CAUSAL ? min(N, qrow + off + 1) : N;  // keys < lim are visible to qrow

  // Q and dO rows of this lane's query: B operands of S^T = K Q^T and dP^T = V dO^T.
  vec8 qb[KK], gb[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    qb[kk] = fold_vec(load_row8<T, DFULL>(Qh, qrow, M, D, 16 * kk + 8 * h), qf);
    gb[kk] = load_row8<T, DFULL>(Gh, qrow, M, D, 16 * kk + 8 * h);
  }
  float l2 = 0.0f, dl = 0.0f;
  if (qrow < M) {
    l2 = Lh[qrow] * LOG2E;
    dl = -Dh[qrow];
  }
  if (l2 == -INFINITY) l2 = 0.0f;  // no visible key: every score of the row is masked
  f32x16 dqa[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) dqa[dt] = f32x16{};

  St sk, sv;
  auto load_tile = [&](int n0) {
    sk.load(Kh, n0, N, D, tid);
    sv.load(Vh, n0, N, D, tid);
  };
  auto store_tile = [&](int stage) {
    sk.store(smem + stage * 2 * TILE, tid);
    sv.store(smem + stage * 2 * TILE + TILE, tid);
  };
  if (ntiles > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();

  const int krow0 = swap23(l32);
  for (int j = 0; j < ntiles; ++j) {
    const int n0 = j * BNK;
    const bool more = j + 1 < ntiles;
    if (more) load_tile(n0 + BNK);
    if (n0 < w_end) {
      const elt* Ks = smem + (j & 1) * 2 * TILE;
      const elt* Vs = Ks + TILE;
      f32x16 s[2] = {f32x16{}, f32x16{}}, dp[2] = {f32x16{}, f32x16{}};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const vec8 ak = *reinterpret_cast<const vec8*>(Ks + (32 * t + krow0) * STR + 16 * kk + 8 * h);
          const vec8 av = *reinterpret_cast<const vec8*>(Vs + (32 * t + krow0) * STR + 16 * kk + 8 * h);
          s[t] = T::mfma(ak, qb[kk], s[t]);
          dp[t] = T::mfma(av, gb[kk], dp[t]);
        }
      }
      const bool need_mask = (n0 + BNK > N) || (CAUSAL && n0 + BNK - 1 > wq_first + off);
      if (need_mask) {  // rare: masked scores become -inf (P = 0); see fa_bwd_dq_fast_kernel
        pin(s[0]);
        pin(s[1]);
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            s[t][r] = n0 + 32 * t + key_of_reg(r, h) < lim ? s[t][r] : -INFINITY;
      }
      f32x16 ds[2];
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(s[t][r], c, -l2));
          ds[t][r] = pr * (dp[t][r] - dl);
        }
      vec8 dsb[4];
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        f32x8 f;
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = ds[cc >> 1][8 * (cc & 1) + e];
        dsb[cc] = __builtin_convertvector(f, vec8);
      }
      // dQ^T += K^T dS^T over the 64 keys of the tile.
#pragma unroll
      for (int cc = 0; cc < 4; ++cc)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const vec8 a = load_tr8<T, STR>(Ks, 16 * cc, 32 * dt, lane);
          dqa[dt] = T::mfma(a, dsb[cc], dqa[dt]);
        }
    }
    if (more) store_tile((j + 1) & 1);
    __syncthreads();
  }

  if (qrow < M) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        store_row4<T, DFULL>(dQh, qrow, D, 32 * dt + 8 * g + 4 * h, dqa[dt], g, scale);
  }
}

// ---------------------------------------------------------------------------
// dQ on the fast path (fp16/bf16, D in {64, 96, 128}): the forward's
// pipelined layout.  NW waves x 32 query rows per workgroup (NW = 8 at D = 96
// and 128, 4 at D = 64); 64-key K and V tiles go HBM -> LDS by global_load_lds
// (no VGPR staging), double-buffered, one barrier per tile.  Both tiles use the
// K-operand swizzle of FastLayout, which keeps the row reads of S^T = K Q^T and
// dP^T = V dO^T and the transposing reads of K^T (for dQ^T += K^T dS^T)
// bank-conflict free.
// PAD: Drow < DP features per row, as in the fast dK/dV kernel (Q and dO
// padding zero in registers, K and V padding zero in LDS).
template <class T, int DP, int NW, bool PAD>
__global__ __launch_bounds__(64 * NW, 2) void fa_bwd_dq_fast_kernel(
    const typename T::elt* __restrict__ q, const typename T::elt* __restrict__ k,
    const typename T::elt* __restrict__ v, const typename T::elt* __restrict__ dout,
    const float* __restrict__ lse, const float* __restrict__ delta, typename T::elt* __restrict__ dq,
    int M, int N, int qtiles, int items, float c, float scale, int causal, QFold qf, int Drow) {
  using elt = typename T::elt;
  using vec8 = typename T::vec8;
  using L = FastLayout<DP>;
  const int D = PAD ? Drow : DP;  // features per row in HBM
  constexpr int KK = DP / 16;
  constexpr int DT = DP / 32;
  constexpr int BPW = L::NBLK / NW;
  constexpr int ROWS = 32 * NW;
  static_assert(L::NBLK % NW == 0, "copy plan");

  __shared__ __attribute__((aligned(1024))) char kb0[L::TILEB];
  __shared__ __attribute__((aligned(1024))) char kb1[L::TILEB];
  __shared__ __attribute__((aligned(1024))) char vb0[L::TILEB];
  __shared__ __attribute__((aligned(1024))) char vb1[L::TILEB];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int h = lane >> 5;
  const int l32 = lane & 31;

  if constexpr (PAD) {  // padding chunks of the K and V buffers read as zeros
    const u32x4 z = {0u, 0u, 0u, 0u};
    for (int i = tid; i < L::TILEB / 16; i += 64 * NW) {
      *reinterpret_cast<u32x4*>(kb0 + 16 * i) = z;
      *reinterpret_cast<u32x4*>(kb1 + 16 * i) = z;
      *reinterpret_cast<u32x4*>(vb0 + 16 * i) = z;
      *reinterpret_cast<u32x4*>(vb1 + 16 * i) = z;
    }
    __syncthreads();
  }

  // Persistent loop for the 8-wave instantiations (one workgroup per CU), as in
  // the forward's fast path; the 4-wave ones take one item per workgroup.
  constexpr bool PERSIST = NW == 8;
  for (int round = 0; PERSIST || round == 0; ++round) {
  const int item = persistent_item(round, items);
  if (item < 0) break;
  const TileCoord tc = item_coord<true, ROWS>(item, qtiles);  // heaviest causal tiles first
  const int q0 = tc.q0;
  const elt* Qh = q + (int64_t)tc.bh * M * D;
  const elt* Kh = k + (int64_t)tc.bh * N * D;
  const elt* Vh = v + (int64_t)tc.bh * N * D;
  const elt* Gh = dout + (int64_t)tc.bh * M * D;
  const float* Lh = lse + (int64_t)tc.bh * M;
  const float* Dh = delta + (int64_t)tc.bh * M;  // -Delta per row (the workspace's first half)
  elt* dQh = dq + (int64_t)tc.bh * M * D;

  // Causal: key j visible to row i iff j <= i + off; without the mask `off` = N
  // (no row reaches it, so only the N tail is masked).
  const int off = causal ? N - M : N;
  const int qrow = q0 + 32 * w + l32;
  const int wq_first = q0 + 32 * w;
  const int wq_last = min(wq_first + 31, M - 1);
  const int n_end = min(N, q0 + ROWS + off);
  const int ntiles = n_end > 0 ? (n_end + 63) / 64 : 0;
  int w_end = min(N, wq_last + 1 + off);
  if (wq_first >= M) w_end = 0;
  const int w_tiles = w_end > 0 ? (w_end + 63) / 64 : 0;
  const int lim = min(N, qrow + off + 1);

  vec8 qb[KK], gb[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    const bool in_d = !PAD || 16 * kk + 8 * h < D;  // padding chunks: zero
    qb[kk] = fold_vec(load_row8<T, true>(Qh, in_d ? qrow : M, M, D, 16 * kk + 8 * h), qf);
    gb[kk] = load_row8<T, true>(Gh, in_d ? qrow : M, M, D, 16 * kk + 8 * h);
  }
  float l2 = 0.0f, dl = 0.0f;
  if (qrow < M) {
    l2 = Lh[qrow] * LOG2E;
    dl = -Dh[qrow];
  }
  if (l2 == -INFINITY) l2 = 0.0f;  // no visible key: every score of the row is masked
  f32x16 dqa[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) dqa[dt] = f32x16{};

  // Copy plan as in the forward's pipelined kernel, one swizzle for K and V.
  const int cp_sub = lane / L::SLOTS;
  const int cp_slot = lane % L::SLOTS;
  const int cp_row = w * L::RPB + cp_sub;
  const int chunk = cp_slot ^ L::swz_k(cp_row);
  const unsigned goff = (unsigned)((cp_row * D + 8 * chunk) * (int)sizeof(elt));
  constexpr int BSTEP = NW * L::RPB;
  static_assert(BSTEP % 16 == 0, "swizzle period");
  const int lds_w = __builtin_amdgcn_readfirstlane(w * 1024);
  auto issue = [&](const elt* src, int n0, char* buf) {
    if (chunk >= L::CPR) return;        // D = 96: slots 12..15 of a row hold no data
    if (PAD && 8 * chunk >= D) return;  // padding: stays zero
    if (n0 + 64 <= N) {
      const char* base = reinterpret_cast<const char*>(src + (int64_t)n0 * D);
#pragma unroll
      for (int b = 0; b < BPW; ++b)
        copy16_to_lds(base + goff + (unsigned)(b * BSTEP * D * (int)sizeof(elt)),
                      buf + lds_w + NW * 1024 * b);
    } else {  // N tail: rows past N copy row N-1 instead (their scores are masked)
#pragma unroll
      for (int b = 0; b < BPW; ++b) {
        const int key = min(n0 + cp_row + b * BSTEP, N - 1);
        copy16_to_lds(src + (int64_t)key * D + 8 * chunk, buf + lds_w + NW * 1024 * b);
      }
    }
  };

  // Row reads (A operands of S^T and dP^T, rows in swap-2-3 order).
  const int krow = swap23(l32);
  int koff[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) koff[kk] = krow * L::ROWB + 16 * ((2 * kk + h) ^ L::swz_k(krow));
  // Transposing reads of K (A operand of dQ^T): lane j of a 16-lane group
  // addresses row 8h + j/4 (+4 for the second read) of a 16-key chunk and 4
  // features at 32dt + 16*dhalf + 4*(j%4).  The swizzle does not depend on the
  // 16-key chunk, so that offset is an immediate.
  const int dhalf = (lane >> 4) & 1;
  const int j16 = lane & 15;
  int toff[DT][2];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int hi = 0; hi < 2; ++hi) {
      const int row = 8 * h + (j16 >> 2) + 4 * hi;
      const int ch = 4 * dt + 2 * dhalf + ((j16 & 3) >> 1);
      toff[dt][hi] = row * L::ROWB + 16 * (ch ^ L::swz_k(row)) + 8 * (j16 & 1);
    }

  auto step = [&](int j, const char* kbuf, const char* vbuf) {
    const int n0 = j * 64;
    f32x16 s[2] = {f32x16{}, f32x16{}}, dp[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const vec8 ak = *reinterpret_cast<const vec8*>(kbuf + koff[kk] + 32 * t * L::ROWB);
        const vec8 av = *reinterpret_cast<const vec8*>(vbuf + koff[kk] + 32 * t * L::ROWB);
        s[t] = T::mfma(ak, qb[kk], s[t]);
        dp[t] = T::mfma(av, gb[kk], dp[t]);
      }
    }
    const bool need_mask = (n0 + 64 > N) || (n0 + 63 > wq_first + off);
    if (need_mask) {  // rare: diagonal or N tail.  Masked scores become -inf
      // (P = 0).  The scores pass through an opaque statement first, so that
      // the selects stay inside this branch instead of running on every tile.
      pin(s[0]);
      pin(s[1]);
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          s[t][r] = n0 + 32 * t + key_of_reg(r, h) < lim ? s[t][r] : -INFINITY;
    }
    f32x16 ds[2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(s[t][r], c, -l2));
        ds[t][r] = pr * (dp[t][r] - dl);
      }
    vec8 dsb[4];
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
      f32x8 f;
#pragma unroll
      for (int e = 0; e < 8; ++e) f[e] = ds[cc >> 1][8 * (cc & 1) + e];
      dsb[cc] = __builtin_convertvector(f, vec8);
    }
#pragma unroll
    for (int cc = 0; cc < 4; ++cc)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4*)(kbuf + toff[dt][0] + 16 * cc * L::ROWB));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4*)(kbuf + toff[dt][1] + 16 * cc * L::ROWB));
        const vec8 a = __builtin_bit_cast(vec8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        dqa[dt] = T::mfma(a, dsb[cc], dqa[dt]);
      }
  };

  if (ntiles > 0) {
    issue(Kh, 0, kb0);
    issue(Vh, 0, vb0);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  for (int j = 0; j < ntiles; j += 2) {
    if (j + 1 < ntiles) {
      issue(Kh, (j + 1) * 64, kb1);
      issue(Vh, (j + 1) * 64, vb1);
    }
    if (j < w_tiles) step(j, kb0, vb0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (j + 1 >= ntiles) break;
    if (j + 2 < ntiles) {
      issue(Kh, (j + 2) * 64, kb0);
      issue(Vh, (j + 2) * 64, vb0);
    }
    if (j + 1 < w_tiles) step(j + 1, kb1, vb1);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  }

  if (qrow < M) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        if (!PAD || 32 * dt + 8 * g + 4 * h < D)  // padding columns are not stored
          store_row4<T, true>(dQh, qrow, D, 32 * dt + 8 * g + 4 * h, dqa[dt], g, scale);
  }
  }  // persistent loop
}

// ---------------------------------------------------------------------------
// fp32 backward ("Module 08", "The backward pass: recompute instead of
// store", for fp32 inputs): the same recomputation on v_mfma_f32_32x32x2f32,
// with P and dS kept in fp32 (as the fp32 forward keeps P), one workgroup of
// four waves per (batch*head, 128-key tile) for dK/dV and per (batch*head,
// 128-query tile) for dQ, 32-row tiles staged through LDS at an odd row
// stride (conflict-free column reads).
//
// Accumulator register r of a 32x32 MFMA tile holds row crow(r, h) of the
// lane's column (l % 32).  The K = 2 dimension of the fp32 MFMA is split over
// the two lane halves, so a product summed over the rows of such a tile takes
// register r of each lane as its B operand for step r (half h contributes row
// crow(r, h)); the A operand reads the matching rows.
__device__ __forceinline__ int crow(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

__device__ __forceinline__ f32x16 mfma_f32(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// Per row: ws[row] = -Delta_i = -sum_d dO[i, d] O[i, d] (fp32), and
// ws[rows + row] = -L_i (unused by the fp32 kernels, kept for the layout).
__global__ __launch_bounds__(BT) void fa_bwd_delta_f32_kernel(const float* __restrict__ o,
                                                              const float* __restrict__ dout,
                                                              const float* __restrict__ lse,
                                                              float* __restrict__ ws, int64_t rows,
                                                              int D) {
  const int sub = threadIdx.x >> 4;
  const int l16 = threadIdx.x & 15;
  for (int64_t row0 = (int64_t)blockIdx.x * 16; row0 < rows; row0 += (int64_t)gridDim.x * 16) {
    const int64_t row = row0 + sub;
    float acc = 0.0f;
    if (row < rows)
      for (int d = l16; d < D; d += 16) acc = __builtin_fmaf(o[row * D + d], dout[row * D + d], acc);
#pragma unroll
    for (int m = 8; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 16);
    if (row < rows && l16 == 0) {
      ws[row] = -acc;
      const float x = lse[row];
      ws[rows + row] = x == -INFINITY ? 0.0f : -x;
    }
  }
}

// dK and dV, fp32.  Wave w owns keys k0 + 32 w .. + 31; K and V rows stay in
// registers as the B operands of S = Q K^T and dP = dO V^T (lane: its key,
// features 2 s + h).
template <int DP, bool CAUSAL>
__global__ __launch_bounds__(BT, 1) void fa_bwd_dkdv_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const float* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ delta,
    float* __restrict__ dk, float* __restrict__ dv, int M, int N, int D, int ktiles, float c,
    float scale, QFold qf) {
  constexpr int STR = DP + 1;
  constexpr int KS = DP / 2;
  constexpr int DT = DP / 32;
  __shared__ float qs[32 * STR], gs[32 * STR], ls[32], dls[32];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int h = lane >> 5;
  const int l32 = lane & 31;

  const TileCoord tc = tile_coord<false, BK>(ktiles);
  const int k0 = tc.q0;
  const float* Qh = q + (int64_t)tc.bh * M * D;
  const float* Kh = k + (int64_t)tc.bh * N * D;
  const float* Vh = v + (int64_t)tc.bh * N * D;
  const float* Gh = dout + (int64_t)tc.bh * M * D;
  const float* Lh = lse + (int64_t)tc.bh * M;
  const float* Dh = delta + (int64_t)tc.bh * M;  // -Delta per row
  float* dKh = dk + (int64_t)tc.bh * N * D;
  float* dVh = dv + (int64_t)tc.bh * N * D;

  const int off = N - M;  // causal: key j visible to query i iff j <= i + off
  const int kw0 = k0 + 32 * w;
  const int key = kw0 + l32;

  float kr[KS], vr[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    const int d = 2 * s + h;
    const bool in = key < N && d < D;
    kr[s] = fold_f32(in ? Kh[(int64_t)key * D + d] : 0.0f, qf);
    vr[s] = in ? Vh[(int64_t)key * D + d] : 0.0f;
  }
  f32x16 dka[DT], dva[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    dka[dt] = f32x16{};
    dva[dt] = f32x16{};
  }

  const int qstart = CAUSAL ? max(0, k0 - off) : 0;
  for (int qb = qstart / 32 * 32; qb < M; qb += 32) {
    __syncthreads();  // the previous block's rows are no longer read
    for (int i = tid; i < 32 * DP; i += BT) {
      const int r = i / DP;
      const int d = i - r * DP;
      const int gq = qb + r;
      const bool in = gq < M && d < D;
      qs[r * STR + d] = in ? Qh[(int64_t)gq * D + d] : 0.0f;
      gs[r * STR + d] = in ? Gh[(int64_t)gq * D + d] : 0.0f;
    }
    if (tid < 32) {
      const int r = qb + tid;
      // rows past M and rows with no visible key are masked: keep them finite
      const float x = r < M ? Lh[r] * LOG2E : 0.0f;
      ls[tid] = x == -INFINITY ? 0.0f : x;
      dls[tid] = r < M ? Dh[r] : 0.0f;
    }
    __syncthreads();
    // Wave-uniform skip: no query of this block sees any key of this wave.
    if (kw0 >= N || (CAUSAL && qb + 31 + off < kw0)) continue;
    f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
    for (int st = 0; st < KS; ++st) {
      s = mfma_f32(qs[l32 * STR + 2 * st + h], kr[st], s);
      dp = mfma_f32(gs[l32 * STR + 2 * st + h], vr[st], dp);
    }
    f32x16 p, ds;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int qr = crow(r, h);
      const int qi = qb + qr;
      float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c, -ls[qr]));
      const bool vis = qi < M && key < N && (!CAUSAL || key <= qi + off);
      pr = vis ? pr : 0.0f;
      p[r] = pr;
      ds[r] = pr * (dp[r] + dls[qr]);
    }
    // dV^T += dO^T P and dK^T += Q^T dS over the 32 queries of this block.
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int qr = crow(r, h);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        dva[dt] = mfma_f32(gs[qr * STR + 32 * dt + l32], p[r], dva[dt]);
        dka[dt] = mfma_f32(qs[qr * STR + 32 * dt + l32], ds[r], dka[dt]);
      }
    }
  }

  if (key < N) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int d = 32 * dt + crow(r, h);
        if (d < D) {
          dVh[(int64_t)key * D + d] = dva[dt][r];
          dKh[(int64_t)key * D + d] = dka[dt][r] * scale;
        }
      }
  }
}

// dQ, fp32.  Wave w owns queries q0 + 32 w .. + 31; Q and dO rows stay in
// registers as the B operands of S^T = K Q^T and dP^T = V dO^T.
template <int DP, bool CAUSAL>
__global__ __launch_bounds__(BT, 1) void fa_bwd_dq_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const float* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ delta,
    float* __restrict__ dq, int M, int N, int D, int qtiles, float c, float scale, QFold qf) {
  constexpr int STR = DP + 1;
  constexpr int KS = DP / 2;
  constexpr int DT = DP / 32;
  __shared__ float ks[32 * STR], vs[32 * STR];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int h = lane >> 5;
  const int l32 = lane & 31;

  const TileCoord tc = tile_coord<CAUSAL, BMQ>(qtiles);
  const int q0 = tc.q0;
  const float* Qh = q + (int64_t)tc.bh * M * D;
  const float* Kh = k + (int64_t)tc.bh * N * D;
  const float* Vh = v + (int64_t)tc.bh * N * D;
  const float* Gh = dout + (int64_t)tc.bh * M * D;
  const float* Lh = lse + (int64_t)tc.bh * M;
  const float* Dh = delta + (int64_t)tc.bh * M;
  float* dQh = dq + (int64_t)tc.bh * M * D;

  const int off = N - M;
  const int qw0 = q0 + 32 * w;
  const int qrow = qw0 + l32;

  float qr[KS], gr[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    const int d = 2 * s + h;
    const bool in = qrow < M && d < D;
    qr[s] = fold_f32(in ? Qh[(int64_t)qrow * D + d] : 0.0f, qf);
    gr[s] = in ? Gh[(int64_t)qrow * D + d] : 0.0f;
  }
  float l2 = 0.0f, nd = 0.0f;
  if (qrow < M) {
    const float x = Lh[qrow] * LOG2E;
    l2 = x == -INFINITY ? 0.0f : x;
    nd = Dh[qrow];
  }
  f32x16 dqa[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) dqa[dt] = f32x16{};

  const int n_end = CAUSAL ? min(N, q0 + BMQ + off) : N;  // keys any row of the workgroup sees
  const int w_last = min(qw0 + 31, M - 1);
  for (int kb = 0; kb < n_end; kb += 32) {
    __syncthreads();
    for (int i = tid; i < 32 * DP; i += BT) {
      const int r = i / DP;
      const int d = i - r * DP;
      const int gk = kb + r;
      const bool in = gk < N && d < D;
      ks[r * STR + d] = in ? Kh[(int64_t)gk * D + d] : 0.0f;
      vs[r * STR + d] = in ? Vh[(int64_t)gk * D + d] : 0.0f;
    }
    __syncthreads();
    if (qw0 >= M || (CAUSAL && kb > w_last + off)) continue;  // no key of this block visible
    f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
    for (int st = 0; st < KS; ++st) {
      s = mfma_f32(ks[l32 * STR + 2 * st + h], qr[st], s);
      dp = mfma_f32(vs[l32 * STR + 2 * st + h], gr[st], dp);
    }
    f32x16 ds;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kj = kb + crow(r, h);
      float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c, -l2));
      const bool vis = qrow < M && kj < N && (!CAUSAL || kj <= qrow + off);
      pr = vis ? pr : 0.0f;
      ds[r] = pr * (dp[r] + nd);
    }
    // dQ^T += K^T dS^T over the 32 keys of this block.
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kr2 = crow(r, h);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) dqa[dt] = mfma_f32(ks[kr2 * STR + 32 * dt + l32], ds[r], dqa[dt]);
    }
  }

  if (qrow < M) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int d = 32 * dt + crow(r, h);
        if (d < D) dQh[(int64_t)qrow * D + d] = dqa[dt][r] * scale;
      }
  }
}

// ---------------------------------------------------------------------------
// Host dispatch.  Every launch returns its own status (see `launch`).

struct BwdArgs {
  const void *q, *k, *v, *o, *dout;
  const float* lse;
  void *dq, *dk, *dv;
  float* delta;
  int64_t BH;
  int M, N, D;
  float c;      // positive exponent constant of the score product (fold_scale)
  float s_eff;  // positive scale of the score product (the row statistics use it)
  float scale;  // the caller's scale: the factor of dQ and dK
  QFold qf;     // sign fold of the stationary score operand (K in dK/dV, Q in dQ)
  hipStream_t stream;
  int dev;      // device of `stream`
};

// Smallest D of the padded fast path (at or below it the general kernels).
constexpr int BWD_PAD_MIN_D = 32;

template <class T, int DP, bool CAUSAL, bool DFULL>
hipError_t launch_bwd_tiles(const BwdArgs& a) {
  using elt = typename T::elt;
  hipError_t e = hipSuccess;
  // Fast kernels: D == DP, or (PAD) D a multiple of 8 above BWD_PAD_MIN_D,
  // zero-padded to DP.
  constexpr bool FAST_DP = DP == 64 || DP == 96 || DP == 128;
  constexpr bool PAD = !DFULL;
  const bool fast = FAST_DP && (DFULL || (a.D % 8 == 0 && a.D > BWD_PAD_MIN_D));
  if (a.N > 0) {
    const int ktiles = (a.N + BK - 1) / BK;
    bool done = false;
    if constexpr (FAST_DP) {
      if (fast && a.M > 0) {
        const int items = (int)(a.BH * ktiles);
        int slots = 0;  // the kernel loops over items at D >= 96 only
        if constexpr (DP >= 96)
          slots = persistent_workgroups<fa_bwd_dkdv_fast_kernel<T, DP, DKDV_NBUF, PAD>>(BT, a.dev);
        const int P = slots >= NXCD && slots < items ? slots : items;
        e = launch(fa_bwd_dkdv_fast_kernel<T, DP, DKDV_NBUF, PAD>, dim3((unsigned)P), dim3(BT),
                   a.stream, (const elt*)a.q, (const elt*)a.k, (const elt*)a.v,
                   (const elt*)a.dout, a.lse, (const float*)a.delta, (elt*)a.dk, (elt*)a.dv, a.M,
                   a.N, ktiles, items, a.c, a.scale, CAUSAL ? 1 : 0, a.qf, a.D);
        done = true;
      }
    }
    if (!done)
      e = launch(fa_bwd_dkdv_kernel<T, DP, CAUSAL, DFULL>, dim3((unsigned)(a.BH * ktiles)),
                 dim3(BT), a.stream, (const elt*)a.q, (const elt*)a.k, (const elt*)a.v,
                 (const elt*)a.dout, a.lse, (const float*)a.delta, (elt*)a.dk, (elt*)a.dv, a.M,
                 a.N, a.D, ktiles, a.c, a.scale, a.qf);
    if (e != hipSuccess) return e;
  }
  if (a.M > 0) {
    if constexpr (FAST_DP) {
      if (fast && a.N > 0) {
        constexpr int NW = DP == 64 ? 4 : 8;
        const int qtiles = (a.M + 32 * NW - 1) / (32 * NW);
        const int items = (int)(a.BH * qtiles);
        int slots = 0;  // the kernel loops over items with 8 waves only
        if constexpr (NW == 8)
          slots = persistent_workgroups<fa_bwd_dq_fast_kernel<T, DP, NW, PAD>>(64 * NW, a.dev);
        const int P = slots >= NXCD && slots < items ? slots : items;
        return launch(fa_bwd_dq_fast_kernel<T, DP, NW, PAD>, dim3((unsigned)P), dim3(64 * NW),
                      a.stream, (const elt*)a.q, (const elt*)a.k, (const elt*)a.v,
                      (const elt*)a.dout, a.lse, (const float*)a.delta, (elt*)a.dq, a.M, a.N,
                      qtiles, items, a.c, a.scale, CAUSAL ? 1 : 0, a.qf, a.D);
      }
    }
    const int qtiles = (a.M + BMQ - 1) / BMQ;
    return launch(fa_bwd_dq_kernel<T, DP, CAUSAL, DFULL>, dim3((unsigned)(a.BH * qtiles)),
                  dim3(BT), a.stream, (const elt*)a.q, (const elt*)a.k, (const elt*)a.v,
                  (const elt*)a.dout, a.lse, (const float*)a.delta, (elt*)a.dq, a.M, a.N, a.D,
                  qtiles, a.c, a.scale, a.qf);
  }
  return e;
}

template <class T, int DP, bool CAUSAL>
hipError_t dispatch_full(const BwdArgs& a) {
  if (a.D == DP) return launch_bwd_tiles<T, DP, CAUSAL, true>(a);
  return launch_bwd_tiles<T, DP, CAUSAL, false>(a);
}

template <int DP, bool CAUSAL>
hipError_t launch_bwd_f32(const BwdArgs& a) {
  hipError_t e = hipSuccess;
  if (a.N > 0) {
    const int ktiles = (a.N + BK - 1) / BK;
    e = launch(fa_bwd_dkdv_f32_kernel<DP, CAUSAL>, dim3((unsigned)(a.BH * ktiles)), dim3(BT),
               a.stream, (const float*)a.q, (const float*)a.k, (const float*)a.v,
               (const float*)a.dout, a.lse, (const float*)a.delta, (float*)a.dk, (float*)a.dv, a.M,
               a.N, a.D, ktiles, a.c, a.scale, a.qf);
    if (e != hipSuccess) return e;
  }
  if (a.M > 0) {
    const int qtiles = (a.M + BMQ - 1) / BMQ;
    e = launch(fa_bwd_dq_f32_kernel<DP, CAUSAL>, dim3((unsigned)(a.BH * qtiles)), dim3(BT),
               a.stream, (const float*)a.q, (const float*)a.k, (const float*)a.v,
               (const float*)a.dout, a.lse, (const float*)a.delta, (float*)a.dq, a.M, a.N, a.D,
               qtiles, a.c, a.scale, a.qf);
  }
  return e;
}

template <bool CAUSAL>
hipError_t dispatch_bwd_f32(const BwdArgs& a) {
  if (a.M > 0) {
    const int64_t rows = a.BH * a.M;
    const int64_t blocks = (rows + 15) / 16;
    const hipError_t e = launch(fa_bwd_delta_f32_kernel,
                                dim3((unsigned)(blocks < 65536 ? blocks : 65536)), dim3(BT),
                                a.stream, (const float*)a.o, (const float*)a.dout, a.lse, a.delta,
                                rows, a.D);
    if (e != hipSuccess) return e;
  }
  if (a.D <= 32) return launch_bwd_f32<32, CAUSAL>(a);
  if (a.D <= 64) return launch_bwd_f32<64, CAUSAL>(a);
  if (a.D <= 96) return launch_bwd_f32<96, CAUSAL>(a);
  return launch_bwd_f32<128, CAUSAL>(a);
}

template <class T, bool CAUSAL>
hipError_t dispatch_bwd(const BwdArgs& a) {
  if (a.M > 0) {
    const int64_t rows = a.BH * a.M;
    const int lpr = a.D <= 32 ? 4 : a.D <= 64 ? 8 : 16;
    const int64_t blocks = (rows + BT / lpr - 1) / (BT / lpr);
    const dim3 grid((unsigned)(blocks < 65536 ? blocks : 65536));
    using elt = typename T::elt;
    const hipError_t e =
        lpr == 4 ? launch(fa_bwd_delta_kernel<T, 4>, grid, dim3(BT), a.stream, (const elt*)a.o,
                          (const elt*)a.dout, a.lse, a.delta, rows, a.D, a.s_eff)
        : lpr == 8 ? launch(fa_bwd_delta_kernel<T, 8>, grid, dim3(BT), a.stream, (const elt*)a.o,
                            (const elt*)a.dout, a.lse, a.delta, rows, a.D, a.s_eff)
                   : launch(fa_bwd_delta_kernel<T, 16>, grid, dim3(BT), a.stream, (const elt*)a.o,
                            (const elt*)a.dout, a.lse, a.delta, rows, a.D, a.s_eff);
    if (e != hipSuccess) return e;
  }
  if (a.D <= 32) return dispatch_full<T, 32, CAUSAL>(a);
  if (a.D <= 64) return dispatch_full<T, 64, CAUSAL>(a);
  if (a.D <= 96) return dispatch_full<T, 96, CAUSAL>(a);
  return dispatch_full<T, 128, CAUSAL>(a);
}

}  // namespace

extern "C" int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                      const void* dout, void* dq, void* dk, void* dv, float* delta, int64_t B,
                      int64_t H, int64_t M, int64_t N, int64_t D, float scale, int causal, int dtype,
                      void* stream) {
  const int st = fa_bwd_check_args(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, M, N, D, scale,
                                   causal, dtype);
  if (st != FA_OK) return st;
  if (B == 0 || H == 0 || (M == 0 && N == 0)) return FA_OK;
  BwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.dout = dout;
  a.lse = lse;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.delta = delta;
  a.BH = B * H;
  a.M = (int)M;
  a.N = (int)N;
  a.D = (int)D;
  // The same fp32 constant as the forward pass: exp2(s * c - L * log2 e), with
  // the scale's sign moved into the stationary score operand.
  const ScaleFold f = fold_scale(scale, dtype == FA_DTYPE_F32 ? 4 : 2);
  a.c = f.c;
  a.s_eff = f.s_eff;
  a.scale = scale;
  a.qf = f.q;
  a.stream = (hipStream_t)stream;
  a.dev = stream_device(a.stream);
  hipError_t e;
  if (dtype == FA_DTYPE_F16)
    e = causal ? dispatch_bwd<TF16, true>(a) : dispatch_bwd<TF16, false>(a);
  else if (dtype == FA_DTYPE_BF16)
    e = causal ? dispatch_bwd<TBF16, true>(a) : dispatch_bwd<TBF16, false>(a);
  else
    e = causal ? dispatch_bwd_f32<true>(a) : dispatch_bwd_f32<false>(a);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}
