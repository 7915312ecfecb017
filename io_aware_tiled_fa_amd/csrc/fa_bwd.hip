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

typedef float f32x4 __attribute__((ext_vector_type(4)));

// Delta_i = sum_d dO[i, d] * O[i, d] in fp32; 16 lanes per row.
template <class T>
__global__ __launch_bounds__(BT) void fa_bwd_delta_kernel(const typename T::elt* __restrict__ o,
                                                          const typename T::elt* __restrict__ dout,
                                                          float* __restrict__ delta, int64_t rows,
                                                          int D) {
  using elt = typename T::elt;
  using vec8 = typename T::vec8;
  const int sub = threadIdx.x >> 4;
  const int l16 = threadIdx.x & 15;
  for (int64_t row0 = (int64_t)blockIdx.x * 16; row0 < rows; row0 += (int64_t)gridDim.x * 16) {
    const int64_t row = row0 + sub;
    float acc = 0.0f;
    if (row < rows) {
      const elt* orow = o + row * D;
      const elt* grow = dout + row * D;
      if ((D & 7) == 0) {
        for (int c8 = l16; 8 * c8 < D; c8 += 16) {
          const vec8 a = __builtin_bit_cast(vec8, *reinterpret_cast<const u32x4*>(orow + 8 * c8));
          const vec8 b = __builtin_bit_cast(vec8, *reinterpret_cast<const u32x4*>(grow + 8 * c8));
#pragma unroll
          for (int e = 0; e < 8; ++e) acc = __builtin_fmaf((float)a[e], (float)b[e], acc);
        }
      } else {
        for (int d = l16; d < D; d += 16) acc = __builtin_fmaf((float)orow[d], (float)grow[d], acc);
      }
    }
#pragma unroll
    for (int m = 8; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 16);
    if (row < rows && l16 == 0) delta[row] = acc;
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
    typename T::elt* __restrict__ dv, int M, int N, int D, int ktiles, float c, float scale) {
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
  const float* Dh = delta + (int64_t)tc.bh * M;
  elt* dKh = dk + (int64_t)tc.bh * N * D;
  elt* dVh = dv + (int64_t)tc.bh * N * D;

  const int off = N - M;  // causal: key j visible to query i iff j <= i + off
  const int kw0 = k0 + 32 * w;
  const int key = kw0 + l32;

  // K and V rows of this lane's key: B operands of S = Q K^T and dP = dO V^T.
  vec8 kb[KK], vb[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    kb[kk] = load_row8<T, DFULL>(Kh, key, N, D, 16 * kk + 8 * h);
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
      if (r < M) x = tid < BQ ? Lh[r] * LOG2E : Dh[r];
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
      for (int r = 0; r < 16; ++r) {
        float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c, -l2[r]));
        if (need_mask) {
          const int qi = qb + key_of_reg(r, h);
          const bool vis = qi < M && key < N && (!CAUSAL || key <= qi + off);
          pr = vis ? pr : 0.0f;
        }
        p[r] = pr;
        ds[r] = pr * (dp[r] - dl[r]);
      }
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
// dQ.  DP: head dim padded to a multiple of 32; DFULL: D == DP.
template <class T, int DP, bool CAUSAL, bool DFULL>
__global__ __launch_bounds__(BT, 1) void fa_bwd_dq_kernel(
    const typename T::elt* __restrict__ q, const typename T::elt* __restrict__ k,
    const typename T::elt* __restrict__ v, const typename T::elt* __restrict__ dout,
    const float* __restrict__ lse, const float* __restrict__ delta, typename T::elt* __restrict__ dq,
    int M, int N, int D, int qtiles, float c, float scale) {
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
  const float* Dh = delta + (int64_t)tc.bh * M;
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
    qb[kk] = load_row8<T, DFULL>(Qh, qrow, M, D, 16 * kk + 8 * h);
    gb[kk] = load_row8<T, DFULL>(Gh, qrow, M, D, 16 * kk + 8 * h);
  }
  float l2 = 0.0f, dl = 0.0f;
  if (qrow < M) {
    l2 = Lh[qrow] * LOG2E;
    dl = Dh[qrow];
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
      f32x16 ds[2];
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(s[t][r], c, -l2));
          if (need_mask) pr = (n0 + 32 * t + key_of_reg(r, h) < lim) ? pr : 0.0f;
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
template <class T, int DP, int NW>
__global__ __launch_bounds__(64 * NW, 2) void fa_bwd_dq_fast_kernel(
    const typename T::elt* __restrict__ q, const typename T::elt* __restrict__ k,
    const typename T::elt* __restrict__ v, const typename T::elt* __restrict__ dout,
    const float* __restrict__ lse, const float* __restrict__ delta, typename T::elt* __restrict__ dq,
    int M, int N, int qtiles, float c, float scale, int causal) {
  using elt = typename T::elt;
  using vec8 = typename T::vec8;
  using L = FastLayout<DP>;
  constexpr int D = DP;
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

  const TileCoord tc = tile_coord<true, ROWS>(qtiles);  // heaviest causal tiles first
  const int q0 = tc.q0;
  const elt* Qh = q + (int64_t)tc.bh * M * D;
  const elt* Kh = k + (int64_t)tc.bh * N * D;
  const elt* Vh = v + (int64_t)tc.bh * N * D;
  const elt* Gh = dout + (int64_t)tc.bh * M * D;
  const float* Lh = lse + (int64_t)tc.bh * M;
  const float* Dh = delta + (int64_t)tc.bh * M;
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
    qb[kk] = load_row8<T, true>(Qh, qrow, M, D, 16 * kk + 8 * h);
    gb[kk] = load_row8<T, true>(Gh, qrow, M, D, 16 * kk + 8 * h);
  }
  float l2 = 0.0f, dl = 0.0f;
  if (qrow < M) {
    l2 = Lh[qrow] * LOG2E;
    dl = Dh[qrow];
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
    if (chunk >= L::CPR) return;  // D = 96: slots 12..15 of a row hold no data
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
    f32x16 ds[2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(s[t][r], c, -l2));
        if (need_mask) pr = (n0 + 32 * t + key_of_reg(r, h) < lim) ? pr : 0.0f;
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
        store_row4<T, true>(dQh, qrow, D, 32 * dt + 8 * g + 4 * h, dqa[dt], g, scale);
  }
}

// ---------------------------------------------------------------------------
// Host dispatch.

struct BwdArgs {
  const void *q, *k, *v, *o, *dout;
  const float* lse;
  void *dq, *dk, *dv;
  float* delta;
  int64_t BH;
  int M, N, D;
  float c, scale;
  hipStream_t stream;
};

template <class T, int DP, bool CAUSAL, bool DFULL>
void launch_bwd_tiles(const BwdArgs& a) {
  using elt = typename T::elt;
  if (a.N > 0) {
    const int ktiles = (a.N + BK - 1) / BK;
    hipLaunchKernelGGL((fa_bwd_dkdv_kernel<T, DP, CAUSAL, DFULL>), dim3((unsigned)(a.BH * ktiles)),
                       dim3(BT), 0, a.stream, (const elt*)a.q, (const elt*)a.k, (const elt*)a.v,
                       (const elt*)a.dout, a.lse, a.delta, (elt*)a.dk, (elt*)a.dv, a.M, a.N, a.D,
                       ktiles, a.c, a.scale);
  }
  if (a.M > 0) {
    if constexpr (DFULL && (DP == 64 || DP == 96 || DP == 128)) {
      if (a.N > 0) {
        constexpr int NW = DP == 64 ? 4 : 8;
        const int qtiles = (a.M + 32 * NW - 1) / (32 * NW);
        hipLaunchKernelGGL((fa_bwd_dq_fast_kernel<T, DP, NW>), dim3((unsigned)(a.BH * qtiles)),
                           dim3(64 * NW), 0, a.stream, (const elt*)a.q, (const elt*)a.k,
                           (const elt*)a.v, (const elt*)a.dout, a.lse, a.delta, (elt*)a.dq, a.M,
                           a.N, qtiles, a.c, a.scale, CAUSAL ? 1 : 0);
        return;
      }
    }
    const int qtiles = (a.M + BMQ - 1) / BMQ;
    hipLaunchKernelGGL((fa_bwd_dq_kernel<T, DP, CAUSAL, DFULL>), dim3((unsigned)(a.BH * qtiles)),
                       dim3(BT), 0, a.stream, (const elt*)a.q, (const elt*)a.k, (const elt*)a.v,
                       (const elt*)a.dout, a.lse, a.delta, (elt*)a.dq, a.M, a.N, a.D, qtiles, a.c,
                       a.scale);
  }
}

template <class T, int DP, bool CAUSAL>
void dispatch_full(const BwdArgs& a) {
  if (a.D == DP) launch_bwd_tiles<T, DP, CAUSAL, true>(a);
  else launch_bwd_tiles<T, DP, CAUSAL, false>(a);
}

template <class T, bool CAUSAL>
void dispatch_bwd(const BwdArgs& a) {
  if (a.M > 0) {
    const int64_t rows = a.BH * a.M;
    const int64_t blocks = (rows + 15) / 16;
    hipLaunchKernelGGL((fa_bwd_delta_kernel<T>), dim3((unsigned)(blocks < 65536 ? blocks : 65536)),
                       dim3(BT), 0, a.stream, (const typename T::elt*)a.o,
                       (const typename T::elt*)a.dout, a.delta, rows, a.D);
  }
  if (a.D <= 32) dispatch_full<T, 32, CAUSAL>(a);
  else if (a.D <= 64) dispatch_full<T, 64, CAUSAL>(a);
  else if (a.D <= 96) dispatch_full<T, 96, CAUSAL>(a);
  else dispatch_full<T, 128, CAUSAL>(a);
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
  // The same fp32 constant as the forward pass: exp2(s * c - L * log2 e).
  a.c = (float)((double)scale * 1.4426950408889634074);
  a.scale = scale;
  a.stream = (hipStream_t)stream;
  (void)hipGetLastError();
  if (dtype == FA_DTYPE_F16) causal ? dispatch_bwd<TF16, true>(a) : dispatch_bwd<TF16, false>(a);
  else causal ? dispatch_bwd<TBF16, true>(a) : dispatch_bwd<TBF16, false>(a);
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_HIP;
}
