// fa_fwd.hip - FlashAttention forward for CDNA4 (gfx950): kernels and the C-ABI entry.
//
// What is computed (per batch b, head h): O = softmax(scale * Q K^T) V and
// LSE = m + ln(l) per query row, by the online-softmax recurrence over K/V tiles
// ("Module 08: FlashAttention and Memory-Efficient Kernels", "Tiling and the
// online softmax"; the loop of the "FlashAttention-style kernel" page): running
// max m, running sum l, and an un-normalised fp32 accumulator rescaled by
// alpha = exp2(m_old - m_new), one division at the end.  No M x N matrix exists
// anywhere; the largest score array is one 32-key x 32-query register tile.
//
// Mapping onto gfx950:
//  * One workgroup = 4 waves = 128 query rows; each wave owns 32 rows.  The Q
//    rows stay in registers for the whole K/V loop.
//  * K/V tiles of 64 keys are loaded from HBM with 16-byte coalesced loads,
//    double-buffered through LDS (one barrier per tile).  V is transposed on its
//    way into LDS so that every MFMA operand read is one 16-byte LDS read.
//  * Both products run on MFMA (v_mfma_f32_32x32x16_{bf16,f16}; fp32 inputs use
//    v_mfma_f32_32x32x2f32).  The kernel computes S^T = K Q^T rather than S: in
//    the 32x32 accumulator layout each lane then holds 16 keys of ONE query, so
//    the row max/sum is a register reduction plus one exchange with lane^32, the
//    rescale of O^T is one multiplier per lane, and P^T is already in the B
//    operand layout of O^T += V^T P^T (no data movement between the two MFMAs).
//    The K rows feeding the S^T tile are permuted (bits 2 and 3 of the row index
//    swapped) so that the 8 keys each lane contributes to a PV MFMA are
//    consecutive, which makes the V^T operand one contiguous LDS read.
//  * exp2 with scale*log2(e) folded into one FMA per score; LSE converted back
//    to natural log once per row ("FlashAttention-style kernel", "The loop").
//  * The 16-bit kernels move a row's running max only when a tile raises it by
//    more than 8 (log2 units); until then p may exceed 1 by up to 2^8.  The
//    result is the same softmax (the max cancels between O and l, and LSE uses
//    the max actually subtracted); the accumulator rescale becomes rare.  Two
//    row sums are kept: the fp32 sum of p for the LSE, and for O the same sum
//    with each tile's largest p counted as rounded into the PV operand (that
//    weight is no longer exactly 1, so its rounding must cancel in O).
//  * Causal (bottom-right, key j visible to row i iff j <= i + N - M): K/V tiles
//    beyond the workgroup's last visible key are never loaded; a wave skips the
//    MFMAs of tiles none of its rows can see; masks are applied only on tiles
//    that cross a row's diagonal or the N tail.  An all-masked running max is
//    clamped to 0 so that -inf - (-inf) never happens (Module 08, "Common
//    mistakes"); a row with no visible key ends with l = 0 and stores O = 0,
//    LSE = -inf.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <type_traits>

#include "fa.h"
#include "fa_device.h"

namespace {

constexpr int BM = 128;       // query rows per workgroup
constexpr int BN = 64;        // keys per K/V tile (16/bf16 kernel)
constexpr int BN32 = 32;      // keys per K/V tile (fp32 kernel)
constexpr int NTHREADS = 256; // 4 waves of 64
// Row max and row sum over a lane's NT x 16 accumulator registers, as tree
// reductions (short dependency chains; every kernel uses the same order).
__device__ __forceinline__ float fmax3(float a, float b, float c) { return fmaxf(fmaxf(a, b), c); }

// Row max with three-input maxima (v_max3_f32), fixed order.
__device__ __forceinline__ float max_tree16(const f32x16& s) {
  const float a0 = fmax3(s[0], s[1], s[2]), a1 = fmax3(s[3], s[4], s[5]);
  const float a2 = fmax3(s[6], s[7], s[8]), a3 = fmax3(s[9], s[10], s[11]);
  const float a4 = fmax3(s[12], s[13], s[14]);
  return fmaxf(fmax3(a0, a1, a2), fmax3(a3, a4, s[15]));
}
template <int NT>
__device__ __forceinline__ float max_tree(const f32x16 (&s)[NT]);
template <>
__device__ __forceinline__ float max_tree<1>(const f32x16 (&s)[1]) {
  return max_tree16(s[0]);
}
template <>
__device__ __forceinline__ float max_tree<2>(const f32x16 (&s)[2]) {
  const f32x16& x = s[0];
  const f32x16& y = s[1];
  const float a0 = fmax3(x[0], x[1], x[2]), a1 = fmax3(x[3], x[4], x[5]);
  const float a2 = fmax3(x[6], x[7], x[8]), a3 = fmax3(x[9], x[10], x[11]);
  const float a4 = fmax3(x[12], x[13], x[14]), a5 = fmax3(x[15], y[0], y[1]);
  const float a6 = fmax3(y[2], y[3], y[4]), a7 = fmax3(y[5], y[6], y[7]);
  const float a8 = fmax3(y[8], y[9], y[10]), a9 = fmax3(y[11], y[12], y[13]);
  const float a10 = fmaxf(y[14], y[15]);
  const float b0 = fmax3(a0, a1, a2), b1 = fmax3(a3, a4, a5), b2 = fmax3(a6, a7, a8);
  const float b3 = fmaxf(a9, a10);
  return fmaxf(fmax3(b0, b1, b2), b3);
}
template <int NT>
__device__ __forceinline__ float sum_tree(const f32x16 (&s)[NT]) {
  float m[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) m[r] = s[0][r];
#pragma unroll
  for (int t = 1; t < NT; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) m[r] = m[r] + s[t][r];
#pragma unroll
  for (int wdt = 8; wdt >= 1; wdt >>= 1)
#pragma unroll
    for (int r = 0; r < wdt; ++r) m[r] = m[r] + m[r + wdt];
  return m[0];
}

// Online-softmax update for one lane's query row over NT accumulator tiles of
// raw scores (already masked with -inf).  m_run is in scaled base-2 units:
//   m_new = max(m_run, rowmax * c),  alpha = exp2(m_run - m_new),
//   p = exp2(s * c - m_new),         l_run = l_run * alpha + sum(p).
// An all-masked running max (-inf) is clamped to 0 before it is subtracted.
// Replaces the scores with p.  Returns alpha and whether any lane of the wave
// moved a finite maximum (otherwise alpha is 1 everywhere and the O rescale is
// skipped; multiplying by 1 would change nothing).
struct SoftmaxStep {
  float alpha;
  bool rescale;
};
template <int NT>
__device__ __forceinline__ SoftmaxStep softmax_update(f32x16 (&s)[NT], float c, float& m_run,
                                                      float& l_run) {
  const float mx = pair_max(max_tree<NT>(s)) * c;
  const float m_new = fmaxf(m_run, mx);
  const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;  // nothing visible yet: clamp
  const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) s[t][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[t][r], c, -m_use));
  l_run = l_run * alpha + sum_tree<NT>(s);
  const bool rescale = __any(m_new > m_run && m_run != -INFINITY);
  m_run = m_new;
  return SoftmaxStep{alpha, rescale};
}

// Online-softmax update with a lazily moved maximum: the running max m_run of
// a row moves only when the row's scaled tile max exceeds it by more than
// LAZY_SLACK (in log2 units), and then to that tile max.  Until then
// p = exp2(s*c - m_run) may reach 2^LAZY_SLACK, which the fp32 sums and the
// 16-bit P operand hold without loss; the normalisation by l at the end, and
// LSE = m + log2(l), do not depend on which max was used.  Each row's maxima
// depend on its own scores only, so a row's result does not depend on the
// other rows of its wave.  alpha = exp2(m_old - m_new) is exactly 1 for rows
// whose max stayed; `grow` (any row of the wave moved) gates the rescale of
// the accumulator.
constexpr float LAZY_SLACK = 8.0f;
struct LazyMax {
  float m_new, m_use, alpha;
  bool grow;
};
__device__ __forceinline__ LazyMax lazy_max(float mx, float m_run) {
  const bool up = mx > m_run + LAZY_SLACK;
  LazyMax r;
  r.m_new = up ? mx : m_run;
  r.m_use = (r.m_new == -INFINITY) ? 0.0f : r.m_new;  // nothing visible yet: clamp
  r.alpha = __builtin_amdgcn_exp2f(m_run - r.m_use);
  r.grow = __any(up);
  return r;
}
// What rounding the lane's largest p of a tile into the 16-bit PV operand
// changes it by: p = exp2(lmax * c - m_use) for the lane's raw score maximum
// lmax, computed exactly as that element's own exponential, minus its
// rounded value (0 for an all-masked lane).  With a lazily moved max the
// largest p is up to 2^LAZY_SLACK instead of exactly 1, so its rounding would
// otherwise bias a peaked row's output; the sum O is normalised by counts the
// rounded value instead.
template <class T>
__device__ __forceinline__ float top_rounding(float lmax, float c, float m_use) {
  const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(lmax, c, -m_use));
  return (float)(typename T::elt)p - p;
}

// Sum of 8 values as a fixed tree.
__device__ __forceinline__ float sum8(const f32x8& p) {
  return ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
}
// Sum of a lane's 32 p values in the order the pipelined kernel uses: one
// 8-value tree per P operand chunk (registers 8cc .. 8cc+7), then a tree of the
// four chunk sums.
__device__ __forceinline__ float sum_p32(const f32x16 (&s)[2]) {
  float ps[4];
#pragma unroll
  for (int cc = 0; cc < 4; ++cc) {
    f32x8 pf;
#pragma unroll
    for (int e = 0; e < 8; ++e) pf[e] = s[cc >> 1][8 * (cc & 1) + e];
    ps[cc] = sum8(pf);
  }
  return (ps[0] + ps[1]) + (ps[2] + ps[3]);
}
template <class T>
__device__ __forceinline__ SoftmaxStep softmax_update_lazy(f32x16 (&s)[2], float c, float& m_run,
                                                           float& l_run, float& lr_run) {
  const float lmax = max_tree<2>(s);
  const LazyMax lm = lazy_max(pair_max(lmax) * c, m_run);
  const float corr = top_rounding<T>(lmax, c, lm.m_use);
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      s[t][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[t][r], c, -lm.m_use));
  const float ps = sum_p32(s);
  l_run = __builtin_fmaf(l_run, lm.alpha, ps);
  lr_run = __builtin_fmaf(lr_run, lm.alpha, ps + corr);
  m_run = lm.m_new;
  return SoftmaxStep{lm.alpha, lm.grow};
}

// p of a 64-key tile rounded to the 16-bit input type: pb[cc] holds keys
// 16cc + 8h + e (e = 0..7), the B operand of the PV MFMA for key chunk cc.
template <class T>
__device__ __forceinline__ void pack_p(const f32x16 (&s)[2], typename T::vec8 (&pb)[4]) {
#pragma unroll
  for (int cc = 0; cc < 4; ++cc) {
    f32x8 pf;
#pragma unroll
    for (int e = 0; e < 8; ++e) pf[e] = s[cc >> 1][8 * (cc & 1) + e];
    pb[cc] = __builtin_convertvector(pf, typename T::vec8);
  }
}

// Mask keys a lane's row may not see in the tile starting at key n0.
// lim: exclusive key limit of the row (min(N, i + N - M + 1) or N).
// The test key >= lim is done as (key - n0 - 8h) >= (lim - n0 - 8h): the left
// side is a compile-time constant per register, so the mask needs one
// per-lane threshold instead of a key offset per register.
template <int NT>
__device__ __forceinline__ void apply_mask(f32x16 (&s)[NT], int n0, int h, int lim) {
  const int thr = lim - n0 - 8 * h;
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      if (32 * t + key_of_reg(r, 0) >= thr) s[t][r] = -INFINITY;
    }
}

// Key chunking of one launch of the general kernels (the split-KV forward):
// blockIdx.y = g selects keys [g*chunk, min(N, (g+1)*chunk)) of every head, and
// the outputs of chunk g start g*o_gstride (O) and g*l_gstride (LSE) elements
// further.  A plain forward launch has one chunk of N keys and zero strides.
struct KeySplit {
  int chunk;
  int64_t o_gstride;
  int64_t l_gstride;
};

// Four consecutive output values of a row (16-bit or fp32 outputs).
template <class OUT>
__device__ __forceinline__ void store4(OUT* p, const OUT (&y)[4]) {
  if constexpr (sizeof(OUT) == 4) *reinterpret_cast<u32x4*>(p) = __builtin_bit_cast(u32x4, y);
  else *reinterpret_cast<u32x2*>(p) = __builtin_bit_cast(u32x2, y);
}

// ---------------------------------------------------------------------------
// fp16 / bf16 kernel.  DP: head dim padded to a multiple of 32 (32..128).
// DFULL: D == DP (rows are whole 16-byte chunks, no column masks).
template <class T, int DP, bool CAUSAL, bool DFULL, class OUT>
__global__ __launch_bounds__(NTHREADS, 2) void fa_fwd_lp_kernel(
    const typename T::elt* __restrict__ q, const typename T::elt* __restrict__ k,
    const typename T::elt* __restrict__ v, OUT* __restrict__ o, float* __restrict__ lse, int M,
    int Ntot, int D, int qtiles, float c, KeySplit ks, QFold qf) {
  using elt = typename T::elt;
  using vec8 = typename T::vec8;
  constexpr int KSTR = DP + 8;          // LDS row stride of K (elements)
  constexpr int VSTR = BN + 8;          // LDS row stride of V^T (elements)
  constexpr int K_ELEMS = BN * KSTR;
  constexpr int V_ELEMS = DP * VSTR;
  constexpr int STAGE = K_ELEMS + V_ELEMS;
  constexpr int KCH = DP / 8;           // 16-byte chunks per K row
  constexpr int KLD = BN * KCH / NTHREADS;  // K chunks per thread
  constexpr int NVB = (BN / 8) * (DP / 4);  // 8-key x 4-column V blocks per tile
  constexpr int DT = DP / 32;           // 32-column O^T tiles
  constexpr int KK = DP / 16;           // k-steps of S^T
  static_assert(BN * KCH % NTHREADS == 0, "K staging");
  static_assert(NVB <= NTHREADS, "V staging");

  __shared__ __attribute__((aligned(16))) elt smem[2 * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int h = lane >> 5;
  const int l32 = lane & 31;

  const TileCoord tc = tile_coord<CAUSAL>(qtiles);
  const int q0 = tc.q0;
  const int nlo = (int)blockIdx.y * ks.chunk;  // first key of this launch's chunk
  const int N = min(ks.chunk, Ntot - nlo);     // keys in the chunk
  const elt* Qh = q + (int64_t)tc.bh * M * D;
  const elt* Kh = k + ((int64_t)tc.bh * Ntot + nlo) * D;
  const elt* Vh = v + ((int64_t)tc.bh * Ntot + nlo) * D;
  OUT* Oh = o + (int64_t)blockIdx.y * ks.o_gstride + (int64_t)tc.bh * M * D;
  float* Lh = lse + (int64_t)blockIdx.y * ks.l_gstride + (int64_t)tc.bh * M;

  // causal: row i sees chunk key j (global key nlo + j) iff j <= i + off
  const int off = Ntot - M - nlo;
  const int qrow = q0 + 32 * w + l32;
  const int wq_first = q0 + 32 * w;
  const int wq_last = min(wq_first + 31, M - 1);
  int n_end = CAUSAL ? min(N, q0 + BM + off) : N;
  const int ntiles = n_end > 0 ? (n_end + BN - 1) / BN : 0;
  int w_end = CAUSAL ? min(N, wq_last + 1 + off) : N;
  if (wq_first >= M) w_end = 0;
  const int lim = CAUSAL ? min(N, qrow + off + 1) : N;

  // Q^T as the B operand of S^T = K Q^T: lane holds row qrow, 8 features per k-step.
  vec8 qreg[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    const int d0 = 16 * kk + 8 * h;
    if (DFULL) {
      u32x4 raw = {0u, 0u, 0u, 0u};
      if (qrow < M) raw = *reinterpret_cast<const u32x4*>(Qh + (int64_t)qrow * D + d0);
      qreg[kk] = __builtin_bit_cast(vec8, fold_bits(raw, qf));
    } else {
      vec8 x;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        x[e] = (qrow < M && d0 + e < D) ? Qh[(int64_t)qrow * D + d0 + e] : (elt)0.0f;
      qreg[kk] = fold_vec(x, qf);
    }
  }

  f32x16 acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x16{};
  float m_run = -INFINITY;
  float l_run = 0.0f;
  float lr_run = 0.0f;  // the sum O is normalised by (see top_rounding)

  // Register staging of one K/V tile (global -> registers -> LDS).
  u32x4 kreg[KLD];
  u32x2 vreg[8];
  const int vb_kg = tid / (DP / 4);
  const int vb_dc = tid - vb_kg * (DP / 4);

  auto load_tile = [&](int n0) {
#pragma unroll
    for (int i = 0; i < KLD; ++i) {
      const int ci = tid + NTHREADS * i;
      const int row = ci / KCH;
      const int col = (ci - row * KCH) * 8;
      const int key = n0 + row;
      if (DFULL) {
        u32x4 raw = {0u, 0u, 0u, 0u};
        if (key < N) raw = *reinterpret_cast<const u32x4*>(Kh + (int64_t)key * D + col);
        kreg[i] = raw;
      } else {
        vec8 x;
#pragma unroll
        for (int e = 0; e < 8; ++e)
          x[e] = (key < N && col + e < D) ? Kh[(int64_t)key * D + col + e] : (elt)0.0f;
        kreg[i] = __builtin_bit_cast(u32x4, x);
      }
    }
    if (tid < NVB) {
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const int key = n0 + 8 * vb_kg + kk;
        const int d0 = 4 * vb_dc;
        if (DFULL) {
          u32x2 raw = {0u, 0u};
          if (key < N) raw = *reinterpret_cast<const u32x2*>(Vh + (int64_t)key * D + d0);
          vreg[kk] = raw;
        } else {
          elt x[4];
#pragma unroll
          for (int e = 0; e < 4; ++e)
            x[e] = (key < N && d0 + e < D) ? Vh[(int64_t)key * D + d0 + e] : (elt)0.0f;
          vreg[kk] = __builtin_bit_cast(u32x2, x);
        }
      }
    }
  };

  auto store_tile = [&](int stage) {
    elt* Ks = smem + stage * STAGE;
    elt* Vs = Ks + K_ELEMS;
#pragma unroll
    for (int i = 0; i < KLD; ++i) {
      const int ci = tid + NTHREADS * i;
      const int row = ci / KCH;
      const int col = (ci - row * KCH) * 8;
      *reinterpret_cast<u32x4*>(Ks + row * KSTR + col) = kreg[i];
    }
    if (tid < NVB) {
      // 8 keys x 4 columns -> 4 rows of V^T with 8 consecutive keys each.
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const unsigned sel = (j & 1) ? 0x07060302u : 0x05040100u;
        u32x4 out;
#pragma unroll
        for (int m = 0; m < 4; ++m)
          out[m] = __builtin_amdgcn_perm(vreg[2 * m + 1][j >> 1], vreg[2 * m][j >> 1], sel);
        *reinterpret_cast<u32x4*>(Vs + (4 * vb_dc + j) * VSTR + 8 * vb_kg) = out;
      }
    }
  };

  if (ntiles > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();

  const int krow0 = swap23(l32);
  for (int j = 0; j < ntiles; ++j) {
    const int n0 = j * BN;
    const bool more = j + 1 < ntiles;
    if (more) load_tile(n0 + BN);
    if (n0 < w_end) {
      const elt* Ks = smem + (j & 1) * STAGE;
      const elt* Vs = Ks + K_ELEMS;
      f32x16 s[2] = {f32x16{}, f32x16{}};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const vec8 a0 = *reinterpret_cast<const vec8*>(Ks + krow0 * KSTR + 16 * kk + 8 * h);
        const vec8 a1 =
            *reinterpret_cast<const vec8*>(Ks + (32 + krow0) * KSTR + 16 * kk + 8 * h);
        s[0] = T::mfma(a0, qreg[kk], s[0]);
        s[1] = T::mfma(a1, qreg[kk], s[1]);
      }
      const bool need_mask = (n0 + BN > N) || (CAUSAL && n0 + BN - 1 > wq_first + off);
      if (need_mask) apply_mask<2>(s, n0, h, lim);
      const SoftmaxStep st = softmax_update_lazy<T>(s, c, m_run, l_run, lr_run);
      vec8 pb[4];
      pack_p<T>(s, pb);
      if (st.rescale) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) acc[dt] *= st.alpha;
      }
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const vec8 a =
              *reinterpret_cast<const vec8*>(Vs + (32 * dt + l32) * VSTR + 16 * cc + 8 * h);
          acc[dt] = T::mfma(a, pb[cc], acc[dt]);
        }
      }
    }
    if (more) store_tile((j + 1) & 1);
    __syncthreads();
  }

  // Epilogue: O = acc / lr (0 for an empty row), LSE = ln2 * (m + log2 l).
  const float l_tot = pair_sum(l_run);  // LSE
  const float lr_tot = pair_sum(lr_run);
  const float inv = lr_tot > 0.0f ? 1.0f / lr_tot : 0.0f;
  if (qrow < M) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * dt + 8 * g + 4 * h;
        OUT y[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = (OUT)(acc[dt][4 * g + e] * inv);
        if (DFULL) {
          store4<OUT>(Oh + (int64_t)qrow * D + d0, y);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (d0 + e < D) Oh[(int64_t)qrow * D + d0 + e] = y[e];
        }
      }
    if (h == 0)
      Lh[qrow] = l_tot > 0.0f ? LN2F * (m_run + __builtin_amdgcn_logf(l_tot)) : -INFINITY;
  }
}


// ---------------------------------------------------------------------------
// Software-pipelined fast path (fp16/bf16, D in {64, 96, 128}).
//
// Three tiles are in flight per wave.  Step j issues, on the MFMA unit, the
// scores of tile j+2 (S(j+2) = K(j+2) Q^T) and the product O^T += V(j)^T P(j)^T,
// while the VALU computes softmax(j+1) (exp2, row sum, rounding P to 16 bits)
// and, at the end of the step, the row max of S(j+2).  The step is laid out
// in slots of two MFMAs with the softmax cut into parts spread over the slots
// and a scheduling fence after each slot, so that with two waves per SIMD
// the VALU work of one wave issues under the MFMAs of the other.  K runs two
// tiles ahead of V; each has a pair of LDS buffers (64 KB at D = 128), and
// the copies of K(j+3) and V(j+1) are in flight during step j (one barrier
// per step).  The running max moves lazily (see softmax_update_lazy), so the
// O rescale is a rare branch instead of DT*16 multiplies per step.
//
// One instantiation serves causal and non-causal calls: `off_all` is the
// causal diagonal offset (key j visible to row i iff j <= i + off_all), N - M
// for a bottom-right causal mask and N for no mask (no row can reach it, so
// only the N tail is ever masked).  With a key split (blockIdx.y = chunk) the
// same offset, less the chunk's first key, applies to the chunk's keys.
//
// PAD: the rows hold Drow < DP features, Drow a multiple of 8, so every row is
// a whole number of 16-byte chunks and starts 16-byte aligned.  Chunks at or
// past Drow are neither loaded nor copied: Q's are zero in registers, K's and
// V's stay zero in LDS (cleared once at the start), so they add nothing to the
// scores and only fill output columns that are not stored.
template <class T, int DP, int NW, class OUT, bool PAD>
__global__ __launch_bounds__(64 * NW, 2) void fa_fwd_lp_pipe_kernel(
    const typename T::elt* __restrict__ q, const typename T::elt* __restrict__ k,
    const typename T::elt* __restrict__ v, OUT* __restrict__ o, float* __restrict__ lse, int M,
    int Ntot, int off_all, int qtiles, int items, float c, KeySplit ks, QFold qf, int Drow) {
  constexpr bool CAUSAL = true;  // masking logic always on; `off` decides what it masks
  const int D = PAD ? Drow : DP;  // features per row in HBM
  using elt = typename T::elt;
  using vec8 = typename T::vec8;
  using L = FastLayout<DP>;
  constexpr int DT = DP / 32;
  constexpr int KK = DP / 16;
  constexpr int BPW = L::NBLK / NW;  // copy instructions per wave per tile matrix
  constexpr int ROWS = 32 * NW;      // query rows per workgroup
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

  if constexpr (PAD) {  // padding chunks of all four tile buffers read as zeros
    constexpr int NB = L::TILEB / 16;
    const u32x4 z = {0u, 0u, 0u, 0u};
    for (int i = tid; i < NB; i += 64 * NW) {
      *reinterpret_cast<u32x4*>(kb0 + 16 * i) = z;
      *reinterpret_cast<u32x4*>(kb1 + 16 * i) = z;
      *reinterpret_cast<u32x4*>(vb0 + 16 * i) = z;
      *reinterpret_cast<u32x4*>(vb1 + 16 * i) = z;
    }
    __syncthreads();
  }

  // Persistent loop (8-wave instantiations, one workgroup per CU): with fewer
  // workgroups than work items a workgroup takes several items, one after the
  // other, and the next item starts while the previous one's output stores
  // drain.  The 4-wave instantiations (two workgroups per CU) run one item.
  constexpr bool PERSIST = NW == 8;
  for (int round = 0; PERSIST || round == 0; ++round) {
  const int item = persistent_item(round, items);
  if (item < 0) break;
  const TileCoord tc = item_coord<CAUSAL, ROWS>(item, qtiles);
  const int q0 = tc.q0;
  const int nlo = (int)blockIdx.y * ks.chunk;  // first key of this launch's chunk
  const int N = min(ks.chunk, Ntot - nlo);     // keys in the chunk
  const int off = off_all - nlo;               // chunk key j visible to row i iff j <= i + off
  const elt* Qh = q + (int64_t)tc.bh * M * D;
  const elt* Kh = k + ((int64_t)tc.bh * Ntot + nlo) * D;
  const elt* Vh = v + ((int64_t)tc.bh * Ntot + nlo) * D;
  OUT* Oh = o + (int64_t)blockIdx.y * ks.o_gstride + (int64_t)tc.bh * M * D;
  float* Lh = lse + (int64_t)blockIdx.y * ks.l_gstride + (int64_t)tc.bh * M;

  const int qrow = q0 + 32 * w + l32;
  const int wq_first = q0 + 32 * w;
  const int wq_last = min(wq_first + 31, M - 1);
  const int n_end = CAUSAL ? min(N, q0 + ROWS + off) : N;
  const int ntiles = n_end > 0 ? (n_end + BN - 1) / BN : 0;
  int w_end = CAUSAL ? min(N, wq_last + 1 + off) : N;
  if (wq_first >= M) w_end = 0;
  const int w_tiles = w_end > 0 ? (w_end + BN - 1) / BN : 0;  // tiles this wave computes
  const int lim = CAUSAL ? min(N, qrow + off + 1) : N;

  vec8 qreg[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    u32x4 raw = {0u, 0u, 0u, 0u};
    if (qrow < M && (!PAD || 16 * kk + 8 * h < D))
      raw = *reinterpret_cast<const u32x4*>(Qh + (int64_t)qrow * D + 16 * kk + 8 * h);
    qreg[kk] = __builtin_bit_cast(vec8, fold_bits(raw, qf));
  }

  const int cp_sub = lane / L::SLOTS;
  const int cp_slot = lane % L::SLOTS;
  // Copy plan: wave w issues the 1 KB copy instructions i = w + NW*b (b < BPW).
  // Instruction i fills LDS rows i*RPB .. i*RPB+RPB-1; lane l writes slot
  // l % SLOTS of row i*RPB + l / SLOTS.  Because NW*RPB rows span whole periods
  // of both swizzles, the logical chunk a lane copies does not depend on b, and
  // one byte offset per matrix serves all of the lane's copies (b only adds
  // NW*RPB rows).
  const int cp_row = w * L::RPB + cp_sub;  // row of the lane's first copy (b = 0)
  const int chunk_k = cp_slot ^ L::swz_k(cp_row);
  const int chunk_v = cp_slot ^ L::swz_v(cp_row);
  const unsigned goff_k = (unsigned)((cp_row * D + 8 * chunk_k) * (int)sizeof(elt));
  const unsigned goff_v = (unsigned)((cp_row * D + 8 * chunk_v) * (int)sizeof(elt));
  constexpr int BSTEP = NW * L::RPB;  // rows between a lane's consecutive copies
  static_assert(BSTEP % 16 == 0, "swizzle period");
  const int lds_w = __builtin_amdgcn_readfirstlane(w * 1024);  // wave-uniform LDS offset
  auto issue = [&](const elt* src, int n0, char* buf, bool is_v) {
    const int chunk = is_v ? chunk_v : chunk_k;
    if (chunk >= L::CPR) return;       // D = 96: slots 12..15 of a row hold no data
    if (PAD && 8 * chunk >= D) return;  // padding: stays zero
    const unsigned goff = is_v ? goff_v : goff_k;
    if (n0 + BN <= N) {
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

  const int krow = swap23(l32);
  int koff[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) koff[kk] = krow * L::ROWB + 16 * ((2 * kk + h) ^ L::swz_k(krow));
  // V^T transpose reads: lane j of a 16-lane group addresses row (8h + 4q + j/4)
  // of the 16-key chunk and 4 columns starting at 32dt + 16*dhalf + 4*(j%4).
  // Rows 4 apart share the swizzle, so q (and the key chunk) are immediates.
  const int g16 = lane >> 4;
  const int dhalf = g16 & 1;
  const int j16 = lane & 15;
  int voff[DT];
  {
    const int row = 8 * h + (j16 >> 2);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const int chunk = 4 * dt + 2 * dhalf + ((j16 & 3) >> 1);
      voff[dt] = row * L::ROWB + 16 * (chunk ^ L::swz_v(row)) + 8 * (j16 & 1);
    }
  }

  f32x16 acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x16{};
  float m_run = -INFINITY;
  float l_run = 0.0f;
  float lr_run = 0.0f;  // the sum O is normalised by (see top_rounding)

  auto s_mfma = [&](f32x16 (&sx)[2], const char* kbuf) {
    sx[0] = f32x16{};
    sx[1] = f32x16{};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const vec8 a0 = *reinterpret_cast<const vec8*>(kbuf + koff[kk]);
      const vec8 a1 = *reinterpret_cast<const vec8*>(kbuf + koff[kk] + 32 * L::ROWB);
      sx[0] = T::mfma(a0, qreg[kk], sx[0]);
      sx[1] = T::mfma(a1, qreg[kk], sx[1]);
    }
  };

  f32x16 sa[2], sb[2];
  // Three-stage variant: step j computes S(j+2) and O += V(j)^T P(j)^T on the
  // MFMA unit while the VALU runs softmax(j+1); the VALU work is spread over
  // all MFMAs of the step.
  // One step in slots of two MFMAs: NSS score slots (S(j+2), rows 0-31 and
  // 32-63 of the K tile for one 16-wide slice of d) then 2*DT PV slots.  The
  // operands of slot s+1 are read from LDS during slot s.  The softmax of
  // tile j+1 (its row max was taken in the previous step) is cut into parts
  // spread over the slots; the last two slots take the row max of S(j+2),
  // whose MFMAs are done by then.  A scheduling fence after each slot keeps
  // every part, MFMA and LDS read in its slot, so the VALU work of one wave
  // runs under the MFMAs of the other wave on its SIMD.
  float mx_next = -INFINITY;  // scaled row max of the next tile to soften
  float lmax_next = -INFINITY;  // the lane's raw score max of that tile
  auto body3 = [&](auto sm_tag, auto s2_tag, f32x16 (&cur)[2], f32x16 (&nxt)[2],
                   const vec8 (&p_use)[4], vec8 (&p_make)[4], const char* kbuf_s2,
                   const char* vbuf, int n2, bool mask_next) __attribute__((always_inline)) {
    constexpr bool SM = decltype(sm_tag)::value;
    constexpr bool S2 = decltype(s2_tag)::value;
    constexpr int NSS = S2 ? KK : 0;
    constexpr int NSL = NSS + 2 * DT;
    constexpr int NPART = 10;                    // softmax parts of tile j+1
    constexpr int NSMSL = S2 ? NSL - 2 : NSL;    // slots that carry them
    auto load_ops = [&](int sl, vec8 (&o)[2]) __attribute__((always_inline)) {
      if (sl < NSS) {
        o[0] = *reinterpret_cast<const vec8*>(kbuf_s2 + koff[sl]);
        o[1] = *reinterpret_cast<const vec8*>(kbuf_s2 + koff[sl] + 32 * L::ROWB);
      } else {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int idx = 2 * (sl - NSS) + u;
          const int cc = idx / DT, dt = idx % DT;
          const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_i16x4*)(vbuf + voff[dt] + 16 * cc * L::ROWB));
          const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_i16x4*)(vbuf + voff[dt] + (16 * cc + 4) * L::ROWB));
          o[u] = __builtin_bit_cast(vec8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
      }
    };
    LazyMax lm{};
    float part_sum[4], corr = 0.0f;
    auto part = [&](int pi) __attribute__((always_inline)) {
      if (pi == 0) {
        lm = lazy_max(mx_next, m_run);
        corr = top_rounding<T>(lmax_next, c, lm.m_use);
        pin(corr);
        pin(lm.alpha);
      } else if (pi < 9) {
        const int g = pi - 1;  // registers 4g .. 4g+3 of the lane's 32 scores
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = g >> 2, r = 4 * (g & 3) + e;
          cur[t][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(cur[t][r], c, -lm.m_use));
        }
        if (g & 1) {  // registers 8cc .. 8cc+7 are done: P operand cc and its sum
          const int cc = g >> 1;
          f32x8 pf;
#pragma unroll
          for (int e = 0; e < 8; ++e) pf[e] = cur[cc >> 1][8 * (cc & 1) + e];
          p_make[cc] = __builtin_convertvector(pf, vec8);
          part_sum[cc] = sum8(pf);
          pin(p_make[cc]);  // computed in this slot, not sunk towards its use
          pin(part_sum[cc]);
        } else {
          pin(cur[g >> 2]);
        }
      } else {
        const float ps = (part_sum[0] + part_sum[1]) + (part_sum[2] + part_sum[3]);
        l_run = __builtin_fmaf(l_run, lm.alpha, ps);
        lr_run = __builtin_fmaf(lr_run, lm.alpha, ps + corr);
        m_run = lm.m_new;
      }
    };
    vec8 op[2][2];
    load_ops(0, op[0]);
    if (S2) {
      nxt[0] = f32x16{};
      nxt[1] = f32x16{};
    }
    float mxa = 0.0f;
#pragma unroll
    for (int sl = 0; sl < NSL; ++sl) {
      if (sl + 1 < NSL) load_ops(sl + 1, op[(sl + 1) & 1]);
      const vec8(&o)[2] = op[sl & 1];
      if (sl < NSS) {
        nxt[0] = T::mfma(o[0], qreg[sl], nxt[0]);
        nxt[1] = T::mfma(o[1], qreg[sl], nxt[1]);
      } else {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int idx = 2 * (sl - NSS) + u;
          acc[idx % DT] = T::mfma(o[u], p_use[idx / DT], acc[idx % DT]);
        }
      }
      if (SM && sl < NSMSL) {
#pragma unroll
        for (int pi = (sl * NPART + NSMSL - 1) / NSMSL;
             pi < ((sl + 1) * NPART + NSMSL - 1) / NSMSL; ++pi)
          part(pi);
      }
      if (S2 && sl == NSL - 2) {
        if (mask_next) {  // rare: diagonal or N tail; a real branch, not predicated
          asm volatile("" ::: "memory");
          apply_mask<2>(nxt, n2, h, lim);
        }
        mxa = max_tree16(nxt[0]);
        pin(mxa);
      }
      if (S2 && sl == NSL - 1) {
        lmax_next = fmaxf(mxa, max_tree16(nxt[1]));
        mx_next = pair_max(lmax_next) * c;
        pin(mx_next);
        pin(lmax_next);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (SM) {
      pin(l_run);
      pin(lr_run);
    }
    if (SM && lm.grow) {  // rare: some row's max moved by more than the slack
      asm volatile("" ::: "memory");
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) acc[dt] *= lm.alpha;
    }
  };
  auto needs_mask = [&](int n0) { return (n0 + BN > N) || (CAUSAL && n0 + BN - 1 > wq_first + off); };
  auto step3 = [&](int j, f32x16 (&cur)[2], f32x16 (&nxt)[2], const vec8 (&p_use)[4],
                   vec8 (&p_make)[4], const char* kbuf_s2, const char* vbuf, char* kbuf_load,
                   char* vbuf_load) __attribute__((always_inline)) {
    if (j + 3 < ntiles) issue(Kh, (j + 3) * BN, kbuf_load, false);
    if (j + 1 < ntiles) issue(Vh, (j + 1) * BN, vbuf_load, true);
    if (j < w_tiles) {
      const int n2 = (j + 2) * BN;
      using T0 = std::integral_constant<bool, false>;
      using T1 = std::integral_constant<bool, true>;
      if (j + 2 < w_tiles)
        body3(T1{}, T1{}, cur, nxt, p_use, p_make, kbuf_s2, vbuf, n2, needs_mask(n2));
      else if (j + 1 < w_tiles)
        body3(T1{}, T0{}, cur, nxt, p_use, p_make, kbuf_s2, vbuf, n2, false);
      else
        body3(T0{}, T0{}, cur, nxt, p_use, p_make, kbuf_s2, vbuf, n2, false);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  };
  // D = 64: two tiles in flight.  Step j issues the score MFMAs of tile j+1
  // interleaved (scheduling hints) with softmax(j)'s VALU work, then the PV
  // MFMAs of tile j; K runs one tile ahead of V.  At D = 64 the VALU work per
  // MFMA is twice that of D = 128 and, with two workgroups per CU whose waves
  // are not in step, this measured faster than the three-tile slots.
  auto body2 = [&](auto mask_tag, auto next_tag, f32x16 (&cur)[2], f32x16 (&nxt)[2],
                   const char* kbuf_next, const char* vbuf, int n0) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    constexpr bool NEXT = decltype(next_tag)::value;
    if (NEXT) s_mfma(nxt, kbuf_next);
    if (MASK) apply_mask<2>(cur, n0, h, lim);
    const SoftmaxStep st = softmax_update_lazy<T>(cur, c, m_run, l_run, lr_run);
    vec8 pb2[4];
    pack_p<T>(cur, pb2);
    if (NEXT) {
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);  // 4 LDS reads
#pragma unroll
      for (int i = 0; i < 2 * KK; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // 1 MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 10, 0);  // 10 VALU
        if (i < 2 * KK - 4) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // next read
      }
    }
    if (st.rescale) {  // rare: some row's max moved by more than the slack
      asm volatile("" ::: "memory");
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) acc[dt] *= st.alpha;
    }
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4*)(vbuf + voff[dt] + 16 * cc * L::ROWB));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4*)(vbuf + voff[dt] + (16 * cc + 4) * L::ROWB));
        const vec8 a = __builtin_bit_cast(vec8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        acc[dt] = T::mfma(a, pb2[cc], acc[dt]);
      }
    }
    // V^T operand reads run two MFMAs ahead of the PV MFMAs.
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 1);
#pragma unroll
    for (int i = 0; i < 4 * DT; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
      if (i < 4 * DT - 2) __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
    }
  };
  auto step2 = [&](int j, f32x16 (&cur)[2], f32x16 (&nxt)[2], const char* kbuf_next,
                   const char* vbuf, char* kbuf_load, char* vbuf_load) __attribute__((always_inline)) {
    if (j + 2 < ntiles) issue(Kh, (j + 2) * BN, kbuf_load, false);
    if (j + 1 < ntiles) issue(Vh, (j + 1) * BN, vbuf_load, true);
    if (j < w_tiles) {
      const int n0 = j * BN;
      const bool next = j + 1 < w_tiles;
      using T0 = std::integral_constant<bool, false>;
      using T1 = std::integral_constant<bool, true>;
      if (!needs_mask(n0)) {
        if (next) body2(T0{}, T1{}, cur, nxt, kbuf_next, vbuf, n0);
        else body2(T0{}, T0{}, cur, nxt, kbuf_next, vbuf, n0);
      } else {
        if (next) body2(T1{}, T1{}, cur, nxt, kbuf_next, vbuf, n0);
        else body2(T1{}, T0{}, cur, nxt, kbuf_next, vbuf, n0);
      }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  };

  if constexpr (DP == 64) {
    if (ntiles > 0) {
      issue(Kh, 0, kb0, false);
      issue(Vh, 0, vb0, true);
    }
    if (ntiles > 1) issue(Kh, BN, kb1, false);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (0 < w_tiles) s_mfma(sa, kb0);
    __syncthreads();  // every wave is done reading K(0) before K(2) overwrites it
    for (int j = 0; j < ntiles; j += 2) {
      step2(j, sa, sb, kb1, vb0, kb0, vb1);
      if (j + 1 >= ntiles) break;
      step2(j + 1, sb, sa, kb0, vb1, kb1, vb0);
    }
  } else {
    vec8 pa[4], pb[4];
    if (ntiles > 0) {
      issue(Kh, 0, kb0, false);
      issue(Vh, 0, vb0, true);
    }
    if (ntiles > 1) issue(Kh, BN, kb1, false);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (0 < w_tiles) s_mfma(sa, kb0);
    if (1 < w_tiles) s_mfma(sb, kb1);
    __syncthreads();  // every wave is done reading K(0) before K(2) overwrites it
    if (ntiles > 2) issue(Kh, 2 * BN, kb0, false);
    if (0 < w_tiles) {
      if (needs_mask(0)) apply_mask<2>(sa, 0, h, lim);
      (void)softmax_update_lazy<T>(sa, c, m_run, l_run, lr_run);  // acc is still zero
      pack_p<T>(sa, pa);
    }
    if (1 < w_tiles) {
      if (needs_mask(BN)) apply_mask<2>(sb, BN, h, lim);
      lmax_next = max_tree<2>(sb);
      mx_next = pair_max(lmax_next) * c;
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    for (int j = 0; j < ntiles; j += 2) {
      step3(j, sb, sa, pa, pb, kb0, vb0, kb1, vb1);
      if (j + 1 >= ntiles) break;
      step3(j + 1, sa, sb, pb, pa, kb1, vb1, kb0, vb0);
    }
  }

  const float l_tot = pair_sum(l_run);  // LSE
  const float lr_tot = pair_sum(lr_run);
  const float inv = lr_tot > 0.0f ? 1.0f / lr_tot : 0.0f;
  if (qrow < M) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * dt + 8 * g + 4 * h;
        OUT y[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = (OUT)(acc[dt][4 * g + e] * inv);
        if (!PAD || d0 < D) store4<OUT>(Oh + (int64_t)qrow * D + d0, y);
      }
    if (h == 0)
      Lh[qrow] = l_tot > 0.0f ? LN2F * (m_run + __builtin_amdgcn_logf(l_tot)) : -INFINITY;
  }
  }  // persistent loop
}

// ---------------------------------------------------------------------------
// fp32 kernel: same structure on v_mfma_f32_32x32x2f32 with P kept in fp32.
// 32-key tiles; K rows in LDS at an odd stride (conflict-free column reads),
// V row-major (the V^T operand of a 2-key step is one row of 32 columns).
template <int DP, bool CAUSAL, bool DFULL>
__global__ __launch_bounds__(NTHREADS, 2) void fa_fwd_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    float* __restrict__ o, float* __restrict__ lse, int M, int Ntot, int D, int qtiles, float c,
    KeySplit ks, QFold qf) {
  constexpr int KSTR = DP + 1;
  constexpr int VSTR = DP + 4;
  constexpr int K_ELEMS = BN32 * KSTR;
  constexpr int V_ELEMS = BN32 * VSTR;
  constexpr int STAGE = K_ELEMS + V_ELEMS;
  constexpr int CH = DP / 4;                    // 16-byte chunks per row
  constexpr int LD = (BN32 * CH + NTHREADS - 1) / NTHREADS;
  constexpr int DT = DP / 32;
  constexpr int KS = DP / 2;                    // k-steps of S^T

  __shared__ __attribute__((aligned(16))) float smem[2 * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int h = lane >> 5;
  const int l32 = lane & 31;

  const TileCoord tc = tile_coord<CAUSAL>(qtiles);
  const int q0 = tc.q0;
  const int nlo = (int)blockIdx.y * ks.chunk;  // first key of this launch's chunk
  const int N = min(ks.chunk, Ntot - nlo);     // keys in the chunk
  const float* Qh = q + (int64_t)tc.bh * M * D;
  const float* Kh = k + ((int64_t)tc.bh * Ntot + nlo) * D;
  const float* Vh = v + ((int64_t)tc.bh * Ntot + nlo) * D;
  float* Oh = o + (int64_t)blockIdx.y * ks.o_gstride + (int64_t)tc.bh * M * D;
  float* Lh = lse + (int64_t)blockIdx.y * ks.l_gstride + (int64_t)tc.bh * M;

  const int off = Ntot - M - nlo;
  const int qrow = q0 + 32 * w + l32;
  const int wq_first = q0 + 32 * w;
  const int wq_last = min(wq_first + 31, M - 1);
  const int n_end = CAUSAL ? min(N, q0 + BM + off) : N;
  const int ntiles = n_end > 0 ? (n_end + BN32 - 1) / BN32 : 0;
  int w_end = CAUSAL ? min(N, wq_last + 1 + off) : N;
  if (wq_first >= M) w_end = 0;
  const int lim = CAUSAL ? min(N, qrow + off + 1) : N;

  float qreg[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    const int d = 2 * s + h;
    qreg[s] = fold_f32((qrow < M && d < D) ? Qh[(int64_t)qrow * D + d] : 0.0f, qf);
  }

  f32x16 acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x16{};
  float m_run = -INFINITY;
  float l_run = 0.0f;

  float4 kr[LD], vr[LD];
  auto load_tile = [&](int n0) {
#pragma unroll
    for (int i = 0; i < LD; ++i) {
      const int ci = tid + NTHREADS * i;
      const int row = ci / CH;
      const int col = (ci - row * CH) * 4;
      const int key = n0 + row;
      float4 a = make_float4(0.f, 0.f, 0.f, 0.f), b = a;
      if (ci < BN32 * CH && key < N) {
        if (DFULL) {
          a = *reinterpret_cast<const float4*>(Kh + (int64_t)key * D + col);
          b = *reinterpret_cast<const float4*>(Vh + (int64_t)key * D + col);
        } else {
          const float* kp = Kh + (int64_t)key * D;
          const float* vp = Vh + (int64_t)key * D;
          a.x = col + 0 < D ? kp[col + 0] : 0.f;
          a.y = col + 1 < D ? kp[col + 1] : 0.f;
          a.z = col + 2 < D ? kp[col + 2] : 0.f;
          a.w = col + 3 < D ? kp[col + 3] : 0.f;
          b.x = col + 0 < D ? vp[col + 0] : 0.f;
          b.y = col + 1 < D ? vp[col + 1] : 0.f;
          b.z = col + 2 < D ? vp[col + 2] : 0.f;
          b.w = col + 3 < D ? vp[col + 3] : 0.f;
        }
      }
      kr[i] = a;
      vr[i] = b;
    }
  };
  auto store_tile = [&](int stage) {
    float* Ks = smem + stage * STAGE;
    float* Vs = Ks + K_ELEMS;
#pragma unroll
    for (int i = 0; i < LD; ++i) {
      const int ci = tid + NTHREADS * i;
      if (ci < BN32 * CH) {
        const int row = ci / CH;
        const int col = (ci - row * CH) * 4;
        float* kp = Ks + row * KSTR + col;
        kp[0] = kr[i].x;
        kp[1] = kr[i].y;
        kp[2] = kr[i].z;
        kp[3] = kr[i].w;
        *reinterpret_cast<float4*>(Vs + row * VSTR + col) = vr[i];
      }
    }
  };

  if (ntiles > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();

  const int krow = swap23(l32);
  for (int j = 0; j < ntiles; ++j) {
    const int n0 = j * BN32;
    const bool more = j + 1 < ntiles;
    if (more) load_tile(n0 + BN32);
    if (n0 < w_end) {
      const float* Ks = smem + (j & 1) * STAGE;
      const float* Vs = Ks + K_ELEMS;
      f32x16 s[1] = {f32x16{}};
#pragma unroll
      for (int st = 0; st < KS; ++st)
        s[0] = __builtin_amdgcn_mfma_f32_32x32x2f32(Ks[krow * KSTR + 2 * st + h], qreg[st], s[0],
                                                    0, 0, 0);
      const bool need_mask = (n0 + BN32 > N) || (CAUSAL && n0 + BN32 - 1 > wq_first + off);
      if (need_mask) apply_mask<1>(s, n0, h, lim);
      const SoftmaxStep st = softmax_update<1>(s, c, m_run, l_run);
      if (st.rescale) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) acc[dt] *= st.alpha;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = key_of_reg(r, h);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
          acc[dt] = __builtin_amdgcn_mfma_f32_32x32x2f32(Vs[key * VSTR + 32 * dt + l32], s[0][r],
                                                         acc[dt], 0, 0, 0);
      }
    }
    if (more) store_tile((j + 1) & 1);
    __syncthreads();
  }

  const float l_tot = pair_sum(l_run);
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  if (qrow < M) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * dt + 8 * g + 4 * h;
        if (DFULL) {
          float4 y = make_float4(acc[dt][4 * g] * inv, acc[dt][4 * g + 1] * inv,
                                 acc[dt][4 * g + 2] * inv, acc[dt][4 * g + 3] * inv);
          *reinterpret_cast<float4*>(Oh + (int64_t)qrow * D + d0) = y;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (d0 + e < D) Oh[(int64_t)qrow * D + d0 + e] = acc[dt][4 * g + e] * inv;
        }
      }
    if (h == 0)
      Lh[qrow] = l_tot > 0.0f ? LN2F * (m_run + __builtin_amdgcn_logf(l_tot)) : -INFINITY;
  }
}

// ---------------------------------------------------------------------------
// fp32 forward for grids far too small to fill the GPU (D <= 64): the four
// waves of a workgroup share its 32 query rows and split every 128-key step
// between them (wave w takes keys 32w..32w+31 of the step), each running the
// recurrence of fa_fwd_f32_kernel over its keys.  At the end the partial
// results are combined through LDS by the concatenation algebra of "Module 08:
// FlashAttention and Memory-Efficient Kernels" ("Tiling and the online
// softmax"): with m = max_w m_w and a_w = 2^(m_w - m) (base-2 scaled units),
//   l = sum_w a_w l_w,   O = sum_w a_w acc_w / l,   LSE = ln2 (m + log2 l).
// A wave that saw no key has m_w = -inf and weight 0; a row that sees no key
// at all keeps O = 0 and LSE = -inf.  Four times the workgroups of the plain
// kernel for the same problem, each with a quarter of the keys.
template <int DP, bool CAUSAL, bool DFULL>
__global__ __launch_bounds__(NTHREADS, 1) void fa_fwd_f32_ksplit_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    float* __restrict__ o, float* __restrict__ lse, int M, int N, int D, int qtiles, float c,
    QFold qf) {
  constexpr int ROWS = 32;
  constexpr int KEYS = 4 * BN32;                // keys per step (all four waves)
  constexpr int KSTR = DP + 1;
  constexpr int VSTR = DP + 4;
  constexpr int K_ELEMS = KEYS * KSTR;
  constexpr int V_ELEMS = KEYS * VSTR;
  constexpr int STAGE = K_ELEMS + V_ELEMS;
  constexpr int CH = DP / 4;                    // 16-byte chunks per row
  constexpr int LD = (KEYS * CH + NTHREADS - 1) / NTHREADS;
  constexpr int DT = DP / 32;
  constexpr int KS = DP / 2;                    // k-steps of S^T
  static_assert(4 * ROWS * DP + 8 * ROWS <= 2 * STAGE, "merge buffers fit in the stages");

  __shared__ __attribute__((aligned(16))) float smem[2 * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int h = lane >> 5;
  const int l32 = lane & 31;

  const TileCoord tc = tile_coord<CAUSAL, ROWS>(qtiles);
  const int q0 = tc.q0;
  const float* Qh = q + (int64_t)tc.bh * M * D;
  const float* Kh = k + (int64_t)tc.bh * N * D;
  const float* Vh = v + (int64_t)tc.bh * N * D;
  float* Oh = o + (int64_t)tc.bh * M * D;
  float* Lh = lse + (int64_t)tc.bh * M;

  const int off = N - M;
  const int qrow = q0 + l32;
  const int q_last = min(q0 + ROWS - 1, M - 1);
  // keys any row of the workgroup sees
  const int w_end = CAUSAL ? min(N, q_last + 1 + off) : N;
  const int ntiles = w_end > 0 ? (w_end + KEYS - 1) / KEYS : 0;
  const int lim = CAUSAL ? min(N, qrow + off + 1) : N;

  float qreg[KS];
#pragma unroll
  for (int st = 0; st < KS; ++st) {
    const int d = 2 * st + h;
    qreg[st] = fold_f32((qrow < M && d < D) ? Qh[(int64_t)qrow * D + d] : 0.0f, qf);
  }

  f32x16 acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x16{};
  float m_run = -INFINITY;
  float l_run = 0.0f;

  float4 kr[LD], vr[LD];
  auto load_tile = [&](int n0) {
#pragma unroll
    for (int i = 0; i < LD; ++i) {
      const int ci = tid + NTHREADS * i;
      const int row = ci / CH;
      const int col = (ci - row * CH) * 4;
      const int key = n0 + row;
      float4 a = make_float4(0.f, 0.f, 0.f, 0.f), b = a;
      if (ci < KEYS * CH && key < N) {
        if (DFULL) {
          a = *reinterpret_cast<const float4*>(Kh + (int64_t)key * D + col);
          b = *reinterpret_cast<const float4*>(Vh + (int64_t)key * D + col);
        } else {
          const float* kp = Kh + (int64_t)key * D;
          const float* vp = Vh + (int64_t)key * D;
          a.x = col + 0 < D ? kp[col + 0] : 0.f;
          a.y = col + 1 < D ? kp[col + 1] : 0.f;
          a.z = col + 2 < D ? kp[col + 2] : 0.f;
          a.w = col + 3 < D ? kp[col + 3] : 0.f;
          b.x = col + 0 < D ? vp[col + 0] : 0.f;
          b.y = col + 1 < D ? vp[col + 1] : 0.f;
          b.z = col + 2 < D ? vp[col + 2] : 0.f;
          b.w = col + 3 < D ? vp[col + 3] : 0.f;
        }
      }
      kr[i] = a;
      vr[i] = b;
    }
  };
  auto store_tile = [&](int stage) {
    float* Ks = smem + stage * STAGE;
    float* Vs = Ks + K_ELEMS;
#pragma unroll
    for (int i = 0; i < LD; ++i) {
      const int ci = tid + NTHREADS * i;
      if (ci < KEYS * CH) {
        const int row = ci / CH;
        const int col = (ci - row * CH) * 4;
        float* kp = Ks + row * KSTR + col;
        kp[0] = kr[i].x;
        kp[1] = kr[i].y;
        kp[2] = kr[i].z;
        kp[3] = kr[i].w;
        *reinterpret_cast<float4*>(Vs + row * VSTR + col) = vr[i];
      }
    }
  };

  if (ntiles > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();

  const int krow = swap23(l32);
  for (int j = 0; j < ntiles; ++j) {
    const int n0 = j * KEYS;
    const bool more = j + 1 < ntiles;
    if (more) load_tile(n0 + KEYS);
    const int nw = n0 + BN32 * w;  // this wave's first key
    if (nw < w_end) {
      const float* Ks = smem + (j & 1) * STAGE + BN32 * w * KSTR;
      const float* Vs = smem + (j & 1) * STAGE + K_ELEMS + BN32 * w * VSTR;
      f32x16 s[1] = {f32x16{}};
#pragma unroll
      for (int st = 0; st < KS; ++st)
        s[0] = __builtin_amdgcn_mfma_f32_32x32x2f32(Ks[krow * KSTR + 2 * st + h], qreg[st], s[0],
                                                    0, 0, 0);
      const bool need_mask = (nw + BN32 > N) || (CAUSAL && nw + BN32 - 1 > q0 + off);
      if (need_mask) apply_mask<1>(s, nw, h, lim);
      const SoftmaxStep st = softmax_update<1>(s, c, m_run, l_run);
      if (st.rescale) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) acc[dt] *= st.alpha;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = key_of_reg(r, h);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
          acc[dt] = __builtin_amdgcn_mfma_f32_32x32x2f32(Vs[key * VSTR + 32 * dt + l32], s[0][r],
                                                         acc[dt], 0, 0, 0);
      }
    }
    if (more) store_tile((j + 1) & 1);
    __syncthreads();
  }

  // Merge the four waves' partial results (the stage buffers are free now).
  float* part = smem;                    // [4][ROWS][DP] accumulators, scaled by a_w
  float* mst = smem + 4 * ROWS * DP;     // [4][ROWS] maxima
  float* lst = mst + 4 * ROWS;           // [4][ROWS] sums
  const float l_w = pair_sum(l_run);
  if (h == 0) {
    mst[w * ROWS + l32] = m_run;
    lst[w * ROWS + l32] = l_w;
  }
  __syncthreads();
  float m_all = -INFINITY;
#pragma unroll
  for (int u = 0; u < 4; ++u) m_all = fmaxf(m_all, mst[u * ROWS + l32]);
  const float a_w = m_run == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_run - m_all);
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int d = 32 * dt + 8 * g + 4 * h + e;
        part[(w * ROWS + l32) * DP + d] = acc[dt][4 * g + e] * a_w;
      }
  __syncthreads();
  // Thread t combines row t / 8, features 8 (t % 8) .. + 7 (DP / 8 at a time).
  {
    constexpr int PER = DP / 8;
    const int row = tid >> 3;
    const int d0 = (tid & 7) * PER;
    float mr = -INFINITY;
#pragma unroll
    for (int u = 0; u < 4; ++u) mr = fmaxf(mr, mst[u * ROWS + row]);
    float l_tot = 0.0f;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float mu = mst[u * ROWS + row];
      l_tot += mu == -INFINITY ? 0.0f : lst[u * ROWS + row] * __builtin_amdgcn_exp2f(mu - mr);
    }
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    const int grow = q0 + row;
    if (grow < M) {
#pragma unroll
      for (int e = 0; e < PER; ++e) {
        const int d = d0 + e;
        const float y = (part[(0 * ROWS + row) * DP + d] + part[(1 * ROWS + row) * DP + d] +
                         part[(2 * ROWS + row) * DP + d] + part[(3 * ROWS + row) * DP + d]) *
                        inv;
        if (DFULL || d < D) Oh[(int64_t)grow * D + d] = y;
      }
      if ((tid & 7) == 0)
        Lh[grow] = l_tot > 0.0f ? LN2F * (mr + __builtin_amdgcn_logf(l_tot)) : -INFINITY;
    }
  }
}

// ---------------------------------------------------------------------------
// Merge of split-KV partial results: the concatenation algebra of "Module 08:
// FlashAttention and Memory-Efficient Kernels" ("Tiling and the online
// softmax": the softmax of a concatenation follows from the maxima and sums of
// its pieces).  Chunk g left a normalised fp32 O_g and LSE_g per row; then
//   LSE = m + ln sum_g exp(LSE_g - m)  (m = max_g LSE_g),
//   O   = sum_g exp(LSE_g - m) O_g / sum_g exp(LSE_g - m).
// A chunk a row cannot see has LSE_g = -inf and weight 0; a row that sees no
// key at all keeps O = 0 and LSE = -inf.  One thread per (row, 4 features).
template <class OUT>
__global__ __launch_bounds__(NTHREADS) void fa_merge_kernel(
    const float* __restrict__ opart, const float* __restrict__ lpart, OUT* __restrict__ o,
    float* __restrict__ lse, int64_t rows, int D, int G, int64_t o_gstride, int64_t l_gstride) {
  constexpr float LOG2E = 1.44269504088896340736f;
  const int groups = (D + 3) / 4;
  const int64_t total = rows * groups;
  for (int64_t t = (int64_t)blockIdx.x * NTHREADS + threadIdx.x; t < total;
       t += (int64_t)gridDim.x * NTHREADS) {
    const int64_t row = t / groups;
    const int d0 = 4 * (int)(t - row * groups);
    float m = -INFINITY;
    for (int g = 0; g < G; ++g) m = fmaxf(m, lpart[g * l_gstride + row]);
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    float tot = 0.0f;
    if (m != -INFINITY) {
      for (int g = 0; g < G; ++g) {
        const float wg = __builtin_amdgcn_exp2f((lpart[g * l_gstride + row] - m) * LOG2E);
        tot += wg;
        const float* og = opart + g * o_gstride + row * D + d0;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (d0 + e < D) acc[e] = __builtin_fmaf(wg, og[e], acc[e]);
      }
    }
    const float inv = tot > 0.0f ? 1.0f / tot : 0.0f;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (d0 + e < D) o[row * D + d0 + e] = (OUT)(acc[e] * inv);
    if (d0 == 0) lse[row] = tot > 0.0f ? m + LN2F * __builtin_amdgcn_logf(tot) : -INFINITY;
  }
}

// ---------------------------------------------------------------------------
// Host dispatch.  Every launch returns its own status (see `launch`).

struct Launch {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int M, N, D, qtiles;
  float c;    // positive exponent constant (see fold_scale)
  QFold qf;   // sign fold of the Q operand
  dim3 grid;
  int64_t BH;
  hipStream_t stream;
  int dev;       // device of `stream`
  bool generic;  // force the general kernel (register-staged tiles)
};

template <class T, int DP, bool CAUSAL>
hipError_t launch_lp(const Launch& a) {
  using elt = typename T::elt;
  const KeySplit ks{a.N, 0, 0};
  if (a.D == DP)
    return launch(fa_fwd_lp_kernel<T, DP, CAUSAL, true, elt>, a.grid, dim3(NTHREADS), a.stream,
                  (const elt*)a.q, (const elt*)a.k, (const elt*)a.v, (elt*)a.o, a.lse, a.M, a.N,
                  a.D, a.qtiles, a.c, ks, a.qf);
  return launch(fa_fwd_lp_kernel<T, DP, CAUSAL, false, elt>, a.grid, dim3(NTHREADS), a.stream,
                (const elt*)a.q, (const elt*)a.k, (const elt*)a.v, (elt*)a.o, a.lse, a.M, a.N, a.D,
                a.qtiles, a.c, ks, a.qf);
}

template <int DP, bool CAUSAL>
hipError_t launch_f32(const Launch& a) {
  const KeySplit ks{a.N, 0, 0};
  if (a.D == DP)
    return launch(fa_fwd_f32_kernel<DP, CAUSAL, true>, a.grid, dim3(NTHREADS), a.stream,
                  (const float*)a.q, (const float*)a.k, (const float*)a.v, (float*)a.o, a.lse, a.M,
                  a.N, a.D, a.qtiles, a.c, ks, a.qf);
  return launch(fa_fwd_f32_kernel<DP, CAUSAL, false>, a.grid, dim3(NTHREADS), a.stream,
                (const float*)a.q, (const float*)a.k, (const float*)a.v, (float*)a.o, a.lse, a.M,
                a.N, a.D, a.qtiles, a.c, ks, a.qf);
}

// Waves per workgroup of the fast path (32 query rows each).  At D = 96 and 128
// a 256-row workgroup halves the K/V copies per FLOP against 128 rows and
// measured faster; at D = 64 the 128-row workgroup (two per CU) is faster.
template <int DP>
constexpr int fast_waves() { return DP == 64 ? 4 : 8; }
// Multiples of 8 that are not fast sizes run the fast kernel of the next size
// up, zero-padded, except D = 32: there the general kernel's 32-wide
// instantiation does half the padded kernel's MFMA work and measured faster
// (at D = 8, 16 and 24 the padded kernel is 1.5-1.8x faster than the general one).
constexpr bool pad_to_fast(int64_t D) { return D % 8 == 0 && D != 32; }

template <class T, int DP, bool CAUSAL, int NW, bool PAD>
hipError_t launch_lp_fast_nw(const Launch& a) {
  using elt = typename T::elt;
  const int off = CAUSAL ? a.N - a.M : a.N;
  const int rows = 32 * NW;
  const int qtiles = (a.M + rows - 1) / rows;
  const int items = (int)(a.BH * qtiles);
  // One workgroup per CU (persistent) where a workgroup fills a CU, else one
  // per item.  Every XCD range needs a workgroup of its own: at least NXCD.
  // Only the 8-wave kernel loops over items; a 4-wave launch has one per item.
  int slots = 0;
  if constexpr (NW == 8)
    slots = persistent_workgroups<fa_fwd_lp_pipe_kernel<T, DP, NW, elt, PAD>>(64 * NW, a.dev);
  const int P = slots >= NXCD && slots < items ? slots : items;
  const KeySplit ks{a.N, 0, 0};
  return launch(fa_fwd_lp_pipe_kernel<T, DP, NW, elt, PAD>, dim3((unsigned)P), dim3(64 * NW),
                a.stream, (const elt*)a.q, (const elt*)a.k, (const elt*)a.v, (elt*)a.o, a.lse, a.M,
                a.N, off, qtiles, items, a.c, ks, a.qf, (int)a.D);
}

// At D = 96 and 128, when even 128-row workgroups (twice as many) leave a CU
// for each, the grid runs on those: the same work on twice the CUs.  (Where
// the doubled grid would put two workgroups on some CUs it measured slower.)
template <class T, int DP, bool CAUSAL, bool PAD>
hipError_t launch_lp_fast(const Launch& a) {
  constexpr int NW = fast_waves<DP>();
  if constexpr (NW == 8) {
    const int64_t wide = a.BH * ((a.M + 32 * NW - 1) / (32 * NW));
    const int cus = device_cus(a.dev);
    if (cus > 0 && a.BH * ((a.M + 127) / 128) <= cus && wide < cus)
      return launch_lp_fast_nw<T, DP, CAUSAL, 4, PAD>(a);
  }
  return launch_lp_fast_nw<T, DP, CAUSAL, NW, PAD>(a);
}

// Split-KV partials on the fast path (fp32 outputs into the workspace).
template <class T, int DP, bool CAUSAL, bool PAD>
hipError_t launch_lp_fast_split(const Launch& a, const KeySplit& ks, int G, float* opart,
                                float* lpart) {
  using elt = typename T::elt;
  constexpr int NW = fast_waves<DP>();
  const int off = CAUSAL ? a.N - a.M : a.N;
  const int rows = 32 * NW;
  const int qtiles = (a.M + rows - 1) / rows;
  const int items = (int)(a.BH * qtiles);  // one workgroup per item and chunk
  const dim3 grid((unsigned)items, (unsigned)G);
  return launch(fa_fwd_lp_pipe_kernel<T, DP, NW, float, PAD>, grid, dim3(64 * NW), a.stream,
                (const elt*)a.q, (const elt*)a.k, (const elt*)a.v, opart, lpart, a.M, a.N, off,
                qtiles, items, a.c, ks, a.qf, (int)a.D);
}

template <class T, bool CAUSAL>
hipError_t dispatch_lp(const Launch& a) {
  if (a.N > 0 && !a.generic) {
    if (a.D == 128) return launch_lp_fast<T, 128, CAUSAL, false>(a);
    if (a.D == 96) return launch_lp_fast<T, 96, CAUSAL, false>(a);
    if (a.D == 64) return launch_lp_fast<T, 64, CAUSAL, false>(a);
    if (pad_to_fast(a.D)) {  // zero-padded to the next fast size
      if (a.D < 64) return launch_lp_fast<T, 64, CAUSAL, true>(a);
      if (a.D < 96) return launch_lp_fast<T, 96, CAUSAL, true>(a);
      return launch_lp_fast<T, 128, CAUSAL, true>(a);
    }
  }
  if (a.D <= 32) return launch_lp<T, 32, CAUSAL>(a);
  if (a.D <= 64) return launch_lp<T, 64, CAUSAL>(a);
  if (a.D <= 96) return launch_lp<T, 96, CAUSAL>(a);
  return launch_lp<T, 128, CAUSAL>(a);
}

// fp32 with D <= 64 on a grid that would leave most of the GPU idle: split
// each workgroup's keys over its four waves (four times the workgroups).
template <int DP, bool CAUSAL>
hipError_t launch_f32_ksplit(const Launch& a) {
  const int qtiles = (a.M + 31) / 32;
  const dim3 grid((unsigned)(a.BH * qtiles));
  if (a.D == DP)
    return launch(fa_fwd_f32_ksplit_kernel<DP, CAUSAL, true>, grid, dim3(NTHREADS), a.stream,
                  (const float*)a.q, (const float*)a.k, (const float*)a.v, (float*)a.o, a.lse, a.M,
                  a.N, a.D, qtiles, a.c, a.qf);
  return launch(fa_fwd_f32_ksplit_kernel<DP, CAUSAL, false>, grid, dim3(NTHREADS), a.stream,
                (const float*)a.q, (const float*)a.k, (const float*)a.v, (float*)a.o, a.lse, a.M,
                a.N, a.D, qtiles, a.c, a.qf);
}

template <bool CAUSAL>
hipError_t dispatch_f32(const Launch& a) {
  const int cus = device_cus(a.dev);
  if (!a.generic && a.N > 0 && a.D <= 64 && cus > 0 && 2 * (int64_t)a.grid.x < cus) {
    if (a.D <= 32) return launch_f32_ksplit<32, CAUSAL>(a);
    return launch_f32_ksplit<64, CAUSAL>(a);
  }
  if (a.D <= 32) return launch_f32<32, CAUSAL>(a);
  if (a.D <= 64) return launch_f32<64, CAUSAL>(a);
  if (a.D <= 96) return launch_f32<96, CAUSAL>(a);
  return launch_f32<128, CAUSAL>(a);
}

// Split-KV partials: chunk g of every head's keys into the fp32 workspace.
template <class T, int DP, bool CAUSAL>
hipError_t launch_lp_split(const Launch& a, const KeySplit& ks, int G, float* opart,
                           float* lpart) {
  using elt = typename T::elt;
  const dim3 grid(a.grid.x, (unsigned)G);
  if (a.D == DP)
    return launch(fa_fwd_lp_kernel<T, DP, CAUSAL, true, float>, grid, dim3(NTHREADS), a.stream,
                  (const elt*)a.q, (const elt*)a.k, (const elt*)a.v, opart, lpart, a.M, a.N, a.D,
                  a.qtiles, a.c, ks, a.qf);
  return launch(fa_fwd_lp_kernel<T, DP, CAUSAL, false, float>, grid, dim3(NTHREADS), a.stream,
                (const elt*)a.q, (const elt*)a.k, (const elt*)a.v, opart, lpart, a.M, a.N, a.D,
                a.qtiles, a.c, ks, a.qf);
}
template <int DP, bool CAUSAL>
hipError_t launch_f32_split(const Launch& a, const KeySplit& ks, int G, float* opart,
                            float* lpart) {
  const dim3 grid(a.grid.x, (unsigned)G);
  if (a.D == DP)
    return launch(fa_fwd_f32_kernel<DP, CAUSAL, true>, grid, dim3(NTHREADS), a.stream,
                  (const float*)a.q, (const float*)a.k, (const float*)a.v, opart, lpart, a.M, a.N,
                  a.D, a.qtiles, a.c, ks, a.qf);
  return launch(fa_fwd_f32_kernel<DP, CAUSAL, false>, grid, dim3(NTHREADS), a.stream,
                (const float*)a.q, (const float*)a.k, (const float*)a.v, opart, lpart, a.M, a.N,
                a.D, a.qtiles, a.c, ks, a.qf);
}
template <class T, bool CAUSAL>
hipError_t dispatch_lp_split(const Launch& a, const KeySplit& ks, int G, float* op, float* lp) {
  if (a.D == 128) return launch_lp_fast_split<T, 128, CAUSAL, false>(a, ks, G, op, lp);
  if (a.D == 96) return launch_lp_fast_split<T, 96, CAUSAL, false>(a, ks, G, op, lp);
  if (a.D == 64) return launch_lp_fast_split<T, 64, CAUSAL, false>(a, ks, G, op, lp);
  if (pad_to_fast(a.D)) {  // zero-padded to the next fast size
    if (a.D < 64) return launch_lp_fast_split<T, 64, CAUSAL, true>(a, ks, G, op, lp);
    if (a.D < 96) return launch_lp_fast_split<T, 96, CAUSAL, true>(a, ks, G, op, lp);
    return launch_lp_fast_split<T, 128, CAUSAL, true>(a, ks, G, op, lp);
  }
  if (a.D <= 32) return launch_lp_split<T, 32, CAUSAL>(a, ks, G, op, lp);
  if (a.D <= 64) return launch_lp_split<T, 64, CAUSAL>(a, ks, G, op, lp);
  if (a.D <= 96) return launch_lp_split<T, 96, CAUSAL>(a, ks, G, op, lp);
  return launch_lp_split<T, 128, CAUSAL>(a, ks, G, op, lp);
}
template <bool CAUSAL>
hipError_t dispatch_f32_split(const Launch& a, const KeySplit& ks, int G, float* op, float* lp) {
  if (a.D <= 32) return launch_f32_split<32, CAUSAL>(a, ks, G, op, lp);
  if (a.D <= 64) return launch_f32_split<64, CAUSAL>(a, ks, G, op, lp);
  if (a.D <= 96) return launch_f32_split<96, CAUSAL>(a, ks, G, op, lp);
  return launch_f32_split<128, CAUSAL>(a, ks, G, op, lp);
}

// The launch description shared by the entry points (arguments already checked).
Launch make_launch(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
                   int64_t H, int64_t M, int64_t N, int64_t D, float scale, int dtype,
                   void* stream, bool generic) {
  Launch a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.M = (int)M;
  a.N = (int)N;
  a.D = (int)D;
  a.qtiles = (int)((M + BM - 1) / BM);
  // scale * log2(e) folded once (in double, rounded to fp32) so every
  // exponential is exp2; its sign moves into the Q operand (fold_scale).
  const ScaleFold f = fold_scale(scale, dtype == FA_DTYPE_F32 ? 4 : 2);
  a.c = f.c;
  a.qf = f.q;
  a.grid = dim3((unsigned)(B * H * a.qtiles));
  a.BH = B * H;
  a.stream = (hipStream_t)stream;
  a.dev = stream_device(a.stream);
  a.generic = generic;
  return a;
}

}  // namespace

static int fa_fwd_impl(const void* q, const void* k, const void* v, void* o, float* lse,
                       int64_t B, int64_t H, int64_t M, int64_t N, int64_t D, float scale,
                       int causal, int dtype, void* stream, bool generic) {
  const int st = fa_check_args(q, k, v, o, lse, B, H, M, N, D, scale, causal, dtype);
  if (st != FA_OK) return st;
  if (B == 0 || H == 0 || M == 0) return FA_OK;
  const Launch a = make_launch(q, k, v, o, lse, B, H, M, N, D, scale, dtype, stream, generic);
  hipError_t e;
  switch (dtype) {
    case FA_DTYPE_F16:
      e = causal ? dispatch_lp<TF16, true>(a) : dispatch_lp<TF16, false>(a);
      break;
    case FA_DTYPE_BF16:
      e = causal ? dispatch_lp<TBF16, true>(a) : dispatch_lp<TBF16, false>(a);
      break;
    default:
      e = causal ? dispatch_f32<true>(a) : dispatch_f32<false>(a);
      break;
  }
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

extern "C" int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                      int64_t B, int64_t H, int64_t M, int64_t N, int64_t D, float scale,
                      int causal, int dtype, void* stream) {
  return fa_fwd_impl(q, k, v, o, lse, B, H, M, N, D, scale, causal, dtype, stream, false);
}

extern "C" int fa_fwd_general(const void* q, const void* k, const void* v, void* o, float* lse,
                              int64_t B, int64_t H, int64_t M, int64_t N, int64_t D, float scale,
                              int causal, int dtype, void* stream) {
  return fa_fwd_impl(q, k, v, o, lse, B, H, M, N, D, scale, causal, dtype, stream, true);
}

extern "C" int64_t fa_splitkv_workspace_bytes(int64_t B, int64_t H, int64_t M, int64_t D,
                                              int splits) {
  if (B < 0 || H < 0 || M < 0 || D < 1 || D > 128 || splits < 1) return -1;
  int64_t n = (int64_t)splits * (D + 1) * (int64_t)sizeof(float);
  if (__builtin_mul_overflow(n, B, &n) || __builtin_mul_overflow(n, H, &n) ||
      __builtin_mul_overflow(n, M, &n))
    return -1;  // beyond int64: no workspace of that size exists
  return n;
}

// The split-KV forward on a workspace of at least fa_splitkv_workspace_bytes
// (arguments already checked; N > 0).
static int splitkv_run(const void* q, const void* k, const void* v, void* o, float* lse,
                       int64_t B, int64_t H, int64_t M, int64_t N, int64_t D, float scale,
                       int causal, int dtype, int splits, void* workspace, void* stream) {
  // Chunks of ceil(N / splits) keys, rounded up to whole 64-key tiles.
  int64_t chunk = (N + splits - 1) / splits;
  chunk = (chunk + 63) / 64 * 64;
  const int G = (int)((N + chunk - 1) / chunk);
  const int64_t rows = B * H * M;
  float* opart = (float*)workspace;
  float* lpart = opart + (int64_t)G * rows * D;
  const Launch a = make_launch(q, k, v, o, lse, B, H, M, N, D, scale, dtype, stream, true);
  const KeySplit ks{(int)chunk, rows * D, rows};
  hipError_t e;
  switch (dtype) {
    case FA_DTYPE_F16:
      e = causal ? dispatch_lp_split<TF16, true>(a, ks, G, opart, lpart)
                 : dispatch_lp_split<TF16, false>(a, ks, G, opart, lpart);
      break;
    case FA_DTYPE_BF16:
      e = causal ? dispatch_lp_split<TBF16, true>(a, ks, G, opart, lpart)
                 : dispatch_lp_split<TBF16, false>(a, ks, G, opart, lpart);
      break;
    default:
      e = causal ? dispatch_f32_split<true>(a, ks, G, opart, lpart)
                 : dispatch_f32_split<false>(a, ks, G, opart, lpart);
      break;
  }
  if (e != hipSuccess) return FA_ERR_HIP;
  const int64_t work = rows * ((D + 3) / 4);
  const int64_t blocks = (work + NTHREADS - 1) / NTHREADS;
  const dim3 mgrid((unsigned)(blocks < 65536 ? blocks : 65536));
  switch (dtype) {
    case FA_DTYPE_F16:
      e = launch(fa_merge_kernel<_Float16>, mgrid, dim3(NTHREADS), a.stream, (const float*)opart,
                 (const float*)lpart, (_Float16*)o, lse, rows, (int)D, G, rows * D, rows);
      break;
    case FA_DTYPE_BF16:
      e = launch(fa_merge_kernel<__bf16>, mgrid, dim3(NTHREADS), a.stream, (const float*)opart,
                 (const float*)lpart, (__bf16*)o, lse, rows, (int)D, G, rows * D, rows);
      break;
    default:
      e = launch(fa_merge_kernel<float>, mgrid, dim3(NTHREADS), a.stream, (const float*)opart,
                 (const float*)lpart, (float*)o, lse, rows, (int)D, G, rows * D, rows);
      break;
  }
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

extern "C" int fa_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                              int64_t B, int64_t H, int64_t M, int64_t N, int64_t D, float scale,
                              int causal, int dtype, int splits, void* workspace,
                              int64_t workspace_bytes, void* stream) {
  const int st = fa_splitkv_check_args(q, k, v, o, lse, B, H, M, N, D, scale, causal, dtype,
                                       splits, workspace, workspace_bytes);
  if (st != FA_OK) return st;
  if (B == 0 || H == 0 || M == 0) return FA_OK;
  if (N == 0) return fa_fwd_impl(q, k, v, o, lse, B, H, M, N, D, scale, causal, dtype, stream,
                                 true);  // every row is empty: no chunk to merge
  return splitkv_run(q, k, v, o, lse, B, H, M, N, D, scale, causal, dtype, splits, workspace,
                     stream);
}

// ---------------------------------------------------------------------------
// Split-KV forward without any allocation.  The fp32 partials go to a
// file-scope device array; in host code its name is only a stand-in for the
// symbol, so the device address is looked up (hipGetSymbolAddress) once per
// device, with that device current, and that address is what the kernels get.
static __device__ __align__(256) char scratch[FA_NOALLOC_MAX_BYTES];

static void* scratch_address(int dev) {
  static std::mutex mu;
  static void* addr[64];
  if (dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return nullptr;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return nullptr;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) (void)hipSetDevice(cur);
    if (e != hipSuccess || p == nullptr) return nullptr;
    addr[dev] = p;
  }
  return addr[dev];
}

extern "C" int fa_fwd_splitkv_noalloc(const void* q, const void* k, const void* v, void* o,
                                      float* lse, int64_t B, int64_t H, int64_t M, int64_t N,
                                      int64_t D, float scale, int causal, int dtype, int splits,
                                      void* stream) {
  // Host validation with an aligned stand-in for the workspace (never
  // dereferenced) of the scratch's size: a too-large problem is reported as
  // the scratch limit, every other error as fa_fwd_splitkv reports it.
  const int st = fa_splitkv_check_args(q, k, v, o, lse, B, H, M, N, D, scale, causal, dtype,
                                       splits, reinterpret_cast<void*>(256),
                                       FA_NOALLOC_MAX_BYTES);
  if (st == FA_ERR_WORKSPACE) return FA_ERR_SCRATCH_LIMIT;
  if (st != FA_OK) return st;
  if (B == 0 || H == 0 || M == 0) return FA_OK;
  if (N == 0) return fa_fwd_impl(q, k, v, o, lse, B, H, M, N, D, scale, causal, dtype, stream,
                                 true);  // every row is empty: no partials
  void* ws = scratch_address(stream_device((hipStream_t)stream));
  if (ws == nullptr) return FA_ERR_HIP;
  return splitkv_run(q, k, v, o, lse, B, H, M, N, D, scale, causal, dtype, splits, ws, stream);
}
