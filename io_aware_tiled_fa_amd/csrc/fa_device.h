// fa_device.h - device-side definitions shared by the forward and backward
// attention kernels for gfx950: element types and their MFMA, the row
// permutation that lines the 32x32 MFMA accumulator layout up with the next
// MFMA's operand layout, the XCD-aware workgroup mapping and the lane-pair
// reductions.  Included by fa_fwd.hip and fa_bwd.hip only.
#ifndef FA_DEVICE_H
#define FA_DEVICE_H

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr float LN2F = 0.693147180559945309417f;

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

struct TF16 {
  using elt = _Float16;
  using vec8 = f16x8;
  static __device__ __forceinline__ f32x16 mfma(vec8 a, vec8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
};
struct TBF16 {
  using elt = __bf16;
  using vec8 = bf16x8;
  static __device__ __forceinline__ f32x16 mfma(vec8 a, vec8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};

// Row of the S^T tile <-> key within a 32-key group: swap bits 2 and 3.
__device__ __forceinline__ int swap23(int x) {
  return (x & ~12) | ((x & 4) << 1) | ((x & 8) >> 1);
}

// Key (relative to the tile's first key, within a 32-key half) held by
// accumulator register r of a lane in lane-half h.
__device__ __forceinline__ int key_of_reg(int r, int h) {
  return 16 * (r >> 3) + 8 * h + (r & 7);
}

// Which workgroup works on which (batch*head, query tile).
// Workgroups are handed to the 8 XCDs round-robin (id % 8), and each XCD has
// its own L2.  The id is remapped so that every XCD walks a contiguous range
// of (head, query tile) pairs: the query tiles of one head then run on one XCD
// at about the same time and share that head's K/V in its L2.  Within a head,
// causal tiles are issued heaviest first (the last query tile sees the most
// keys), so the light tiles fill the tail.
struct TileCoord {
  int bh;
  int q0;
};
constexpr int NXCD = 8;
template <bool CAUSAL, int ROWS = 128>
__device__ __forceinline__ TileCoord tile_coord(int qtiles) {
  const int G = gridDim.x;
  const int b = blockIdx.x;
  const int xcd = b % NXCD;
  const int idx = b / NXCD;
  const int per = G / NXCD;
  const int rem = G % NXCD;
  const int t = xcd * per + min(xcd, rem) + idx;  // contiguous range per XCD
  TileCoord c;
  c.bh = t / qtiles;
  int qt = t - c.bh * qtiles;
  if (CAUSAL) qt = qtiles - 1 - qt;
  c.q0 = qt * ROWS;
  return c;
}

// Persistent schedule.  A launch of P = gridDim.x workgroups covers `items`
// work items (P <= items).  The items are cut into NXCD contiguous ranges, one
// per XCD (workgroup g runs on XCD g % NXCD, so an XCD's L2 keeps its heads'
// K and V), and the Px workgroups of an XCD take that range in rounds of Px,
// in snake order: workgroup j takes index j in even rounds and Px - 1 - j in
// odd ones, so that with heavy-first items each workgroup alternates heavy
// and light ones.  Returns the item of `round`, or -1 once the range is done.
// With P == items every workgroup takes exactly the item tile_coord gives it.
__device__ __forceinline__ int persistent_item(int round, int items) {
  const int P = gridDim.x;
  const int g = blockIdx.x;
  const int x = g % NXCD;
  const int j = g / NXCD;
  const int Px = P / NXCD + (x < P % NXCD ? 1 : 0);
  const int per = items / NXCD;
  const int rem = items % NXCD;
  const int cnt = per + (x < rem ? 1 : 0);
  const int jj = (round & 1) ? Px - 1 - j : j;
  const int idx = round * Px + jj;
  return idx < cnt ? x * per + min(x, rem) + idx : -1;
}

// (batch*head, first query row) of work item t: heads in order, and within a
// head the query tiles heaviest-first under the causal mask.
template <bool CAUSAL, int ROWS>
__device__ __forceinline__ TileCoord item_coord(int t, int qtiles) {
  TileCoord c;
  c.bh = t / qtiles;
  int qt = t - c.bh * qtiles;
  if (CAUSAL) qt = qtiles - 1 - qt;
  c.q0 = qt * ROWS;
  return c;
}

// Device a stream belongs to (the current device for the null stream, or if
// the runtime cannot tell).
inline int stream_device(hipStream_t stream) {
  int dev = 0;
  if (stream != nullptr && hipStreamGetDevice(stream, &dev) == hipSuccess) return dev;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  return dev;
}

// Compute units of device `dev` (cached per device; 0 if unknown).
inline int device_cus(int dev) {
  static int cache[64];
  if (dev < 0 || dev >= 64) return 0;
  int v = __atomic_load_n(&cache[dev], __ATOMIC_RELAXED);
  if (v == 0) {
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    __atomic_store_n(&cache[dev], v, __ATOMIC_RELAXED);
  }
  return v;
}

// Workgroup count for a persistent launch of KERNEL (with `threads` threads)
// on device `dev`: one per CU when the occupancy calculator puts exactly one
// workgroup on a CU, else 0 (launch one workgroup per item: co-resident
// workgroups that start together stay in step and stop hiding each other's
// prologue).  Cached per kernel and device (the kernel is a template argument,
// so kernels that share a signature do not share the answer); 0 too if the
// runtime cannot tell.  Only for kernels that loop over work items: a launch
// of P < items workgroups leaves items undone in any other kernel.  (The
// occupancy depends only on the kernel's resources and the architecture, the
// same on every gfx950 device.)
template <auto KERNEL>
int persistent_workgroups(int threads, int dev) {
  static int cache[64];  // per device: -1 no, > 0 the count
  if (dev < 0 || dev >= 64) return 0;
  int v = __atomic_load_n(&cache[dev], __ATOMIC_RELAXED);
  if (v == 0) {
    int cus = 0, occ = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, reinterpret_cast<const void*>(KERNEL),
                                                     threads, 0) != hipSuccess)
      return 0;
    v = occ == 1 && cus > 0 ? cus : -1;
    __atomic_store_n(&cache[dev], v, __ATOMIC_RELAXED);
  }
  return v > 0 ? v : 0;
}

// Launch of a kernel that reports its own status: hipLaunchKernel's return
// value, so no hipGetLastError call reads (and clears) an error the caller
// has not looked at yet.
template <class X>
struct same_type {
  using type = X;
};
template <class... P>
hipError_t launch(void (*kern)(P...), dim3 grid, dim3 block, hipStream_t stream,
                  typename same_type<P>::type... args) {
  void* argv[] = {(void*)&args..., nullptr};
  return hipLaunchKernel(reinterpret_cast<const void*>(kern), grid, block, argv, 0, stream);
}

// Lanes l and l^32 hold the same query row (different keys).  v_permlane32_swap
// exchanges the two wave halves in one VALU op (no LDS round trip).
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// Direct-to-LDS tile layout for fp16/bf16 with D in {64, 96, 128}: K and V tiles are copied from
// HBM straight into LDS (global_load_lds, 16 B per lane, no VGPR staging), in
// their natural row-major layout with a per-row XOR swizzle of the 16-byte
// chunks.  The K operand of S^T is one ds_read_b128 per lane and k-step; the
// V^T operand of O^T is read transposed out of row-major V with two
// ds_read_b64_tr_b16 per MFMA (each lane of a 16-lane group receives one
// column of a 4-row x 4-column block).  The swizzle makes both read patterns
// bank-conflict free: 16 consecutive rows hit 16 distinct chunk positions for
// the K reads, and the 4 rows of a transpose read land in 4 distinct 64-byte
// groups of banks.
template <int DP>
struct FastLayout {
  static constexpr int ROWB = DP == 64 ? 128 : 256;  // LDS bytes per K/V row
  static constexpr int CPR = DP / 8;                  // 16-byte chunks holding data
  static constexpr int SLOTS = ROWB / 16;             // 16-byte slots per row
  static constexpr int TILEB = 64 * ROWB;             // one 64-row K (or V) tile
  static constexpr int RPB = 1024 / ROWB;             // rows per 1 KB copy instruction
  static constexpr int NBLK = TILEB / 1024;           // copy instructions per tile matrix
  // Physical slot of logical chunk c in row r is c ^ swz(r).
  // K: the 16 rows of a score-MFMA read land on 16 distinct slots.
  static __device__ __forceinline__ int swz_k(int r) {
    return DP == 64 ? ((((r >> 1) & 1) << 2) | ((r >> 2) & 3)) : (((r & 3) << 2) | ((r >> 2) & 3));
  }
  // V: the 4 rows of a transpose read land in 4 distinct 64-byte bank groups;
  // depends only on r mod 4 so that rows 4 apart share the pattern.
  static __device__ __forceinline__ int swz_v(int r) {
    return DP == 64 ? (((r >> 1) & 1) << 2) : ((r & 3) << 2);
  }
};


// Sign of the scale.  Every kernel takes the row maximum of raw scores q.k and
// multiplies it by c = scale*log2(e) afterwards, and masks invisible keys with
// -inf before that multiply; both need c > 0.  For c < 0, S*c equals
// ((-Q) K^T)*|c| exactly (negation is exact and the MFMA's round-to-nearest is
// symmetric under it), and for c == 0 every score is 0 = (0*Q) K^T.  So the
// operand that enters the score product from registers (Q in the forward and
// dQ kernels, K in the dK/dV kernels) is sign-flipped or zeroed as it is
// loaded, word by word as (x & qand) ^ qxor, and the kernels see a positive c.
struct QFold {
  unsigned qand;
  unsigned qxor;
};
__device__ __forceinline__ u32x4 fold_bits(u32x4 x, QFold f) { return (x & f.qand) ^ f.qxor; }
template <class V>
__device__ __forceinline__ V fold_vec(V x, QFold f) {
  return __builtin_bit_cast(V, fold_bits(__builtin_bit_cast(u32x4, x), f));
}
__device__ __forceinline__ float fold_f32(float x, QFold f) {
  return __uint_as_float((__float_as_uint(x) & f.qand) ^ f.qxor);
}

// Host side: the positive exponent constant c, the positive scale s_eff the
// kernels' row statistics use (|scale|, or 1 for a zero scale, where every
// score is 0 and any positive constant gives the uniform weights), and the fold
// of the score operand.  `elt_bytes` is the element size of that operand.
struct ScaleFold {
  float c;
  float s_eff;
  QFold q;
};
inline ScaleFold fold_scale(float scale, int elt_bytes) {
  const double log2e = 1.4426950408889634074;
  const float c = (float)((double)scale * log2e);  // rounded once, as every exponential uses it
  const unsigned sign = elt_bytes == 4 ? 0x80000000u : 0x80008000u;
  if (c > 0.0f) return ScaleFold{c, scale, QFold{~0u, 0u}};
  if (c < 0.0f) return ScaleFold{-c, -scale, QFold{~0u, sign}};
  return ScaleFold{(float)log2e, 1.0f, QFold{0u, 0u}};
}

// Pins a value at this point of the instruction stream: an empty statement
// that reads and rewrites it, so the arithmetic producing it cannot be moved
// past a later scheduling fence (device pass only; the host pass has no
// vector registers).
template <class X>
__device__ __forceinline__ void pin(X& x) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("" : "+v"(x));
#else
  (void)x;
#endif
}

__device__ __forceinline__ void copy16_to_lds(const void* g, char* lds_block) {
  __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)g,
                                   (void __attribute__((address_space(3)))*)lds_block, 16, 0, 0);
}

}  // namespace

#endif  // FA_DEVICE_H
