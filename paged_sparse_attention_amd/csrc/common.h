// common.h -- device helpers shared by the gfx950 kernels of the paged top-K
// chunk attention library (one chunk step of OOMB's chunk-recurrent attention
// over a paged KV cache: page "Out of the Memory Barrier", technical summary,
// section 2, "Paged Memory Management" and "Page-level Sparse Attention").
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace oomb {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Geometry of one chunk step, as the kernels see it.
struct Geo {
  int hq, hkv, G;          // query heads, kv heads, group size Hq/Hkv
  uint64_t g_magic;        // ceil(2^40 / G): x / G == (x * g_magic) >> 40 for x < 2^24
  int c;                   // chunk tokens
  int n;                   // prior pages
  int keff;                // selected pages per kv-head
  int ps_log2;             // log2(page size)
  int n_slots;
  float scale;             // softmax scale
};

// ---------------------------------------------------------------------------
// MFMA 32x32 tiles.  For an instruction with M = N = 32 and contraction depth
// KS, lane l holds
//   A operand: row  l % 32, k = (l / 32) * KL + [0, KL)
//   B operand: col  l % 32, k = (l / 32) * KL + [0, KL)
//   C/D:       col  l % 32, row 8 * (e / 4) + 4 * (l / 32) + (e % 4), e < 16
// with KL = KS / 2 values per lane.
// ---------------------------------------------------------------------------
template <typename T> struct Mma;

template <> struct Mma<__bf16> {
  static constexpr int KS = 16;
  static constexpr int KL = 8;
  typedef bf16x8 frag;
  __device__ static inline f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  __device__ static inline frag load(const __bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }
  __device__ static inline frag zero() {
    frag f;
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = (__bf16)0.f;
    return f;
  }
  // KL accumulator values (elements e0 .. e0+KL-1 of a 32x32 tile) as an operand
  __device__ static inline frag pack(const f32x16& acc, int e0) {
    frag f;
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = (__bf16)acc[e0 + i];
    return f;
  }
};

template <> struct Mma<float> {
  static constexpr int KS = 2;
  static constexpr int KL = 1;
  typedef float frag;
  __device__ static inline f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
  __device__ static inline frag load(const float* p) { return *p; }
  __device__ static inline frag zero() { return 0.f; }
  __device__ static inline frag pack(const f32x16& acc, int e0) { return acc[e0]; }
};

// Row of a 32x32 accumulator held in element e by a lane of half hh (= lane / 32).
__device__ __forceinline__ int acc_row(int e, int hh) { return 8 * (e >> 2) + 4 * hh + (e & 3); }

// Position of row rho (0..31) of a 32-row block in the "operand order" used by
// transposed tiles: for lane half hh the 16 rows it holds in an accumulator, in
// element order, are stored contiguously at [16 hh, 16 hh + 16).  An accumulator
// reused as a B operand then meets an A operand read with KL consecutive loads.
__device__ __forceinline__ int operand_pos(int rho) { return 16 * ((rho >> 2) & 1) + 4 * (rho >> 3) + (rho & 3); }

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// ---------------------------------------------------------------------------
// Paged key addressing.  The key list of kv-head h is J(h): the tokens of the
// keff selected pages (sel order, then row order), then the c chunk tokens,
// which live in logical pages n .. n + c/ps - 1.  Returns the element offset
// of (slot, h, row, 0) in a [n_slots][hkv][ps][D] pool.
// ---------------------------------------------------------------------------
template <int D>
__device__ __forceinline__ int64_t key_offset(const Geo& g, const int32_t* __restrict__ pt,
                                              const int32_t* __restrict__ sel, int h, int jj) {
  const int pk = g.keff << g.ps_log2;
  int page, row;
  if (jj < pk) {
    page = sel[h * g.keff + (jj >> g.ps_log2)];
    row = jj & ((1 << g.ps_log2) - 1);
  } else {
    const int u = jj - pk;
    page = g.n + (u >> g.ps_log2);
    row = u & ((1 << g.ps_log2) - 1);
  }
  const int64_t slot = pt[page];
  return ((slot * g.hkv + h) * (int64_t)(1 << g.ps_log2) + row) * D;
}

// x / G for 0 <= x < 2^24 and G < 1024: the product stays below 2^64 and the
// error of the rounded-up reciprocal, x * (g_magic - 2^40/G) / 2^40 < 2^-16,
// stays below 1/G, so the floor is exact.
__device__ __forceinline__ int div_g(const Geo& g, int x) {
  return (int)(((uint64_t)(uint32_t)x * g.g_magic) >> 40);
}

// Workgroup b runs on XCD b % 8 (dispatch is round-robin over the 8 XCDs).
// Map it to a work item so that each XCD gets a contiguous range of items,
// whose K/V (or Q/dO) tiles then stay in that XCD's L2.
__device__ __forceinline__ int xcd_remap(int b, int total) {
  const int per = total / 8;
  if (b >= per * 8) return b;
  return (b % 8) * per + b / 8;
}

// Row-block items of the query-major kernels (forward, dQ): nrb row blocks per
// kv-head, ranked heaviest first (rank 0 = the last block, which sees the most
// chunk keys).  Contiguous ranges per XCD would give one XCD a head's heavy
// half and the next its light half, and the heavy XCD would finish last.
// When the heads divide evenly over the XCDs (S = 8 / hkv of them per head,
// nrb a multiple of S), the S XCDs of a head take its ranks in turn (the
// head's s-th XCD gets ranks s, s + S, s + 2S, ...): equal shares of heavy and
// light blocks, heaviest first on each, and still one head's pages per XCD.
// Otherwise each XCD gets a contiguous range of items.
struct RowItem {
  int h, rank;
};
__device__ __forceinline__ RowItem row_item(int b, int nrb, int hkv) {
  if (hkv <= 8 && 8 % hkv == 0 && nrb % (8 / hkv) == 0) {
    const int S = 8 / hkv, x = b % 8;
    return {x / S, (b / 8) * S + x % S};
  }
  const int item = xcd_remap(b, nrb * hkv);
  return {item / nrb, item % nrb};
}

// Physical slots of the pages of a kv-head's key list J(h) -- the K_eff
// selected pages, then the chunk's C/ps pages -- cached in LDS by a workgroup
// (when they fit in CAP entries; otherwise read from global memory).
// The table pointer is typed as LDS (address space 3): reads through a generic
// pointer compile to flat loads, which count as vector memory operations, so
// the wait for the slot would also wait for every tile load still in flight.
typedef __attribute__((address_space(3))) int lds_int;

template <int CAP> struct PageSlots {
  lds_int* tab;  // LDS, CAP entries
  bool cached;

  // all threads of the workgroup call this, then synchronise before use
  __device__ __forceinline__ void fill(const Geo& g, const int32_t* __restrict__ pt,
                                       const int32_t* __restrict__ sel, int h, int npages, int tid, int nt) {
    cached = npages <= CAP;
    if (cached)
      for (int i = tid; i < npages; i += nt) tab[i] = pt[i < g.keff ? sel[h * g.keff + i] : g.n + i - g.keff];
  }
  template <int D>
  __device__ __forceinline__ int64_t key_offset(const Geo& g, const int32_t* __restrict__ pt,
                                                const int32_t* __restrict__ sel, int h, int jj) const {
    if (!cached) return oomb::key_offset<D>(g, pt, sel, h, jj);
    return key_offset_cached<D>(g, h, jj);
  }
  // the same, for a caller that has already checked `cached`
  template <int D>
  __device__ __forceinline__ int64_t key_offset_cached(const Geo& g, int h, int jj) const {
    const int64_t slot = tab[jj >> g.ps_log2];
    return ((slot * g.hkv + h) * (int64_t)(1 << g.ps_log2) + (jj & ((1 << g.ps_log2) - 1))) * D;
  }
};
// Compile-time bool for generic lambdas: a kernel runs its key loop through
// run(Bool<true>()) or run(Bool<false>()), so each copy of the loop holds one
// kind of page lookup only.
template <bool B> struct Bool {
  static constexpr bool value = B;
};
constexpr int kPageCache = 1024;

// Warp-wide helpers (wave64).
__device__ __forceinline__ float wave_xor_max(float v, int mask) { return fmaxf(v, __shfl_xor(v, mask, 64)); }
__device__ __forceinline__ float wave_xor_sum(float v, int mask) { return v + __shfl_xor(v, mask, 64); }

}  // namespace oomb
