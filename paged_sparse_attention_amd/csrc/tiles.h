// tiles.h -- LDS tiles and MFMA operand reads for the gfx950 attention kernels.
//
// A tile holds BR rows of D elements, row-major.  Operands read from it:
//   frag_rm(row, s, hh): the A operand whose row is a tile row and whose
//     contraction runs along D -- lane (row, half hh) takes elements
//     [s*KS + hh*KL, +KL) of that row (one 16-byte read for bf16).
//   frag_tr(rb, cb, s, lane): the A operand of the transposed tile -- its rows
//     are the D columns cb*32 .. cb*32+31 and its contraction runs over the
//     tile rows of the 32-row block rb, in the order in which a 32x32
//     accumulator holds its rows (lane half hh holds rows 8*(e/4) + 4*hh + e%4,
//     e < 16), so that an accumulator computed with tile rows as its M
//     dimension can be fed back as the B operand of a product that contracts
//     over those rows.
//
// bf16 rows are padded to 288 bytes (D = 128) or 144 bytes (D = 64) and, for
// D = 128, rows 8..15 of every 16 swap neighbouring 16-byte chunks: then the 16
// rows of a 16-lane group of 16-byte reads, and the 4 rows x 32 bytes of a
// 16-lane group of transposing reads, fall in distinct LDS banks, while every
// operand address stays affine (immediate offsets, few registers).  A bf16 tile
// is filled straight from global memory with direct-to-LDS loads
// (global_load_lds_dwordx4: lane l of a wave writes bytes [16 l, 16 l + 16) of
// a 1 KB block; padding slots get a dummy chunk), so staging needs no
// registers; the transposed operand is read with the gfx950 transposing LDS
// read (ds_read_b64_tr_b16: within 16 lanes, lane i gets value i%4 of the
// 8-byte chunk addressed by lane 4k + i/4, for k = 0..3).
// fp32 tiles are padded, filled through registers, and keep a second,
// transposed copy for frag_tr.
#pragma once

#include "common.h"

namespace oomb {

typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) const void gbl_void;

// Direct global -> LDS loads issued through inline asm (lane l of a wave
// writes bytes [n l, n l + n) of the block at the wave-uniform LDS address
// `lds`; no registers are written).  The compiler cannot tell which LDS bytes
// such a load writes, so after one it makes the next LDS read of any tile wait
// for every load still in flight: with the builtin, a ring's tiles in flight
// ahead of their use are waited for at the first read of the tile in use.
// Issued as asm the loads are invisible to it, and a kernel waits for its own
// (wait_vmem_le, counting this wave's loads issued later) before the barrier
// that publishes a tile.  M0 holds the LDS address (one wait state before the
// load reads it) and is restored afterwards.
__device__ __forceinline__ unsigned lds_addr(const void* p) {
  return (unsigned)__builtin_amdgcn_readfirstlane(
      (int)(unsigned)(uintptr_t)(const __attribute__((address_space(3))) void*)p);
}
__device__ __forceinline__ const void* uniform_ptr(const void* p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  return (const void*)(uintptr_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(v >> 32)) << 32) |
                                  (uint32_t)__builtin_amdgcn_readfirstlane((int)v));
}
// 16 bytes a lane from the lane's own global address
__device__ __forceinline__ void lds_load16(const void* gptr, const void* lds) {
  int save;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off\n\ts_mov_b32 m0, %0"
      : "=&s"(save)
      : "v"(gptr), "s"(lds_addr(lds))
      : "memory");
}
// 16 bytes a lane from a wave-uniform base plus the lane's byte offset
__device__ __forceinline__ void lds_load16(const void* base, unsigned byte_off, const void* lds) {
  int save;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2\n\ts_mov_b32 m0, %0"
      : "=&s"(save)
      : "v"(byte_off), "s"(uniform_ptr(base)), "s"(lds_addr(lds))
      : "memory");
}
// 4 bytes a lane
__device__ __forceinline__ void lds_load4(const void* gptr, const void* lds) {
  int save;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %1, off\n\ts_mov_b32 m0, %0"
               : "=&s"(save)
               : "v"(gptr), "s"(lds_addr(lds))
               : "memory");
}

template <typename T, int D, int BR> struct Tile;

template <int D, int BR> struct Tile<__bf16, D, BR> {
  typedef __bf16 T;
  static constexpr int VEC = 8;                      // elements per 16-byte chunk
  static constexpr int CPR = D / VEC;                // data chunks per row (16 or 8)
  static constexpr int SLOTS = D == 128 ? 18 : 9;    // chunk slots per row, padding included
  static constexpr int RS = SLOTS * VEC;             // row stride (elements): 288 B or 144 B
  static constexpr int ELEMS = BR * RS;              // LDS elements per tile
  static constexpr int BLOCKS = BR * SLOTS / 64;     // 1 KB blocks (one direct load per wave each)
  static_assert(D == 128 || D == 64, "bf16 tiles support D = 64 and 128");
  static_assert((BR * SLOTS) % 64 == 0, "tile must be whole 1 KB blocks");
  T* rm;

  // chunk position of logical chunk c in row r: for D = 128 rows 8..15 of each
  // 16 swap neighbouring chunks, which puts the 16 rows of a 16-byte read in 16
  // distinct bank groups; the addresses stay affine in the chunk index
  __device__ static __forceinline__ int flip(int r) { return D == 128 ? (r >> 3) & 1 : 0; }

  // Direct global -> LDS fill of this tile by `nwaves` waves.  off(r): element
  // offset in src of tile row r (callers clamp rows past the end to a real one).
  // Padding slots are filled from the row's first chunk.
  template <typename OffFn>
  __device__ __forceinline__ void fill(const T* __restrict__ src, int wave, int nwaves, int lane, OffFn off) const {
    for (int b = wave; b < BLOCKS; b += nwaves) {
      const int q = b * 64 + lane;
      const int r = q / SLOTS, p = q % SLOTS;
      const int c = p < CPR ? (p ^ flip(r)) : 0;
      lds_load16(src + off(r) + c * VEC, rm + b * 512);
    }
  }
  // (2s + hh) ^ flip(row) == 2s + (hh ^ flip(row)): s only adds an immediate offset
  __device__ __forceinline__ bf16x8 frag_rm(int row, int s, int hh) const {
    return *reinterpret_cast<const bf16x8*>(rm + row * RS + (hh ^ flip(row)) * VEC + s * 2 * VEC);
  }
  __device__ __forceinline__ bf16x8 frag_tr(int rb, int cb, int s, int lane) const {
    // lane (g, j) = (lane / 16, lane % 16) reads row rb*32 + 16s + rl (+ 8) and
    // chunk 4cb + cl; rl < 8, so flip() is 0 on the first row and 1 on the
    // second, and rb, s and cb only add immediate offsets
    const int g = lane >> 4, j = lane & 15;
    const int rl = 4 * (g >> 1) + (j >> 2);
    const int cl = 2 * (g & 1) + ((j & 3) >> 1);
    const int half = (j & 1) * 4;
    const int fixed = (rb * 32 + 16 * s) * RS + 4 * cb * VEC;
    const T* p0 = rm + fixed + rl * RS + cl * VEC + half;
    const T* p1 = rm + fixed + (rl + 8) * RS + (cl ^ flip(8)) * VEC + half;
    const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p0);
    const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p1);
    bf16x8 f;
    const __bf16* pa = reinterpret_cast<const __bf16*>(&a);
    const __bf16* pb = reinterpret_cast<const __bf16*>(&b);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[i] = pa[i];
      f[4 + i] = pb[i];
    }
    return f;
  }
};

// fp32: row-major copy (stride D+4) plus a transposed copy in operand order,
// tr[(row/32) * D * TRS + d * TRS + operand_pos(row % 32)], TRS = 36.
template <int D, int BR> struct Tile<float, D, BR> {
  typedef float T;
  static constexpr int VEC = 4;
  static constexpr int CPR = D / VEC;
  static constexpr int RS = D + 4;
  static constexpr int TRS = 36;
  static constexpr int ELEMS = BR * RS + (BR / 32) * D * TRS;
  T* rm;

  __device__ __forceinline__ void put(int row, int cg, const f32x4& v) const {
    *reinterpret_cast<f32x4*>(rm + row * RS + cg * VEC) = v;
    T* tr = rm + BR * RS + (row >> 5) * D * TRS + (cg * VEC) * TRS + operand_pos(row & 31);
#pragma unroll
    for (int e = 0; e < 4; ++e) tr[e * TRS] = v[e];
  }
  __device__ __forceinline__ float frag_rm(int row, int s, int hh) const { return rm[row * RS + s * 2 + hh]; }
  __device__ __forceinline__ float frag_tr(int rb, int cb, int s, int lane) const {
    const int col = lane & 31, hh = lane >> 5;
    return rm[BR * RS + rb * D * TRS + (cb * 32 + col) * TRS + hh * 16 + s];
  }
};

// Register staging for fp32 tiles: NT threads each carry N 16-byte chunks;
// chunk c of the tile is (row c / CPR, column group c % CPR).
template <int D, int BR, int NT> struct Stager {
  typedef Tile<float, D, BR> TL;
  static constexpr int N = (BR * TL::CPR + NT - 1) / NT;
  f32x4 v[N];

  template <typename OffFn>
  __device__ __forceinline__ void load(const float* __restrict__ src, int tid, OffFn off) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int c = tid + i * NT;
      v[i] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (c < BR * TL::CPR) v[i] = *reinterpret_cast<const f32x4*>(src + off(c / TL::CPR) + (c % TL::CPR) * 4);
    }
  }
  __device__ __forceinline__ void store(const TL& t, int tid) const {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int c = tid + i * NT;
      if (c < BR * TL::CPR) t.put(c / TL::CPR, c % TL::CPR, v[i]);
    }
  }
};

// Waits for every vector-memory operation of this wave, as an instruction the
// compiler sees (unlike wait_vmem_le): afterwards it knows that the registers
// loaded before are ready, and does not wait for them again inside a key loop,
// where that wait would also wait for the ring's loads in flight.
__device__ __forceinline__ void vmem_drain() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)

// Waits until at most n of this wave's vector-memory operations are still in
// flight (direct-to-LDS loads included); n is clamped to the counter's range.
__device__ __forceinline__ void wait_vmem_le(int n) {
  switch (n < 0 ? 0 : (n > 15 ? 15 : n)) {
#define OOMB_WAIT_CASE(k) \
  case k: asm volatile("s_waitcnt vmcnt(" #k ")" ::: "memory"); break;
    OOMB_WAIT_CASE(0) OOMB_WAIT_CASE(1) OOMB_WAIT_CASE(2) OOMB_WAIT_CASE(3) OOMB_WAIT_CASE(4)
    OOMB_WAIT_CASE(5) OOMB_WAIT_CASE(6) OOMB_WAIT_CASE(7) OOMB_WAIT_CASE(8) OOMB_WAIT_CASE(9)
    OOMB_WAIT_CASE(10) OOMB_WAIT_CASE(11) OOMB_WAIT_CASE(12) OOMB_WAIT_CASE(13) OOMB_WAIT_CASE(14)
    OOMB_WAIT_CASE(15)
#undef OOMB_WAIT_CASE
  }
}

// 1 KB direct-load blocks of a tile (tiles filled through registers have none)
template <typename TL, bool direct> struct BlockCount {
  static constexpr int value = 1;
};
template <typename TL> struct BlockCount<TL, true> {
  static constexpr int value = TL::BLOCKS;
};

// Two tensors with the same row addressing (K and V, or Q and dO) streamed
// through a ring of NSLOTS LDS tile slots, PD = NSLOTS - 1 tiles in flight
// ahead of the one in use.  bf16 tiles are filled by direct-to-LDS loads (any
// number of slots); fp32 tiles are staged through registers (two slots, one
// tile in flight).  Use, per tile index j:
//   load(j) for the first PD tiles; then for each j:
//     commit(j, tiles_issued_after_j, extra) -- tile j has landed for this wave
//     barrier                                 -- ... and for every wave
//     load(j + PD) if it exists               -- refills the slot of tile j - 1
//     read tiles ta(j), tb(j)

// ASM: direct loads through inline asm (above).  The forward keeps the
// builtin: its key loop, at the register limit, is compiled with spill
// reloads between the asm loads, each of which waits for the loads issued
// before it.
template <typename T, int D, int BR, int NT, int NSLOTS = sizeof(T) == 2 ? 3 : 2, bool ASM = true> struct Ring {
  typedef Tile<T, D, BR> TL;
  static constexpr bool kDirect = sizeof(T) == 2;
  static constexpr int NS = NSLOTS;           // slots
  static constexpr int PD = NS - 1;           // tiles in flight ahead of the one in use
  T* pa;                                      // slot s of tensor a: pa + s * TL::ELEMS
  T* pb;
  Stager<D, BR, NT> sa, sb;                   // fp32 only

  __device__ __forceinline__ TL ta(int j) const { return TL{pa + (j % NS) * TL::ELEMS}; }
  __device__ __forceinline__ TL tb(int j) const { return TL{pb + (j % NS) * TL::ELEMS}; }

  // direct loads one wave issues per tile (both tensors)
  __device__ static __forceinline__ int loads_per_tile(int wave) {
    if constexpr (kDirect) return 2 * ((TL::BLOCKS - wave + NT / 64 - 1) / (NT / 64));
    else return 0;
  }

  template <typename OffFn>
  __device__ __forceinline__ void load(int j, const T* __restrict__ srca, const T* __restrict__ srcb, int tid,
                                       OffFn off) {
    if constexpr (kDirect) {
      const int wave = tid >> 6, lane = tid & 63;
      T* da = pa + (j % NS) * TL::ELEMS;
      T* db = pb + (j % NS) * TL::ELEMS;
      for (int blk = wave; blk < TL::BLOCKS; blk += NT / 64) {
        const int q = blk * 64 + lane;
        const int r = q / TL::SLOTS, p = q % TL::SLOTS;
        const int c = p < TL::CPR ? (p ^ TL::flip(r)) : 0;
        const int64_t o = off(r) + c * TL::VEC;
        if constexpr (ASM) {
          lds_load16(srca + o, da + blk * 512);
          lds_load16(srcb + o, db + blk * 512);
        } else {
          __builtin_amdgcn_global_load_lds((gbl_void*)(srca + o), (lds_void*)(da + blk * 512), 16, 0, 0);
          __builtin_amdgcn_global_load_lds((gbl_void*)(srcb + o), (lds_void*)(db + blk * 512), 16, 0, 0);
        }
      }
    } else {
      sa.load((const float*)srca, tid, off);
      sb.load((const float*)srcb, tid, off);
    }
  }
  // Direct loads of a tile whose rows lie row_stride elements apart (row r at
  // base + r * row_stride).  The element offsets of a wave's load slots within
  // a tile never change, so lane_offsets computes them once; a tile then costs
  // one wave-uniform base per tensor and no per-lane address arithmetic.
  static constexpr int NW = NT / 64;
  static constexpr int NBW = (BlockCount<TL, kDirect>::value + NW - 1) / NW;  // 1 KB blocks a wave loads, at most
  struct Lanes {
    int off[NBW];
  };
  __device__ static __forceinline__ Lanes lane_offsets(int tid, int row_stride) {
    Lanes l;
    if constexpr (kDirect) {
      const int wave = tid >> 6, lane = tid & 63;
#pragma unroll
      for (int i = 0; i < NBW; ++i) {
        const int q = (wave + i * NW) * 64 + lane;
        const int r = q / TL::SLOTS, p = q % TL::SLOTS;
        const int c = p < TL::CPR ? (p ^ TL::flip(r)) : 0;
        l.off[i] = r * row_stride + c * TL::VEC;
      }
    }
    return l;
  }
  __device__ __forceinline__ void load_rows(int j, const T* __restrict__ srca, const T* __restrict__ srcb,
                                            int64_t base, const Lanes& l, int tid) {
    static_assert(kDirect, "row loads are direct-to-LDS (bf16)");
    const int wave = tid >> 6;
    const int64_t b = (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(base >> 32)) << 32) |
                                (uint32_t)__builtin_amdgcn_readfirstlane((int)base));
    const T* a0 = srca + b;
    const T* b0 = srcb + b;
    T* da = pa + (j % NS) * TL::ELEMS;
    T* db = pb + (j % NS) * TL::ELEMS;
#pragma unroll
    for (int i = 0; i < NBW; ++i) {
      const int blk = wave + i * NW;
      if (blk < TL::BLOCKS) {
        if constexpr (ASM) {
          lds_load16(a0, (unsigned)l.off[i] * (unsigned)sizeof(T), da + blk * 512);
          lds_load16(b0, (unsigned)l.off[i] * (unsigned)sizeof(T), db + blk * 512);
        } else {
          __builtin_amdgcn_global_load_lds((gbl_void*)(a0 + l.off[i]), (lds_void*)(da + blk * 512), 16, 0, 0);
          __builtin_amdgcn_global_load_lds((gbl_void*)(b0 + l.off[i]), (lds_void*)(db + blk * 512), 16, 0, 0);
        }
      }
    }
  }
  // tile j is in LDS as far as this thread is concerned; `newer` tiles were
  // issued after it, each costing `vm_per_tile` vector-memory operations
  __device__ __forceinline__ void commit(int j, int newer, int vm_per_tile, int tid) {
    if constexpr (kDirect) {
      wait_vmem_le(newer * vm_per_tile);
    } else {
      sa.store(Tile<float, D, BR>{(float*)pa + (j % NS) * TL::ELEMS}, tid);
      sb.store(Tile<float, D, BR>{(float*)pb + (j % NS) * TL::ELEMS}, tid);
    }
  }
};

// One 32-bit value per lane straight from global memory to LDS (lane l writes
// dst[l]); lanes outside exec write nothing.
__device__ __forceinline__ void load_lds_dword(const float* src, float* dst_wave_base) {
  lds_load4(src, dst_wave_base);
}

}  // namespace oomb
