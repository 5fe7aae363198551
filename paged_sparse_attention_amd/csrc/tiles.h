// tiles.h -- global -> LDS staging of attention tiles for the gfx950 kernels.
#pragma once

#include "common.h"

namespace oomb {

// LDS strides, in elements.  Row-major tiles pad each D-row by 16 bytes and
// transposed tiles pad each 32-entry row by 16 bytes, so that the 16-byte
// operand reads of consecutive lanes fall in different banks.
template <typename T, int D> struct TileDims {
  static constexpr int VEC = 16 / (int)sizeof(T);  // elements per 16-byte load
  static constexpr int CPR = D / VEC;             // 16-byte loads per row
  static constexpr int RM = D + VEC;              // row-major row stride
  static constexpr int TR = 32 + VEC;             // transposed row stride
};

// Stage BR rows of D elements into LDS.  Row i starts at element off[i] of src
// (off[i] < 0: a row of zeros).  With RMAJ the tile is written row-major,
// rm[i * RM + d]; with TRAN it is also written transposed in operand order,
// tr[(i / 32) * D * TR + d * TR + operand_pos(i % 32)], which is how an A
// operand meets an accumulator reused as the B operand.
template <typename T, int D, int BR, bool RMAJ, bool TRAN, int NT = 256>
__device__ __forceinline__ void stage_tile(const T* __restrict__ src, const int64_t* off, T* rm, T* tr,
                                           int tid) {
  typedef TileDims<T, D> TD;
#pragma unroll 2
  for (int i = tid; i < BR * TD::CPR; i += NT) {
    const int row = i / TD::CPR, cg = i % TD::CPR;
    const int64_t o = off[row];
    f32x4 raw = {0.f, 0.f, 0.f, 0.f};
    if (o >= 0) raw = *reinterpret_cast<const f32x4*>(src + o + cg * TD::VEC);
    if constexpr (RMAJ) *reinterpret_cast<f32x4*>(rm + row * TD::RM + cg * TD::VEC) = raw;
    if constexpr (TRAN) {
      const T* v = reinterpret_cast<const T*>(&raw);
      T* dst = tr + (row >> 5) * D * TD::TR + (cg * TD::VEC) * TD::TR + operand_pos(row & 31);
#pragma unroll
      for (int e = 0; e < TD::VEC; ++e) dst[e * TD::TR] = v[e];
    }
  }
}

}  // namespace oomb
