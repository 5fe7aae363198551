// attn_fwd.hip -- fused forward of paged top-K chunk attention on gfx950.
//
// Page "Out of the Memory Barrier" (OOMB), technical summary, section 2: each
// chunk attends to the top-K pages chosen for its kv-head ("Page-level Sparse
// Attention") plus its own tokens, causally; the KV cache is read in place
// from its pages ("Paged Memory Management").  The forward saves O and the
// log-sum-exp for the backward.
//
// Work split: one workgroup = one kv-head h and 128 query rows of that head's
// C*G rows (row r = token r / G, query head h*G + r % G), so every K/V tile
// staged in LDS serves all G query heads of the group.  Four waves own 32 rows
// each.  Scores are computed transposed, S^T = K Q^T on bf16 MFMA 32x32x16
// (fp32 MFMA 32x32x2 for fp32 inputs): a lane then owns one query row, and the
// online-softmax max and sum are in-lane plus one cross-half exchange.  P^T
// (rounded to the input type) is reused in registers as the B operand of
// O^T += V^T P^T, whose A operand comes from V staged transposed in operand
// order.
#include "common.h"
#include "launch.h"
#include "tiles.h"
#include "trace.h"

namespace oomb {

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* pt;
  const int32_t* sel;
  void* o;
  float* lse;
  Geo g;
  float scale_log2;  // softmax scale * log2(e)
};

constexpr int kFwdBM = 128;  // query rows per workgroup
constexpr int kFwdBN = 64;   // keys per tile

template <typename T, int D>
__global__ __launch_bounds__(256, 2) void fwd_kernel(FwdArgs a) {
  typedef Mma<T> M;
  typedef TileDims<T, D> TD;
  constexpr int KS = M::KS, KL = M::KL, BN = kFwdBN;
  __shared__ __attribute__((aligned(16))) T Ks[BN * TD::RM];
  __shared__ __attribute__((aligned(16))) T Vt[(BN / 32) * D * TD::TR];
  __shared__ int64_t koff[BN];

  const Geo& g = a.g;
  const T* __restrict__ q = (const T*)a.q;
  const int h = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, hh = lane >> 5;
  const int rows_total = g.c * g.G;
  const int r0 = blockIdx.x * kFwdBM;
  const int my_row = r0 + wave * 32 + col;
  const bool row_ok = my_row < rows_total;
  const int my_t = row_ok ? my_row / g.G : g.c - 1;
  const int my_g = h * g.G + (row_ok ? my_row % g.G : 0);

  // Q^T as B operands: lane (row col, half hh) holds Q[row][s*KS + hh*KL + i]
  typename M::frag qf[D / KS];
  const T* qrow = q + ((int64_t)my_t * g.hq + my_g) * D;
#pragma unroll
  for (int s = 0; s < D / KS; ++s) qf[s] = row_ok ? M::load(qrow + s * KS + hh * KL) : M::zero();

  const int pk = g.keff << g.ps_log2;
  const int last_row = min(r0 + kFwdBM, rows_total) - 1;
  const int nkeys = pk + last_row / g.G + 1;  // prior keys + chunk tokens up to the block's last

  float m = -INFINITY, l = 0.f;
  f32x16 oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) oacc[db] = zero16();

  for (int j0 = 0; j0 < nkeys; j0 += BN) {
    __syncthreads();
    if (tid < BN) koff[tid] = (j0 + tid < nkeys) ? key_offset<D>(g, a.pt, a.sel, h, j0 + tid) : (int64_t)-1;
    __syncthreads();
    stage_tile<T, D, BN, true, false>((const T*)a.k, koff, Ks, nullptr, tid);
    stage_tile<T, D, BN, false, true>((const T*)a.v, koff, nullptr, Vt, tid);
    __syncthreads();

    f32x16 sacc[BN / 32];
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb) {
      sacc[kb] = zero16();
#pragma unroll
      for (int s = 0; s < D / KS; ++s)
        sacc[kb] = M::mma(M::load(&Ks[(kb * 32 + col) * TD::RM + s * KS + hh * KL]), qf[s], sacc[kb]);
    }
    const bool need_mask = j0 + BN > pk;  // the tile reaches chunk tokens or the tail
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        float x = sacc[kb][e] * a.scale_log2;
        if (need_mask) {
          const int j = j0 + kb * 32 + acc_row(e, hh);
          if (j >= nkeys || (j >= pk && j - pk > my_t)) x = -INFINITY;
        }
        sacc[kb][e] = x;
        mx = fmaxf(mx, x);
      }
    mx = wave_xor_max(mx, 32);
    const float m_new = fmaxf(m, mx);
    const bool any = m_new != -INFINITY;
    const float alpha = any ? exp2f(m - m_new) : 1.f;
    float rs = 0.f;
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float p = any ? exp2f(sacc[kb][e] - m_new) : 0.f;
        sacc[kb][e] = p;
        rs += p;
      }
    rs = wave_xor_sum(rs, 32);
    l = l * alpha + rs;
    m = m_new;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) oacc[db][e] *= alpha;

#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
      for (int s = 0; s < 32 / KS; ++s) {
        const typename M::frag pf = M::pack(sacc[kb], s * KL);
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
          oacc[db] = M::mma(M::load(&Vt[kb * D * TD::TR + (db * 32 + col) * TD::TR + hh * 16 + s * KL]), pf,
                            oacc[db]);
      }
  }

  if (row_ok) {
    const float inv = 1.f / l;
    T* orow = (T*)a.o + ((int64_t)my_t * g.hq + my_g) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const int d = db * 32 + 8 * e4 + 4 * hh;
        if constexpr (sizeof(T) == 2) {
          bf16x4 w;
#pragma unroll
          for (int i = 0; i < 4; ++i) w[i] = (__bf16)(oacc[db][4 * e4 + i] * inv);
          *reinterpret_cast<bf16x4*>(orow + d) = w;
        } else {
          f32x4 w;
#pragma unroll
          for (int i = 0; i < 4; ++i) w[i] = oacc[db][4 * e4 + i] * inv;
          *reinterpret_cast<f32x4*>(orow + d) = w;
        }
      }
    if (hh == 0) a.lse[(int64_t)my_g * g.c + my_t] = (m + log2f(l)) * kLn2;
  }
}

hipError_t launch_fwd(const Shape& s, const void* q, const void* k_pool, const void* v_pool, const int32_t* pt,
                      const int32_t* sel, void* o, float* lse, hipStream_t st) {
  FwdArgs a;
  a.q = q;
  a.k = k_pool;
  a.v = v_pool;
  a.pt = pt;
  a.sel = sel;
  a.o = o;
  a.lse = lse;
  a.g = make_geo(s);
  a.scale_log2 = s.scale * kLog2e;
  const int rows = s.c * (s.hq / s.hkv);
  dim3 grid((rows + kFwdBM - 1) / kFwdBM, s.hkv);
  Traced tr(st, "fwd_kernel");
  if (s.bf16) {
    if (s.d == 128) hipLaunchKernelGGL((fwd_kernel<__bf16, 128>), grid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((fwd_kernel<__bf16, 64>), grid, dim3(256), 0, st, a);
  } else {
    if (s.d == 128) hipLaunchKernelGGL((fwd_kernel<float, 128>), grid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((fwd_kernel<float, 64>), grid, dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace oomb
