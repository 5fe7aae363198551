// attn_bwd.hip -- fused backward of paged top-K chunk attention on gfx950.
//
// Page "Out of the Memory Barrier" (OOMB), technical summary, section 2:
// "Paged Memory Management" -- the KV cache's gradients live in page-granular
// buffers and are accumulated in place, outside any autograd graph;
// "Page-level Sparse Attention" -- the pages chosen in the forward pass are
// reused here unchanged.
//
// Three kernels on one stream:
//   1. dt_kernel:   Dt[g][t] = dO[t][g] . O[t][g]                (HBM-bound)
//   2. dkdv_kernel: key-major.  A workgroup owns 128 keys of one kv-head's key
//      list (4 waves x 32 keys, K and V held in registers) and walks every query
//      row that sees them, recomputing S = Q K^T and dP = dO V^T on MFMA, then
//      dV^T += dO^T P and dK^T += Q^T dS.  Each (slot, kv-head, row) of the
//      gradient pools has exactly one owner, which adds its sums in place once:
//      no atomics, bitwise reproducible, untouched slots stay untouched.
//   3. dq_kernel:   query-major, like the forward: S^T and dP^T per key tile,
//      dQ^T += K^T dS^T, written (not accumulated) once per row.
// P and dS are rounded to the input type before they enter an MFMA.
#include "common.h"
#include "launch.h"
#include "tiles.h"
#include "trace.h"

namespace oomb {

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* pt;
  const int32_t* sel;
  const void* o;
  const float* lse;
  const void* dout;
  float* dq;
  float* dk;
  float* dv;
  float* dt;  // workspace [Hq][C]
  Geo g;
  float scale_log2;
};

// ---------------------------------------------------------------------------
// Dt = rowsum(dO * O), one row per group of D/VEC lanes.
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void dt_kernel(BwdArgs a) {
  constexpr int VEC = 16 / (int)sizeof(T);
  constexpr int LPR = D / VEC;  // lanes per row (power of two, <= 32)
  const int rows = a.g.c * a.g.hq;
  const int lane_in_row = threadIdx.x % LPR;
  const int row = blockIdx.x * (256 / LPR) + threadIdx.x / LPR;
  float s = 0.f;
  if (row < rows) {
    const int64_t off = (int64_t)row * D + lane_in_row * VEC;
    const f32x4 ro = *reinterpret_cast<const f32x4*>((const T*)a.o + off);
    const f32x4 rd = *reinterpret_cast<const f32x4*>((const T*)a.dout + off);
    const T* po = reinterpret_cast<const T*>(&ro);
    const T* pd = reinterpret_cast<const T*>(&rd);
#pragma unroll
    for (int i = 0; i < VEC; ++i) s += (float)po[i] * (float)pd[i];
  }
#pragma unroll
  for (int m = LPR / 2; m >= 1; m >>= 1) s = wave_xor_sum(s, m);
  if (row < rows && lane_in_row == 0) {
    const int t = row / a.g.hq, g = row % a.g.hq;  // row = t * Hq + g
    a.dt[(int64_t)g * a.g.c + t] = s;
  }
}

// ---------------------------------------------------------------------------
// dK / dV, key-major.
// ---------------------------------------------------------------------------
constexpr int kKvKeys = 128;  // keys per workgroup (32 per wave)
constexpr int kKvBM = 64;     // query rows per tile

template <typename T, int D>
__global__ __launch_bounds__(256, 1) void dkdv_kernel(BwdArgs a) {
  typedef Mma<T> M;
  typedef TileDims<T, D> TD;
  constexpr int KS = M::KS, KL = M::KL, BM = kKvBM;
  __shared__ __attribute__((aligned(16))) T Qs[BM * TD::RM];
  __shared__ __attribute__((aligned(16))) T Ds[BM * TD::RM];
  __shared__ __attribute__((aligned(16))) T Qt[(BM / 32) * D * TD::TR];
  __shared__ __attribute__((aligned(16))) T Dtr[(BM / 32) * D * TD::TR];
  __shared__ int64_t roff[BM];
  __shared__ float rlse[BM], rdt[BM];
  __shared__ int rtok[BM];

  const Geo& g = a.g;
  const int h = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, hh = lane >> 5;
  const int pk = g.keff << g.ps_log2;
  const int nkeys = pk + g.c;
  const int jb = blockIdx.x * kKvKeys;
  const int my_key = jb + wave * 32 + col;
  const bool key_ok = my_key < nkeys;
  const int64_t koff = key_ok ? key_offset<D>(g, a.pt, a.sel, h, my_key) : 0;
  const int my_u = my_key - pk;  // chunk token index when >= 0

  // K^T and V^T as B operands: lane (key col, half hh) holds K[key][s*KS + hh*KL + i]
  typename M::frag kf[D / KS], vf[D / KS];
#pragma unroll
  for (int s = 0; s < D / KS; ++s) {
    kf[s] = key_ok ? M::load((const T*)a.k + koff + s * KS + hh * KL) : M::zero();
    vf[s] = key_ok ? M::load((const T*)a.v + koff + s * KS + hh * KL) : M::zero();
  }
  f32x16 dkacc[D / 32], dvacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    dkacc[db] = zero16();
    dvacc[db] = zero16();
  }

  // rows that can see any key of this block: all rows for prior keys, else
  // rows of chunk tokens t >= the block's first chunk token
  const int rows_total = g.c * g.G;
  const int row_start = jb < pk ? 0 : (jb - pk) * g.G;

  for (int r0 = row_start; r0 < rows_total; r0 += BM) {
    __syncthreads();
    if (tid < BM) {
      const int r = r0 + tid;
      if (r < rows_total) {
        const int t = r / g.G, qh = h * g.G + r % g.G;
        roff[tid] = ((int64_t)t * g.hq + qh) * D;
        rlse[tid] = a.lse[(int64_t)qh * g.c + t] * kLog2e;
        rdt[tid] = a.dt[(int64_t)qh * g.c + t];
        rtok[tid] = t;
      } else {
        roff[tid] = -1;
        rlse[tid] = 0.f;
        rdt[tid] = 0.f;
        rtok[tid] = -1;
      }
    }
    __syncthreads();
    stage_tile<T, D, BM, true, true>((const T*)a.q, roff, Qs, Qt, tid);
    stage_tile<T, D, BM, true, true>((const T*)a.dout, roff, Ds, Dtr, tid);
    __syncthreads();

#pragma unroll
    for (int rb = 0; rb < BM / 32; ++rb) {
      f32x16 sacc = zero16(), pacc = zero16();
#pragma unroll
      for (int s = 0; s < D / KS; ++s) {
        sacc = M::mma(M::load(&Qs[(rb * 32 + col) * TD::RM + s * KS + hh * KL]), kf[s], sacc);
        pacc = M::mma(M::load(&Ds[(rb * 32 + col) * TD::RM + s * KS + hh * KL]), vf[s], pacc);
      }
      // element e of this lane: query row rb*32 + acc_row(e, hh), key my_key
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int r = rb * 32 + acc_row(e, hh);
        const int t = rtok[r];
        const bool vis = key_ok && t >= 0 && (my_u < 0 || my_u <= t);
        const float p = vis ? exp2f(sacc[e] * a.scale_log2 - rlse[r]) : 0.f;
        sacc[e] = p;
        pacc[e] = p * (pacc[e] - rdt[r]);
      }
#pragma unroll
      for (int s = 0; s < 32 / KS; ++s) {
        const typename M::frag pf = M::pack(sacc, s * KL);
        const typename M::frag sf = M::pack(pacc, s * KL);
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const int at = rb * D * TD::TR + (db * 32 + col) * TD::TR + hh * 16 + s * KL;
          dvacc[db] = M::mma(M::load(&Dtr[at]), pf, dvacc[db]);
          dkacc[db] = M::mma(M::load(&Qt[at]), sf, dkacc[db]);
        }
      }
    }
  }

  if (key_ok) {
    float* dkp = a.dk + koff;
    float* dvp = a.dv + koff;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const int d = db * 32 + 8 * e4 + 4 * hh;
        f32x4 ok = *reinterpret_cast<f32x4*>(dkp + d);
        f32x4 ov = *reinterpret_cast<f32x4*>(dvp + d);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          ok[i] += g.scale * dkacc[db][4 * e4 + i];
          ov[i] += dvacc[db][4 * e4 + i];
        }
        *reinterpret_cast<f32x4*>(dkp + d) = ok;
        *reinterpret_cast<f32x4*>(dvp + d) = ov;
      }
  }
}

// ---------------------------------------------------------------------------
// dQ, query-major.
// ---------------------------------------------------------------------------
constexpr int kDqBM = 128;  // query rows per workgroup
constexpr int kDqBN = 64;   // keys per tile

template <typename T, int D>
__global__ __launch_bounds__(256, 1) void dq_kernel(BwdArgs a) {
  typedef Mma<T> M;
  typedef TileDims<T, D> TD;
  constexpr int KS = M::KS, KL = M::KL, BN = kDqBN;
  __shared__ __attribute__((aligned(16))) T Ks[BN * TD::RM];
  __shared__ __attribute__((aligned(16))) T Vs[BN * TD::RM];
  __shared__ __attribute__((aligned(16))) T Kt[(BN / 32) * D * TD::TR];
  __shared__ int64_t koff[BN];

  const Geo& g = a.g;
  const int h = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, hh = lane >> 5;
  const int rows_total = g.c * g.G;
  const int r0 = blockIdx.x * kDqBM;
  const int my_row = r0 + wave * 32 + col;
  const bool row_ok = my_row < rows_total;
  const int my_t = row_ok ? my_row / g.G : g.c - 1;
  const int my_g = h * g.G + (row_ok ? my_row % g.G : 0);
  const int64_t qoff = ((int64_t)my_t * g.hq + my_g) * D;

  typename M::frag qf[D / KS], df[D / KS];
#pragma unroll
  for (int s = 0; s < D / KS; ++s) {
    qf[s] = row_ok ? M::load((const T*)a.q + qoff + s * KS + hh * KL) : M::zero();
    df[s] = row_ok ? M::load((const T*)a.dout + qoff + s * KS + hh * KL) : M::zero();
  }
  const float my_lse = row_ok ? a.lse[(int64_t)my_g * g.c + my_t] * kLog2e : 0.f;
  const float my_dt = row_ok ? a.dt[(int64_t)my_g * g.c + my_t] : 0.f;

  const int pk = g.keff << g.ps_log2;
  const int last_row = min(r0 + kDqBM, rows_total) - 1;
  const int nkeys = pk + last_row / g.G + 1;

  f32x16 qacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) qacc[db] = zero16();

  for (int j0 = 0; j0 < nkeys; j0 += BN) {
    __syncthreads();
    if (tid < BN) koff[tid] = (j0 + tid < nkeys) ? key_offset<D>(g, a.pt, a.sel, h, j0 + tid) : (int64_t)-1;
    __syncthreads();
    stage_tile<T, D, BN, true, true>((const T*)a.k, koff, Ks, Kt, tid);
    stage_tile<T, D, BN, true, false>((const T*)a.v, koff, Vs, nullptr, tid);
    __syncthreads();

#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb) {
      f32x16 sacc = zero16(), pacc = zero16();
#pragma unroll
      for (int s = 0; s < D / KS; ++s) {
        sacc = M::mma(M::load(&Ks[(kb * 32 + col) * TD::RM + s * KS + hh * KL]), qf[s], sacc);
        pacc = M::mma(M::load(&Vs[(kb * 32 + col) * TD::RM + s * KS + hh * KL]), df[s], pacc);
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int j = j0 + kb * 32 + acc_row(e, hh);
        const bool vis = j < nkeys && (j < pk || j - pk <= my_t);
        const float p = vis ? exp2f(sacc[e] * a.scale_log2 - my_lse) : 0.f;
        pacc[e] = p * (pacc[e] - my_dt);
      }
#pragma unroll
      for (int s = 0; s < 32 / KS; ++s) {
        const typename M::frag sf = M::pack(pacc, s * KL);
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
          qacc[db] = M::mma(M::load(&Kt[kb * D * TD::TR + (db * 32 + col) * TD::TR + hh * 16 + s * KL]), sf,
                            qacc[db]);
      }
    }
  }

  if (row_ok) {
    float* dqrow = a.dq + qoff;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        f32x4 w;
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = g.scale * qacc[db][4 * e4 + i];
        *reinterpret_cast<f32x4*>(dqrow + db * 32 + 8 * e4 + 4 * hh) = w;
      }
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
BwdPlan bwd_plan(const Shape& s) {
  BwdPlan p;
  p.off_dt = 0;
  p.bytes = (((size_t)s.hq * s.c * 4) + 255) & ~(size_t)255;
  return p;
}

template <typename T, int D>
static hipError_t bwd_t(const BwdArgs& a, hipStream_t st) {
  constexpr int LPR = D / (16 / (int)sizeof(T));
  const int rows = a.g.c * a.g.hq;
  {
    Traced tr(st, "dt_kernel");
    hipLaunchKernelGGL((dt_kernel<T, D>), dim3((rows + 256 / LPR - 1) / (256 / LPR)), dim3(256), 0, st, a);
  }
  const int pk = a.g.keff << a.g.ps_log2;
  const int nkeys = pk + a.g.c;
  {
    Traced tr(st, "dkdv_kernel");
    hipLaunchKernelGGL((dkdv_kernel<T, D>), dim3((nkeys + kKvKeys - 1) / kKvKeys, a.g.hkv), dim3(256), 0, st, a);
  }
  const int qrows = a.g.c * a.g.G;
  {
    Traced tr(st, "dq_kernel");
    hipLaunchKernelGGL((dq_kernel<T, D>), dim3((qrows + kDqBM - 1) / kDqBM, a.g.hkv), dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

hipError_t launch_bwd(const Shape& s, const void* q, const void* k_pool, const void* v_pool, const int32_t* pt,
                      const int32_t* sel, const void* o, const float* lse, const void* dout, float* dq,
                      float* dk_pool, float* dv_pool, void* ws, hipStream_t st) {
  BwdArgs a;
  a.q = q;
  a.k = k_pool;
  a.v = v_pool;
  a.pt = pt;
  a.sel = sel;
  a.o = o;
  a.lse = lse;
  a.dout = dout;
  a.dq = dq;
  a.dk = dk_pool;
  a.dv = dv_pool;
  a.dt = (float*)((char*)ws + bwd_plan(s).off_dt);
  a.g = make_geo(s);
  a.scale_log2 = s.scale * kLog2e;
  if (s.bf16) return s.d == 128 ? bwd_t<__bf16, 128>(a, st) : bwd_t<__bf16, 64>(a, st);
  return s.d == 128 ? bwd_t<float, 128>(a, st) : bwd_t<float, 64>(a, st);
}

}  // namespace oomb
