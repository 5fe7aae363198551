// attn_bwd.hip -- fused backward of paged top-K chunk attention on gfx950.
//
// Page "Out of the Memory Barrier" (OOMB), technical summary, section 2:
// "Paged Memory Management" -- the KV cache's gradients live in page-granular
// buffers and are accumulated in place, outside any autograd graph;
// "Page-level Sparse Attention" -- the pages chosen in the forward pass are
// reused here unchanged.
//
// Kernels, in stream order:
//   1. dt_kernel:   Dt[g][t] = dO[t][g] . O[t][g]                 (HBM-bound)
//   2. dkdv_kernel: key-major.  A workgroup owns 256 keys of one kv-head's key
//      list (4 waves x 64 keys; K and V stay in registers) and walks a share of
//      the query rows that see them in tiles of 64 rows, recomputing
//      S = Q K^T and dP = dO V^T on MFMA, then dV^T += dO^T P and
//      dK^T += Q^T dS (dO^T and Q^T read transposed from the row-major LDS
//      tiles).  When the rows are split over several workgroups for load
//      balance, each writes its partial sums to the workspace.
//   3. kv_reduce_kernel (only with a row split): dk_pool/dv_pool += the sum of
//      the partials, in split order.
//   4. dq_kernel:   query-major, like the forward: S^T and dP^T per key tile,
//      dQ^T += K^T dS^T, written once per row.
// Every (slot, kv-head, row) of the gradient pools is changed by exactly one
// thread, once, in a fixed order: no atomics, bitwise reproducible, and slots
// outside the selected and chunk pages are never touched.  P and dS are
// rounded to the input type before they enter an MFMA.
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
  float* dt;       // workspace [Hq][C]
  float* part_k;   // workspace [splits][Hkv][nkeys][D], scaled dK partials
  float* part_v;   // workspace [splits][Hkv][nkeys][D]
  int splits;
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
// dK / dV, key-major.  Four waves (one per SIMD, so up to 512 registers each);
// a wave owns NKB key blocks of 32 keys (64 keys for bf16): every A operand
// read from LDS then feeds NKB MFMAs.
// ---------------------------------------------------------------------------
constexpr int kKvWaves = 4;
template <typename T> constexpr int kv_nkb() { return sizeof(T) == 2 ? 2 : 1; }  // 32-key blocks per wave
template <typename T> constexpr int kv_keys() { return kKvWaves * 32 * kv_nkb<T>(); }  // keys per workgroup
template <typename T> constexpr int kv_bm() { return sizeof(T) == 2 ? 64 : 32; }  // query rows per tile

struct KvPlan {
  int nkb, splits;
};

__host__ __device__ inline KvPlan kv_plan(const Geo& g, int keys_per_wg) {
  KvPlan p;
  const int nkeys = (g.keff << g.ps_log2) + g.c;
  p.nkb = (nkeys + keys_per_wg - 1) / keys_per_wg;
  const int items = p.nkb * g.hkv;
  int s = (512 + items - 1) / items;  // at least two workgroups per CU over the launch
  p.splits = s < 1 ? 1 : (s > 8 ? 8 : s);
  return p;
}

template <typename T, int D>
__global__ __launch_bounds__(kKvWaves * 64) void dkdv_kernel(BwdArgs a) {
  typedef Mma<T> M;
  constexpr int BM = kv_bm<T>(), NKB = kv_nkb<T>(), KEYS = kv_keys<T>();
  typedef Tile<T, D, BM> TL;
  constexpr int KS = M::KS, KL = M::KL, NT = kKvWaves * 64;
  __shared__ __attribute__((aligned(16))) T lds_q[2 * TL::ELEMS];
  __shared__ __attribute__((aligned(16))) T lds_d[2 * TL::ELEMS];
  __shared__ float rlse[2][BM], rdt[2][BM];
  __shared__ int rtok[2][BM];

  const Geo& g = a.g;
  const KvPlan plan = kv_plan(g, KEYS);
  const int item = xcd_remap(blockIdx.x, plan.nkb * plan.splits * g.hkv);
  const int h = item / (plan.nkb * plan.splits);
  const int kblk = (item / plan.splits) % plan.nkb;
  const int sp = item % plan.splits;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, hh = lane >> 5;
  const int pk = g.keff << g.ps_log2;
  const int nkeys = pk + g.c;
  const int jb = kblk * KEYS;

  // this lane's keys (one per 32-key block) and their K^T / V^T B operands:
  // lane (key col, half hh) holds K[key][s*KS + hh*KL + i]
  int my_key[NKB], my_u[NKB];
  bool key_ok[NKB];
  int64_t koff[NKB];
  typename M::frag kf[NKB][D / KS], vf[NKB][D / KS];
#pragma unroll
  for (int kk = 0; kk < NKB; ++kk) {
    my_key[kk] = jb + (wave * NKB + kk) * 32 + col;
    key_ok[kk] = my_key[kk] < nkeys;
    koff[kk] = key_ok[kk] ? key_offset<D>(g, a.pt, a.sel, h, my_key[kk]) : 0;
    my_u[kk] = my_key[kk] - pk;  // chunk token index when >= 0
#pragma unroll
    for (int s = 0; s < D / KS; ++s) {
      kf[kk][s] = key_ok[kk] ? M::load((const T*)a.k + koff[kk] + s * KS + hh * KL) : M::zero();
      vf[kk][s] = key_ok[kk] ? M::load((const T*)a.v + koff[kk] + s * KS + hh * KL) : M::zero();
    }
  }
  f32x16 dkacc[NKB][D / 32], dvacc[NKB][D / 32];
#pragma unroll
  for (int kk = 0; kk < NKB; ++kk)
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      dkacc[kk][db] = zero16();
      dvacc[kk][db] = zero16();
    }

  // rows that can see a key of this block: all rows for prior keys, else rows
  // of chunk tokens t >= the block's first chunk token; this split's share
  const int rows_total = g.c * g.G;
  const int row_start = jb < pk ? 0 : (jb - pk) * g.G;
  const int ntile_all = (rows_total - row_start + BM - 1) / BM;
  const int tile_lo = (int)((int64_t)ntile_all * sp / plan.splits);
  const int tile_hi = (int)((int64_t)ntile_all * (sp + 1) / plan.splits);

  const T* __restrict__ qp = (const T*)a.q;
  const T* __restrict__ dp = (const T*)a.dout;
  PairStages<T, D, BM, NT> qd{lds_q, lds_d};
  // rows past the end are clamped to the last row (finite data, zero weight below)
  auto rows_from = [&](int r0) {
    return [&, r0](int r) -> int64_t {
      const int rr = min(r0 + r, rows_total - 1);
      return ((int64_t)(rr / g.G) * g.hq + h * g.G + rr % g.G) * D;
    };
  };
  float nlse = 0.f, ndt = 0.f;
  int ntok = -1;
  auto fetch = [&](int r0, int stage) {
    qd.load(stage, qp, dp, tid, rows_from(r0));
    if (tid < BM) {
      const int r = r0 + tid;
      ntok = -1;
      nlse = 0.f;
      ndt = 0.f;
      if (r < rows_total) {
        const int t = r / g.G, qh = h * g.G + r % g.G;
        ntok = t;
        nlse = a.lse[(int64_t)qh * g.c + t] * kLog2e;
        ndt = a.dt[(int64_t)qh * g.c + t];
      }
    }
  };
  auto stash = [&](int stage) {
    qd.commit(stage, tid);
    if (tid < BM) {
      rlse[stage][tid] = nlse;
      rdt[stage][tid] = ndt;
      rtok[stage][tid] = ntok;
    }
  };

  if (tile_lo < tile_hi) {
    fetch(row_start + tile_lo * BM, 0);
    stash(0);
  }
  __syncthreads();
  for (int it = tile_lo; it < tile_hi; ++it) {
    const int stage = (it - tile_lo) & 1;
    if (it + 1 < tile_hi) fetch(row_start + (it + 1) * BM, stage ^ 1);
    const TL tq = qd.ta(stage), td = qd.tb(stage);
#pragma unroll 1
    for (int rb = 0; rb < BM / 32; ++rb) {
      f32x16 sacc[NKB], pacc[NKB];
#pragma unroll
      for (int kk = 0; kk < NKB; ++kk) {
        sacc[kk] = zero16();
        pacc[kk] = zero16();
      }
#pragma unroll
      for (int s = 0; s < D / KS; ++s) {
        const typename M::frag fq = tq.frag_rm(rb * 32 + col, s, hh);
#pragma unroll
        for (int kk = 0; kk < NKB; ++kk) sacc[kk] = M::mma(fq, kf[kk][s], sacc[kk]);
      }
#pragma unroll
      for (int s = 0; s < D / KS; ++s) {
        const typename M::frag fd = td.frag_rm(rb * 32 + col, s, hh);
#pragma unroll
        for (int kk = 0; kk < NKB; ++kk) pacc[kk] = M::mma(fd, vf[kk][s], pacc[kk]);
      }
      // element e of a lane: query row rb*32 + acc_row(e, hh), key my_key[kk]
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int r = rb * 32 + acc_row(e, hh);
        const int t = rtok[stage][r];
        const float l2 = rlse[stage][r], dt = rdt[stage][r];
#pragma unroll
        for (int kk = 0; kk < NKB; ++kk) {
          const bool vis = key_ok[kk] && t >= 0 && my_u[kk] <= t;  // my_u < 0 for prior keys
          const float p = vis ? __builtin_amdgcn_exp2f(fmaf(sacc[kk][e], a.scale_log2, -l2)) : 0.f;
          sacc[kk][e] = p;
          pacc[kk][e] = p * (pacc[kk][e] - dt);
        }
      }
#pragma unroll
      for (int s = 0; s < 32 / KS; ++s) {
        typename M::frag pf[NKB], sf[NKB];
#pragma unroll
        for (int kk = 0; kk < NKB; ++kk) {
          pf[kk] = M::pack(sacc[kk], s * KL);
          sf[kk] = M::pack(pacc[kk], s * KL);
        }
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const typename M::frag fdt = td.frag_tr(rb, db, s, lane);
#pragma unroll
          for (int kk = 0; kk < NKB; ++kk) dvacc[kk][db] = M::mma(fdt, pf[kk], dvacc[kk][db]);
          const typename M::frag fqt = tq.frag_tr(rb, db, s, lane);
#pragma unroll
          for (int kk = 0; kk < NKB; ++kk) dkacc[kk][db] = M::mma(fqt, sf[kk], dkacc[kk][db]);
        }
      }
    }
    if (it + 1 < tile_hi) stash(stage ^ 1);
    __syncthreads();
  }

  const float sc = g.scale;
#pragma unroll
  for (int kk = 0; kk < NKB; ++kk) {
    if (!key_ok[kk]) continue;
    if (plan.splits == 1) {
      float* dkp = a.dk + koff[kk];
      float* dvp = a.dv + koff[kk];
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
          const int d = db * 32 + 8 * e4 + 4 * hh;
          f32x4 ok = *reinterpret_cast<f32x4*>(dkp + d);
          f32x4 ov = *reinterpret_cast<f32x4*>(dvp + d);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            ok[i] += sc * dkacc[kk][db][4 * e4 + i];
            ov[i] += dvacc[kk][db][4 * e4 + i];
          }
          *reinterpret_cast<f32x4*>(dkp + d) = ok;
          *reinterpret_cast<f32x4*>(dvp + d) = ov;
        }
    } else {
      const int64_t base = (((int64_t)sp * g.hkv + h) * nkeys + my_key[kk]) * D;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
          const int d = db * 32 + 8 * e4 + 4 * hh;
          f32x4 wk, wv;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            wk[i] = sc * dkacc[kk][db][4 * e4 + i];
            wv[i] = dvacc[kk][db][4 * e4 + i];
          }
          *reinterpret_cast<f32x4*>(a.part_k + base + d) = wk;
          *reinterpret_cast<f32x4*>(a.part_v + base + d) = wv;
        }
    }
  }
}

// dk_pool / dv_pool += sum over splits of the partials (fixed order).
template <int D>
__global__ __launch_bounds__(256) void kv_reduce_kernel(BwdArgs a) {
  const Geo& g = a.g;
  const int nkeys = (g.keff << g.ps_log2) + g.c;
  const int64_t total = (int64_t)g.hkv * nkeys * (D / 4);
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= total) return;
  const int d = (int)(i % (D / 4)) * 4;
  const int64_t hk = i / (D / 4);
  const int h = (int)(hk / nkeys), jj = (int)(hk % nkeys);
  const int64_t stride = (int64_t)g.hkv * nkeys * D;
  const int64_t src = hk * D + d;
  f32x4 sk = *reinterpret_cast<const f32x4*>(a.part_k + src);
  f32x4 sv = *reinterpret_cast<const f32x4*>(a.part_v + src);
  for (int s = 1; s < a.splits; ++s) {
    sk += *reinterpret_cast<const f32x4*>(a.part_k + s * stride + src);
    sv += *reinterpret_cast<const f32x4*>(a.part_v + s * stride + src);
  }
  const int64_t dst = key_offset<D>(g, a.pt, a.sel, h, jj) + d;
  f32x4 ok = *reinterpret_cast<f32x4*>(a.dk + dst);
  f32x4 ov = *reinterpret_cast<f32x4*>(a.dv + dst);
  *reinterpret_cast<f32x4*>(a.dk + dst) = ok + sk;
  *reinterpret_cast<f32x4*>(a.dv + dst) = ov + sv;
}

// ---------------------------------------------------------------------------
// dQ, query-major.
// ---------------------------------------------------------------------------
constexpr int kDqWaves = 8;
constexpr int kDqBM = 32 * kDqWaves;  // query rows per workgroup
template <typename T> constexpr int dq_bn() { return sizeof(T) == 2 ? 64 : 32; }  // keys per tile

template <typename T, int D>
__global__ __launch_bounds__(kDqWaves * 64) void dq_kernel(BwdArgs a) {
  typedef Mma<T> M;
  constexpr int BN = dq_bn<T>();
  typedef Tile<T, D, BN> TL;
  constexpr int KS = M::KS, KL = M::KL, NT = kDqWaves * 64;
  __shared__ __attribute__((aligned(16))) T lds_k[2 * TL::ELEMS];
  __shared__ __attribute__((aligned(16))) T lds_v[2 * TL::ELEMS];

  const Geo& g = a.g;
  const int rows_total = g.c * g.G;
  const int nrb = (rows_total + kDqBM - 1) / kDqBM;
  const int item = xcd_remap(blockIdx.x, nrb * g.hkv);
  const int h = item / nrb;
  const int r0 = (nrb - 1 - item % nrb) * kDqBM;  // later (heavier) row blocks first

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, hh = lane >> 5;
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
  const int t_lo = r0 / g.G;
  const int nkeys = pk + last_row / g.G + 1;
  const int ntiles = (nkeys + BN - 1) / BN;

  const T* __restrict__ kp = (const T*)a.k;
  const T* __restrict__ vp = (const T*)a.v;
  PairStages<T, D, BN, NT> kv{lds_k, lds_v};
  auto rows_from = [&](int j0) {
    return [&, j0](int r) -> int64_t { return key_offset<D>(g, a.pt, a.sel, h, min(j0 + r, nkeys - 1)); };
  };

  f32x16 qacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) qacc[db] = zero16();

  kv.load(0, kp, vp, tid, rows_from(0));
  kv.commit(0, tid);
  __syncthreads();
  for (int it = 0; it < ntiles; ++it) {
    const int j0 = it * BN;
    if (it + 1 < ntiles) kv.load((it + 1) & 1, kp, vp, tid, rows_from(j0 + BN));
    const TL tk = kv.ta(it & 1), tv = kv.tb(it & 1);
    const bool masked = j0 + BN - 1 - pk > t_lo || j0 + BN > nkeys;
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb) {
      f32x16 sacc = zero16(), pacc = zero16();
#pragma unroll
      for (int s = 0; s < D / KS; ++s) {
        sacc = M::mma(tk.frag_rm(kb * 32 + col, s, hh), qf[s], sacc);
        pacc = M::mma(tv.frag_rm(kb * 32 + col, s, hh), df[s], pacc);
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int j = j0 + kb * 32 + acc_row(e, hh);
        const bool vis = !masked || (j < nkeys && (j < pk || j - pk <= my_t));
        const float p = vis ? __builtin_amdgcn_exp2f(fmaf(sacc[e], a.scale_log2, -my_lse)) : 0.f;
        pacc[e] = p * (pacc[e] - my_dt);
      }
#pragma unroll
      for (int s = 0; s < 32 / KS; ++s) {
        const typename M::frag sf = M::pack(pacc, s * KL);
#pragma unroll
        for (int db = 0; db < D / 32; ++db) qacc[db] = M::mma(tk.frag_tr(kb, db, s, lane), sf, qacc[db]);
      }
    }
    if (it + 1 < ntiles) kv.commit((it + 1) & 1, tid);
    __syncthreads();
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
  const KvPlan kp = kv_plan(make_geo(s), s.bf16 ? kv_keys<__bf16>() : kv_keys<float>());
  const size_t nkeys = (size_t)s.keff * s.ps + s.c;
  p.off_dt = 0;
  size_t off = (((size_t)s.hq * s.c * 4) + 255) & ~(size_t)255;
  p.splits = kp.splits;
  p.off_part_k = off;
  const size_t part = kp.splits > 1 ? (size_t)kp.splits * s.hkv * nkeys * s.d * 4 : 0;
  off += (part + 255) & ~(size_t)255;
  p.off_part_v = off;
  off += (part + 255) & ~(size_t)255;
  p.bytes = off;
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
  const KvPlan kp = kv_plan(a.g, kv_keys<T>());
  {
    Traced tr(st, "dkdv_kernel");
    hipLaunchKernelGGL((dkdv_kernel<T, D>), dim3(kp.nkb * kp.splits * a.g.hkv), dim3(kKvWaves * 64), 0, st, a);
  }
  if (kp.splits > 1) {
    const int64_t nkeys = (a.g.keff << a.g.ps_log2) + a.g.c;
    const int64_t total = a.g.hkv * nkeys * (D / 4);
    Traced tr(st, "kv_reduce_kernel");
    hipLaunchKernelGGL((kv_reduce_kernel<D>), dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, a);
  }
  const int qrows = a.g.c * a.g.G;
  {
    Traced tr(st, "dq_kernel");
    hipLaunchKernelGGL((dq_kernel<T, D>), dim3(((qrows + kDqBM - 1) / kDqBM) * a.g.hkv), dim3(kDqWaves * 64), 0,
                       st, a);
  }
  return hipGetLastError();
}

hipError_t launch_bwd(const Shape& s, const void* q, const void* k_pool, const void* v_pool, const int32_t* pt,
                      const int32_t* sel, const void* o, const float* lse, const void* dout, float* dq,
                      float* dk_pool, float* dv_pool, void* ws, hipStream_t st) {
  const BwdPlan p = bwd_plan(s);
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
  a.dt = (float*)((char*)ws + p.off_dt);
  a.part_k = (float*)((char*)ws + p.off_part_k);
  a.part_v = (float*)((char*)ws + p.off_part_v);
  a.splits = p.splits;
  a.g = make_geo(s);
  a.scale_log2 = s.scale * kLog2e;
  if (s.bf16) return s.d == 128 ? bwd_t<__bf16, 128>(a, st) : bwd_t<__bf16, 64>(a, st);
  return s.d == 128 ? bwd_t<float, 128>(a, st) : bwd_t<float, 64>(a, st);
}

}  // namespace oomb
