// attn_fwd.hip -- fused forward of paged top-K chunk attention on gfx950.
//
// Page "Out of the Memory Barrier" (OOMB), technical summary, section 2: each
// chunk attends to the top-K pages chosen for its kv-head ("Page-level Sparse
// Attention") plus its own tokens, causally; the KV cache is read in place
// from its pages ("Paged Memory Management").  The forward saves O and the
// log-sum-exp for the backward.
//
// Work split: one workgroup = one kv-head h and 256 query rows of that head's
// C*G rows (row r = token r / G, query head h*G + r % G), so every K/V tile
// staged in LDS serves all G query heads of the group.  Eight waves own 32 rows
// each (two per SIMD).
// Scores are computed transposed, S^T = K Q^T on bf16 MFMA 32x32x16 (fp32
// MFMA 32x32x2 for fp32 inputs): a lane owns one query row, and the softmax
// max and sum are in-lane plus one cross-half exchange.  P^T (rounded to the
// input type) is the B operand of O^T += V^T P^T, whose A operand is read
// transposed from the row-major V tile.  K/V tiles of 64 keys (32 for fp32)
// stream through a ring of LDS slots with one barrier per tile: fp32 inputs use
// two slots staged through registers (fwd_kernel); bf16 inputs use the
// software-pipelined fwd_pipe_kernel below with four direct-load slots.
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

constexpr int kFwdWaves = 8;
constexpr int kFwdBM = 32 * kFwdWaves;  // query rows per workgroup
template <typename T> constexpr int fwd_bn() { return sizeof(T) == 2 ? 64 : 32; }  // keys per tile
constexpr float kRescaleSlack = 8.f;    // log2 units a stale running max may lag the true one

template <typename T, int D>
__global__ __launch_bounds__(kFwdWaves * 64) void fwd_kernel(FwdArgs a) {
  typedef Mma<T> M;
  constexpr int BN = fwd_bn<T>(), NT = kFwdWaves * 64;
  typedef Ring<T, D, BN, NT> KV;
  typedef typename KV::TL TL;
  constexpr int KS = M::KS, KL = M::KL;
  __shared__ __attribute__((aligned(16))) T lds_k[KV::NS * TL::ELEMS];
  __shared__ __attribute__((aligned(16))) T lds_v[KV::NS * TL::ELEMS];
  __shared__ int page_tab[kPageCache];

  const Geo& g = a.g;
  const int rows_total = g.c * g.G;
  const int nrb = (rows_total + kFwdBM - 1) / kFwdBM;
  const RowItem it = row_item(blockIdx.x, nrb, g.hkv);
  const int h = it.h;
  const int r0 = (nrb - 1 - it.rank) * kFwdBM;  // later (heavier) row blocks first

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, hh = lane >> 5;
  const int my_row = r0 + wave * 32 + col;
  const bool row_ok = my_row < rows_total;
  const int my_t = row_ok ? div_g(g, my_row) : g.c - 1;
  const int my_g = h * g.G + (row_ok ? my_row - div_g(g, my_row) * g.G : 0);

  // Q^T as B operands: lane (row col, half hh) holds Q[row][s*KS + hh*KL + i]
  typename M::frag qf[D / KS];
  const T* qrow = (const T*)a.q + ((int64_t)my_t * g.hq + my_g) * D;
#pragma unroll
  for (int s = 0; s < D / KS; ++s) qf[s] = row_ok ? M::load(qrow + s * KS + hh * KL) : M::zero();

  const int pk = g.keff << g.ps_log2;
  const int last_row = min(r0 + kFwdBM, rows_total) - 1;
  const int t_lo = div_g(g, r0);
  const int nkeys = pk + div_g(g, last_row) + 1;  // prior keys + chunk tokens up to the block's last
  const int ntiles = (nkeys + BN - 1) / BN;
  PageSlots<kPageCache> pages{(lds_int*)page_tab};
  pages.fill(g, a.pt, a.sel, h, (nkeys + (1 << g.ps_log2) - 1) >> g.ps_log2, tid, NT);
  __syncthreads();

  const T* __restrict__ kp = (const T*)a.k;
  const T* __restrict__ vp = (const T*)a.v;
  KV kv{lds_k, lds_v};
  // When a tile lies inside one page (page size a multiple of the tile), its
  // rows are consecutive in the pool and one page lookup per tile suffices;
  // rows past the key list then read the rest of that page (finite data,
  // masked below).  Otherwise every row is looked up, clamped to the last key.
  const bool tile_in_page = BN <= (1 << g.ps_log2);
  auto load = [&](int j) {
    if (tile_in_page) {
      const int64_t base = pages.key_offset<D>(g, a.pt, a.sel, h, j * BN);
      kv.load(j, kp, vp, tid, [base](int r) -> int64_t { return base + (int64_t)r * D; });
    } else {
      kv.load(j, kp, vp, tid, [&, j](int r) -> int64_t {
        return pages.key_offset<D>(g, a.pt, a.sel, h, min(j * BN + r, nkeys - 1));
      });
    }
  };
  const int vm_per_tile = KV::loads_per_tile(wave);

  float m_ref = -INFINITY, l = 0.f;  // running max (log2 domain) and this lane's partial sum
  f32x16 oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) oacc[db] = zero16();

  for (int j = 0; j < KV::PD && j < ntiles; ++j) load(j);
  for (int it = 0; it < ntiles; ++it) {
    const int j0 = it * BN;
    kv.commit(it, min(KV::PD - 1, ntiles - 1 - it), vm_per_tile, tid);
    __syncthreads();
    if (it + KV::PD < ntiles) load(it + KV::PD);
    const TL tk = kv.ta(it), tv = kv.tb(it);

    f32x16 sacc[BN / 32];
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb) {
      sacc[kb] = zero16();
#pragma unroll
      for (int s = 0; s < D / KS; ++s) sacc[kb] = M::mma(tk.frag_rm(kb * 32 + col, s, hh), qf[s], sacc[kb]);
    }
    // keys beyond the causal diagonal of some row, or past the key list
    if (j0 + BN - 1 - pk > t_lo || j0 + BN > nkeys) {
#pragma unroll
      for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int j = j0 + kb * 32 + acc_row(e, hh);
          sacc[kb][e] = (j >= nkeys || (j >= pk && j - pk > my_t)) ? -INFINITY : sacc[kb][e];
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sacc[kb][e]);
    mx = wave_xor_max(mx, 32) * a.scale_log2;
    const bool upd = mx > m_ref + kRescaleSlack;
    if (__ballot(upd)) {
      const float m_new = upd ? mx : m_ref;
      const float alpha = __builtin_amdgcn_exp2f(m_ref - m_new);
      l *= alpha;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[db][e] *= alpha;
      m_ref = m_new;
    }
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float p = __builtin_amdgcn_exp2f(fmaf(sacc[kb][e], a.scale_log2, -m_ref));
        sacc[kb][e] = p;
        l += p;
      }
#pragma unroll
      for (int s = 0; s < 32 / KS; ++s) {
        const typename M::frag pf = M::pack(sacc[kb], s * KL);
#pragma unroll
        for (int db = 0; db < D / 32; ++db) oacc[db] = M::mma(tv.frag_tr(kb, db, s, lane), pf, oacc[db]);
      }
    }
  }

  l = wave_xor_sum(l, 32);
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
    if (hh == 0) a.lse[(int64_t)my_g * g.c + my_t] = (m_ref + log2f(l)) * kLn2;
  }
}

// bf16 forward with the key loop software-pipelined by one tile: while the
// softmax of tile j runs on the VALU, the MFMAs of S for tile j+1 are issued,
// and while O += V_j P_j runs on the matrix core, the VALU masks S_{j+1} and
// takes its row maxima; the two streams of one wave are independent, so the
// compiler and the hardware can overlap them.  K/V tiles stream through a 4-slot ring (three tiles in
// flight); at tile j the ring holds V_j, K_{j+1} and the loads of j+2, j+3.
constexpr int kPipeSlots = 4;

template <int D>
__global__ __launch_bounds__(kFwdWaves * 64) void fwd_pipe_kernel(FwdArgs a) {
  typedef __bf16 T;
  typedef Mma<T> M;
  constexpr int BN = 64, NT = kFwdWaves * 64;
  typedef Ring<T, D, BN, NT, kPipeSlots, false> KV;  // builtin loads (see Ring)
  typedef typename KV::TL TL;
  constexpr int KS = M::KS, KL = M::KL;
  constexpr int PD = kPipeSlots - 1;  // tiles issued ahead of the one whose V is read
  __shared__ __attribute__((aligned(16))) T lds_k[KV::NS * TL::ELEMS];
  __shared__ __attribute__((aligned(16))) T lds_v[KV::NS * TL::ELEMS];
  __shared__ int page_tab[kPageCache];

  const Geo& g = a.g;
  const int rows_total = g.c * g.G;
  const int nrb = (rows_total + kFwdBM - 1) / kFwdBM;
  const RowItem it = row_item(blockIdx.x, nrb, g.hkv);
  const int h = it.h;
  const int r0 = (nrb - 1 - it.rank) * kFwdBM;  // later (heavier) row blocks first

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, hh = lane >> 5;
  const int my_row = r0 + wave * 32 + col;
  const bool row_ok = my_row < rows_total;
  const int my_t = row_ok ? div_g(g, my_row) : g.c - 1;
  const int my_g = h * g.G + (row_ok ? my_row - div_g(g, my_row) * g.G : 0);

  typename M::frag qf[D / KS];
  const T* qrow = (const T*)a.q + ((int64_t)my_t * g.hq + my_g) * D;
#pragma unroll
  for (int s = 0; s < D / KS; ++s) qf[s] = row_ok ? M::load(qrow + s * KS + hh * KL) : M::zero();

  const int pk = g.keff << g.ps_log2;
  const int last_row = min(r0 + kFwdBM, rows_total) - 1;
  const int t_lo = div_g(g, r0);
  const int nkeys = pk + div_g(g, last_row) + 1;
  const int ntiles = (nkeys + BN - 1) / BN;
  PageSlots<kPageCache> pages{(lds_int*)page_tab};
  pages.fill(g, a.pt, a.sel, h, (nkeys + (1 << g.ps_log2) - 1) >> g.ps_log2, tid, NT);
  __syncthreads();

  const T* __restrict__ kp = (const T*)a.k;
  const T* __restrict__ vp = (const T*)a.v;
  KV kv{lds_k, lds_v};
  const bool tile_in_page = BN <= (1 << g.ps_log2);
  const typename KV::Lanes lanes = KV::lane_offsets(tid, D);
  const int vm_per_tile = KV::loads_per_tile(wave);

  // S^T of tile j (keys as rows, this lane's query row as the column)
  auto scores = [&](int j, f32x16* s) {
    const TL tk = kv.ta(j);
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb) {
      s[kb] = zero16();
#pragma unroll
      for (int k = 0; k < D / KS; ++k) s[kb] = M::mma(tk.frag_rm(kb * 32 + col, k, hh), qf[k], s[kb]);
    }
  };
  // keys beyond the causal diagonal of some row of the block, or past the list
  auto mask = [&](int j, f32x16* s) {
    const int j0 = j * BN;
    if (j0 + BN - 1 - pk > t_lo || j0 + BN > nkeys) {
#pragma unroll
      for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int jj = j0 + kb * 32 + acc_row(e, hh);
          s[kb][e] = (jj >= nkeys || (jj >= pk && jj - pk > my_t)) ? -INFINITY : s[kb][e];
        }
    }
  };
  auto row_max = [&](const f32x16* s) {
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[kb][e]);
    return mx;
  };

  float m_ref, l = 0.f;  // running max (log2 domain) and this lane's partial sum
  f32x16 oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) oacc[db] = zero16();

  f32x16 scur[BN / 32], snext[BN / 32];
  // The key loop, once per kind of page lookup (see Bool).
  auto run = [&](auto cached_tag) {
  constexpr bool kCached = decltype(cached_tag)::value;
  auto offset = [&](int jj) -> int64_t {
    if constexpr (kCached) return pages.key_offset_cached<D>(g, h, jj);
    else return key_offset<D>(g, a.pt, a.sel, h, jj);
  };
  auto load = [&](int j) {
    if (tile_in_page) {
      kv.load_rows(j, kp, vp, offset(j * BN), lanes, tid);
    } else {
      kv.load(j, kp, vp, tid, [&, j](int r) -> int64_t { return offset(min(j * BN + r, nkeys - 1)); });
    }
  };
  for (int j = 0; j < PD && j < ntiles; ++j) load(j);
  kv.commit(0, min(PD - 1, ntiles - 1), vm_per_tile, tid);
  __syncthreads();
  scores(0, scur);
  mask(0, scur);
  m_ref = wave_xor_max(row_max(scur), 32) * a.scale_log2;  // every row sees key 0: finite

  for (int it = 0; it < ntiles; ++it) {
    const bool has_next = it + 1 < ntiles;
    if (has_next) kv.commit(it + 1, min(1, ntiles - 2 - it), vm_per_tile, tid);
    __syncthreads();  // every wave is past tile it-1: its slot takes tile it+PD
    if (it + PD < ntiles) load(it + PD);
    const TL tv = kv.tb(it);
    typename M::frag pf[BN / 32][32 / KS];
    if (has_next) {
      // S_{it+1} on the matrix core, P_it on the VALU
      scores(it + 1, snext);
#pragma unroll
      for (int kb = 0; kb < BN / 32; ++kb) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float p = __builtin_amdgcn_exp2f(fmaf(scur[kb][e], a.scale_log2, -m_ref));
          scur[kb][e] = p;
          l += p;
        }
#pragma unroll
        for (int s = 0; s < 32 / KS; ++s) pf[kb][s] = M::pack(scur[kb], s * KL);
      }
      mask(it + 1, snext);
      // O += V_it P_it on the matrix core, row maxima of S_{it+1} on the VALU
#pragma unroll
      for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
        for (int s = 0; s < 32 / KS; ++s)
#pragma unroll
          for (int db = 0; db < D / 32; ++db) oacc[db] = M::mma(tv.frag_tr(kb, db, s, lane), pf[kb][s], oacc[db]);
      float mx = row_max(snext);
      mx = wave_xor_max(mx, 32) * a.scale_log2;
      const bool upd = mx > m_ref + kRescaleSlack;
      if (__ballot(upd)) {
        const float m_new = upd ? mx : m_ref;
        const float alpha = __builtin_amdgcn_exp2f(m_ref - m_new);
        l *= alpha;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int e = 0; e < 16; ++e) oacc[db][e] *= alpha;
        m_ref = m_new;
      }
#pragma unroll
      for (int kb = 0; kb < BN / 32; ++kb) scur[kb] = snext[kb];
    } else {
#pragma unroll
      for (int kb = 0; kb < BN / 32; ++kb) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float p = __builtin_amdgcn_exp2f(fmaf(scur[kb][e], a.scale_log2, -m_ref));
          scur[kb][e] = p;
          l += p;
        }
#pragma unroll
        for (int s = 0; s < 32 / KS; ++s) {
          pf[kb][s] = M::pack(scur[kb], s * KL);
#pragma unroll
          for (int db = 0; db < D / 32; ++db) oacc[db] = M::mma(tv.frag_tr(kb, db, s, lane), pf[kb][s], oacc[db]);
        }
      }
    }
  }
  };
  if (pages.cached) run(Bool<true>());
  else run(Bool<false>());

  l = wave_xor_sum(l, 32);
  if (row_ok) {
    const float inv = 1.f / l;
    T* orow = (T*)a.o + ((int64_t)my_t * g.hq + my_g) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        bf16x4 w;
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = (__bf16)(oacc[db][4 * e4 + i] * inv);
        *reinterpret_cast<bf16x4*>(orow + db * 32 + 8 * e4 + 4 * hh) = w;
      }
    if (hh == 0) a.lse[(int64_t)my_g * g.c + my_t] = (m_ref + log2f(l)) * kLn2;
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
  const dim3 grid(((rows + kFwdBM - 1) / kFwdBM) * s.hkv);
  const dim3 block(kFwdWaves * 64);
  Traced tr(st, "fwd_kernel");
  if (s.bf16) {
    if (s.d == 128) hipLaunchKernelGGL((fwd_pipe_kernel<128>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((fwd_pipe_kernel<64>), grid, block, 0, st, a);
  } else {
    if (s.d == 128) hipLaunchKernelGGL((fwd_kernel<float, 128>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((fwd_kernel<float, 64>), grid, block, 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace oomb
