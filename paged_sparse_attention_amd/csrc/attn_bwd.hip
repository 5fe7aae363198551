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
//   2. dkdv_kernel: key-major.  A workgroup owns 128 keys of one kv-head's key
//      list (4 waves x 32 keys; V in registers, K in LDS; two workgroups per
//      CU) and walks a share of the query rows that see them, head by head in
//      tiles of 32 rows, recomputing S = Q K^T and dP = dO V^T on MFMA, then
//      dV^T += dO^T P and dK^T += Q^T dS (dO^T and Q^T read transposed from the
//      row-major LDS tiles).  When the rows are split over several workgroups
//      for load balance (and split again in two for the chunk's key blocks,
//      when an XCD would otherwise get too few of them to even out its last
//      round), the first piece adds into the pools in place and the others
//      write partial sums to the workspace.
//   3. dq_kernel:   query-major, like the forward: S^T and dP^T per 32-key
//      block of a K/V tile, dQ^T += K^T dS^T, written once per row.  With a
//      row split, trailing workgroups of the same launch then add the other
//      splits' partials into dk_pool/dv_pool, in split order: they are
//      dispatched after every row block and fill the CUs that the last round
//      of row blocks leaves idle.
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
  float* dt;       // workspace [Hq][C]: rowsum(dO * O)
  float* lse2;     // workspace [Hq][C]: lse * log2(e)
  __bf16* bias;    // workspace [Hq][C][16]: -lse2/scale_log2, then -Dt, each as three bf16 parts that sum
                   // to it exactly and five zeros (the dK/dV kernel's bias operands, bf16 inputs)
  float* part_k;   // workspace [splits-1][Hkv][nkeys][D], scaled dK partials of splits 1..
  float* part_v;   // workspace [splits-1][Hkv][nkeys][D]
  float* part2_k;  // workspace [splits][Hkv][nkeys - key0_sub][D], second halves of the chunk blocks' shares
  float* part2_v;  //   (only when sub = 2)
  int splits;
  int sub;         // 2: each share of a chunk key block is split again in two (KvPlan)
  int key0_sub;    // first key of the chunk key blocks (a multiple of the workgroup's keys)
  Geo g;
  float scale_log2;
};

// ---------------------------------------------------------------------------
// Dt = rowsum(dO * O) and lse in log2 units, one row per group of D/VEC lanes;
// a thread takes kDtRows rows, their loads issued together.
// ---------------------------------------------------------------------------
constexpr int kDtRows = 4;

// x as three bf16 values whose sum is x exactly (8 significant bits each; x
// normal and far from the fp32 range limits): hi = x rounded, then the
// remainders, each exact in fp32.
__device__ __forceinline__ void split_bf16x3(float x, __bf16* out) {
  const __bf16 hi = (__bf16)x;
  const float r1 = x - (float)hi;
  const __bf16 mid = (__bf16)r1;
  out[0] = hi;
  out[1] = mid;
  out[2] = (__bf16)(r1 - (float)mid);
}

template <typename T, int D>
__global__ __launch_bounds__(256) void dt_kernel(BwdArgs a) {
  constexpr int VEC = 16 / (int)sizeof(T);
  constexpr int LPR = D / VEC;  // lanes per row (power of two, <= 32)
  constexpr int RPB = 256 / LPR;  // rows per block and pass
  const int rows = a.g.c * a.g.hq;
  const int lane_in_row = threadIdx.x % LPR;
  const int row0 = blockIdx.x * (RPB * kDtRows) + threadIdx.x / LPR;
  f32x4 ro[kDtRows], rd[kDtRows];
#pragma unroll
  for (int k = 0; k < kDtRows; ++k) {
    const int row = row0 + k * RPB;
    if (row < rows) {
      const int64_t off = (int64_t)row * D + lane_in_row * VEC;
      ro[k] = *reinterpret_cast<const f32x4*>((const T*)a.o + off);
      rd[k] = *reinterpret_cast<const f32x4*>((const T*)a.dout + off);
    }
  }
#pragma unroll
  for (int k = 0; k < kDtRows; ++k) {
    const int row = row0 + k * RPB;
    float s = 0.f;
    if (row < rows) {
      const T* po = reinterpret_cast<const T*>(&ro[k]);
      const T* pd = reinterpret_cast<const T*>(&rd[k]);
#pragma unroll
      for (int i = 0; i < VEC; ++i) s += (float)po[i] * (float)pd[i];
    }
#pragma unroll
    for (int m = LPR / 2; m >= 1; m >>= 1) s = wave_xor_sum(s, m);
    if (row < rows && lane_in_row == 0) {
      const int t = row / a.g.hq, g = row % a.g.hq;  // row = t * Hq + g
      const int64_t i = (int64_t)g * a.g.c + t;
      a.dt[i] = s;
      const float l2 = a.lse[i] * kLog2e;
      a.lse2[i] = l2;
      if constexpr (sizeof(T) == 2) {
        bf16x8 rs, rp;
#pragma unroll
        for (int k = 0; k < 8; ++k) rs[k] = rp[k] = (__bf16)0.f;
        __bf16 part[3];
        split_bf16x3(-l2 / a.scale_log2, part);
        rs[0] = part[0], rs[1] = part[1], rs[2] = part[2];
        split_bf16x3(-s, part);
        rp[0] = part[0], rp[1] = part[1], rp[2] = part[2];
        *reinterpret_cast<bf16x8*>(a.bias + i * 16) = rs;
        *reinterpret_cast<bf16x8*>(a.bias + i * 16 + 8) = rp;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// dK / dV, key-major.  Four waves own 32 keys each: V^T fragments stay in
// registers and the dK^T / dV^T accumulators too.  bf16: the workgroup's K rows
// are staged once in LDS as the B operand of S = Q K^T, which keeps a wave
// within 256 registers, so two workgroups share a CU and one wave's softmax
// overlaps the other's MFMAs.  fp32: K fragments in registers.
// ---------------------------------------------------------------------------
template <typename T> constexpr int kv_waves() { return 4; }
template <typename T> constexpr int kv_keys() { return kv_waves<T>() * 32; }  // keys per workgroup
template <typename T, int D> constexpr int kv_bm() { return sizeof(T) == 2 && D == 64 ? 64 : 32; }  // rows per tile

// Work of the dK/dV kernel: nkb key blocks per kv-head, the first nprior of
// which hold prior keys (every query row sees them), the rest chunk keys (only
// the rows at or after them).  Each key block's rows are split into `splits`
// shares.  When the groups (kv-head, share) divide evenly over the 8 XCDs
// (`ordered`, gpx groups per XCD), and an XCD would get at most two chunk key
// blocks per workgroup slot (32 CUs x 2), each share of a chunk key block is
// split again in two (sub = 2): the chunk blocks, which end the kernel, then
// come in pieces of at most half a prior block's work, and the last round
// evens out.
struct KvPlan {
  int nkb, splits, nprior, sub, gpx, items;
  bool ordered;
};

__host__ __device__ inline KvPlan kv_plan(const Geo& g, int keys_per_wg) {
  KvPlan p;
  const int pk = g.keff << g.ps_log2;
  const int nkeys = pk + g.c;
  p.nkb = (nkeys + keys_per_wg - 1) / keys_per_wg;
  const int items = p.nkb * g.hkv;
  // at least three rounds of two workgroups per CU, and never fewer than four
  // row shares: measured on the long-context steps (256K to 4M tokens of
  // context, and 32K dense), four shares beat two, three and five to eight,
  // the extra partial sums costing less than the balance they buy
  int s = (1536 + items - 1) / items;
  p.splits = s < 4 ? 4 : (s > 8 ? 8 : s);
  p.nprior = min(p.nkb, (pk + keys_per_wg - 1) / keys_per_wg);
  const int total = p.nkb * p.splits * g.hkv, per = total / 8;
  p.ordered = total % 8 == 0 && per % p.nkb == 0 && p.nprior > 0 && p.nprior < p.nkb;
  p.gpx = p.ordered ? per / p.nkb : 0;
  p.sub = p.ordered && p.gpx * (p.nkb - p.nprior) <= 128 ? 2 : 1;
  p.items = g.hkv * p.splits * (p.nprior + (p.nkb - p.nprior) * p.sub);
  return p;
}

template <typename T, int D> struct KeyStore;  // where a wave's K^T B operands live

template <int D> struct KeyStore<__bf16, D> {  // LDS, one tile for the workgroup
  typedef Tile<__bf16, D, kv_keys<__bf16>()> TK;
  TK t;
  int row0;  // this wave's first key row in the tile
  template <typename OffFn>
  __device__ __forceinline__ void load(const __bf16* src, int wave, int lane, int tid, OffFn off) {
    row0 = wave * 32;
    t.fill(src, wave, kv_waves<__bf16>(), lane, off);
  }
  __device__ __forceinline__ bf16x8 frag(int s, int col, int hh) const { return t.frag_rm(row0 + col, s, hh); }
};

template <int D> struct KeyStore<float, D> {  // registers
  float f[D / 2];
  template <typename OffFn>
  __device__ __forceinline__ void load(const float* src, int wave, int lane, int tid, OffFn off) {
    const int64_t o = off(wave * 32 + (lane & 31));
#pragma unroll
    for (int s = 0; s < D / 2; ++s) f[s] = src[o + 2 * s + (lane >> 5)];
  }
  __device__ __forceinline__ float frag(int s, int col, int hh) const { return f[s]; }
};

template <typename T, int D>
__global__ __launch_bounds__(kv_waves<T>() * 64, 2) void dkdv_kernel(BwdArgs a) {
  typedef Mma<T> M;
  constexpr int BM = kv_bm<T, D>(), KEYS = kv_keys<T>(), NW = kv_waves<T>(), NT = NW * 64;
  typedef Tile<T, D, BM> TL;
  constexpr int KS = M::KS, KL = M::KL;
  constexpr bool kKeysInLds = sizeof(T) == 2;
  typedef Ring<T, D, BM, NT, 2> QD;  // two slots: two workgroups fit a CU
  __shared__ __attribute__((aligned(16))) T lds_q[QD::NS * TL::ELEMS];
  __shared__ __attribute__((aligned(16))) T lds_d[QD::NS * TL::ELEMS];
  __shared__ __attribute__((aligned(16))) T lds_keys[kKeysInLds ? KeyStore<__bf16, D>::TK::ELEMS : 1];
  // bf16: each tile row's -lse2/scale_log2 and -Dt enter S and dP as the first
  // MFMA of each chain (A = the row's three bf16 parts in k = 0..2 and zeros,
  // B = ones), so the softmax needs no per-row operands.  Two 16-byte A
  // fragments per row; row BM is zeros (the A operand's k = 8..15 half).
  constexpr bool kBias = sizeof(T) == 2;
  __shared__ __attribute__((aligned(16))) float rlse[kBias ? 1 : QD::NS][BM];  // per tile row: lse * log2(e)
  __shared__ __attribute__((aligned(16))) float rdt[kBias ? 1 : QD::NS][BM];   // per tile row: Dt
  __shared__ __attribute__((aligned(16))) __bf16 rbias[kBias ? QD::NS : 1][BM + 1][16];

  const Geo& g = a.g;
  const KvPlan plan = kv_plan(g, KEYS);
  // Work items are (row-share group = kv-head and split, key block), and for
  // chunk key blocks with sub = 2 also the half of the share.  Each XCD takes
  // whole groups, so the workgroups that run together on it stream the same
  // shares of query rows through its L2.  Within an XCD the key blocks that
  // hold prior keys (every row sees them: the heaviest, all alike) go first,
  // group by group, then the chunk's key blocks, which fewer rows see,
  // heaviest first with the groups (and halves) alternating: the light ones
  // end the kernel.  Shapes whose items do not split evenly into whole groups
  // per XCD take contiguous ranges of items per XCD instead.
  int h, sp, kblk, half = 0;
  if (plan.ordered) {
    const int x = blockIdx.x % 8, j = blockIdx.x / 8, gpx = plan.gpx, nprior = plan.nprior;
    int grp;
    if (j < gpx * nprior) {
      grp = j / nprior;
      kblk = j % nprior;
    } else {
      const int jl = j - gpx * nprior, w = gpx * plan.sub;
      grp = jl % gpx;
      half = (jl % w) / gpx;
      kblk = nprior + jl / w;
    }
    const int gi = x * gpx + grp;
    h = gi / plan.splits;
    sp = gi % plan.splits;
  } else {
    const int item = xcd_remap(blockIdx.x, plan.items);
    h = item / (plan.nkb * plan.splits);
    kblk = item % plan.nkb;
    sp = (item / plan.nkb) % plan.splits;
  }
  const int nhalf = kblk >= plan.nprior ? plan.sub : 1;  // pieces of this block's share

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, hh = lane >> 5;
  const int pk = g.keff << g.ps_log2;
  const int nkeys = pk + g.c;
  const int jb = kblk * KEYS;

  // this lane's key and its V^T B operands: lane (key col, half hh) holds
  // V[key][s*KS + hh*KL + i]
  const int my_key = jb + wave * 32 + col;
  const bool key_ok = my_key < nkeys;
  const int64_t koff = key_ok ? key_offset<D>(g, a.pt, a.sel, h, my_key) : 0;
  const int my_u = my_key - pk;  // chunk token index when >= 0
  typename M::frag vf[D / KS];
#pragma unroll
  for (int s = 0; s < D / KS; ++s) vf[s] = key_ok ? M::load((const T*)a.v + koff + s * KS + hh * KL) : M::zero();
  KeyStore<T, D> ks;
  if constexpr (kKeysInLds) ks.t.rm = lds_keys;
  // keys past the list are clamped to its last key (finite data, zero weight below)
  ks.load((const T*)a.k, wave, lane, tid,
          [&](int r) -> int64_t { return key_offset<D>(g, a.pt, a.sel, h, min(jb + r, nkeys - 1)); });
  vmem_drain();  // the K tile (LDS) and the V^T fragments (registers) have landed

  f32x16 dkacc[D / 32], dvacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    dkacc[db] = zero16();
    dvacc[db] = zero16();
  }

  // Query rows are visited head by head: tile (gi, t0) holds tokens t0 .. t0+BM-1
  // of query head h*G + gi, which sit hq*D elements apart in Q and dO.  Rows
  // that can see a key of this block: every token for prior keys, else tokens
  // t >= the block's first chunk token (t0 starts at that token rounded down
  // to a tile).  Tokens past the chunk read the last token (finite data, zero
  // weight below).  This split takes a contiguous share of the tiles.
  const int t_first = jb < pk ? 0 : ((jb - pk) / BM) * BM;
  const int tiles_per_head = (g.c - t_first + BM - 1) / BM;
  const int ntile_all = tiles_per_head * g.G;
  const int nsh = plan.splits * nhalf, ish = sp * nhalf + half;  // this piece among the block's pieces
  const int tile_lo = (int)((int64_t)ntile_all * ish / nsh);
  const int tile_hi = (int)((int64_t)ntile_all * (ish + 1) / nsh);
  const int ntiles = tile_hi - tile_lo;
  auto tile_head = [&](int j) { return (tile_lo + j) / tiles_per_head; };
  auto tile_t0 = [&](int j) { return t_first + ((tile_lo + j) % tiles_per_head) * BM; };

  const T* __restrict__ qp = (const T*)a.q;
  const T* __restrict__ dp = (const T*)a.dout;
  QD qd{lds_q, lds_d};
  const int64_t tok_stride = (int64_t)g.hq * D;
  const typename QD::Lanes qlanes = QD::lane_offsets(tid, (int)tok_stride);
  auto load = [&](int j) {
    const int gi = tile_head(j), t0 = tile_t0(j);
    const int tmax = g.c - 1 - t0;  // last valid row of the tile
    const int64_t base = ((int64_t)t0 * g.hq + h * g.G + gi) * D;
    bool done = false;
    if constexpr (QD::kDirect) {
      if (tmax >= BM - 1) {  // every row of the tile is a real token
        qd.load_rows(j, qp, dp, base, qlanes, tid);
        done = true;
      }
    }
    if (!done) qd.load(j, qp, dp, tid, [=](int r) -> int64_t { return base + (int64_t)min(r, tmax) * tok_stride; });
    if (wave == 0 && lane < BM) {
      const int64_t i = (int64_t)(h * g.G + gi) * g.c + t0 + min(lane, tmax);
      if constexpr (!kBias) {
        load_lds_dword(a.lse2 + i, rlse[j % QD::NS]);
        load_lds_dword(a.dt + i, rdt[j % QD::NS]);
      }
    }
    if constexpr (kBias) {
      // 32 bytes a row: lane l of a load carries half l % 2 of row l / 2 (a
      // wave-uniform base and a lane offset, which need no 64-bit lane address)
      if (wave == 0) {
        const __bf16* brow = a.bias + ((int64_t)(h * g.G + gi) * g.c + t0) * 16;
#pragma unroll
        for (int r0 = 0; r0 < 2 * BM; r0 += 64) {
          const unsigned boff = (unsigned)(min((r0 + lane) / 2, tmax) * 32 + ((r0 + lane) & 1) * 16);
          lds_load16(brow, boff, &rbias[j % QD::NS][r0 / 2][0]);
        }
      }
    }
  };
  const int vm_per_tile = QD::loads_per_tile(wave) + (wave == 0 ? (kBias ? 2 * BM / 64 : 2) : 0);
  if constexpr (kBias) {
    if (tid < QD::NS * 16) rbias[kBias ? tid / 16 : 0][BM][tid % 16] = (__bf16)0.f;  // visible after the first barrier
  }

  // a 32-row block needs no per-element visibility test when every row is a
  // real token and every key of this wave is a valid prior key or a chunk
  // token no later than the block's first token
  const int wave_last = jb + wave * 32 + 31;  // last key of this wave
  const bool wave_keys_ok = wave_last < nkeys;
  const bool wave_prior = wave_last < pk;

  for (int j = 0; j < QD::PD && j < ntiles; ++j) load(j);
  for (int it = 0; it < ntiles; ++it) {
    qd.commit(it, min(QD::PD - 1, ntiles - 1 - it), vm_per_tile, tid);
    if constexpr (!QD::kDirect) {
      if (wave == 0) wait_vmem_le(0);  // the row metadata loads
    }
    __syncthreads();
    if (it + QD::PD < ntiles) load(it + QD::PD);
    const TL tq = qd.ta(it), td = qd.tb(it);
    const float* ml = rlse[kBias ? 0 : it % QD::NS];
    const float* md = rdt[kBias ? 0 : it % QD::NS];
    const int t0 = tile_t0(it);
#pragma unroll 1
    for (int rb = 0; rb < BM / 32; ++rb) {
      f32x16 sacc = zero16(), pacc = zero16();
      if constexpr (kBias) {
        // lane (row col, half hh): its row's parts in k = 0..7 (hh = 0), the zero row (hh = 1);
        // B is ones everywhere, which the zero half makes harmless
        const __bf16* rec = &rbias[it % QD::NS][hh == 0 ? rb * 32 + col : BM][0];
        typename M::frag ones;
#pragma unroll
        for (int k = 0; k < 8; ++k) ones[k] = (__bf16)1.f;
        sacc = M::mma(*reinterpret_cast<const bf16x8*>(rec), ones, sacc);      // S = -lse2/scale_log2 + Q K^T
        pacc = M::mma(*reinterpret_cast<const bf16x8*>(rec + 8), ones, pacc);  // dP = -Dt + dO V^T
      }
#pragma unroll
      for (int s = 0; s < D / KS; ++s) sacc = M::mma(tq.frag_rm(rb * 32 + col, s, hh), ks.frag(s, col, hh), sacc);
#pragma unroll
      for (int s = 0; s < D / KS; ++s) pacc = M::mma(td.frag_rm(rb * 32 + col, s, hh), vf[s], pacc);
      // The softmax below gates this wave's dV/dK MFMAs, while the other wave
      // on the SIMD usually has MFMAs ready: raising this wave's issue priority
      // for the softmax keeps both pipes fed (about 3% on this kernel).
      __builtin_amdgcn_s_setprio(3);
      // element e of a lane: query token tb + acc_row(e, hh) of head gi, key my_key
      const int tb = t0 + rb * 32;
      const bool full = tb + 32 <= g.c && wave_keys_ok && (wave_prior || tb >= wave_last - pk);
      // rows acc_row(4i + j, hh) = 8i + 4hh + j: four consecutive rows per i
      if constexpr (kBias) {
        if (full) {
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const float p = __builtin_amdgcn_exp2f(sacc[e] * a.scale_log2);
            sacc[e] = p;
            pacc[e] = p * pacc[e];
          }
        } else {
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int t = tb + acc_row(e, hh);
            const bool vis = key_ok && t < g.c && my_u <= t;  // my_u < 0 for prior keys
            const float p = __builtin_amdgcn_exp2f(vis ? sacc[e] * a.scale_log2 : -INFINITY);
            sacc[e] = p;
            pacc[e] = p * pacc[e];
          }
        }
      } else if (full) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const f32x4 l4 = *reinterpret_cast<const f32x4*>(ml + rb * 32 + 8 * i + 4 * hh);
          const f32x4 d4 = *reinterpret_cast<const f32x4*>(md + rb * 32 + 8 * i + 4 * hh);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float p = __builtin_amdgcn_exp2f(fmaf(sacc[4 * i + j], a.scale_log2, -l4[j]));
            sacc[4 * i + j] = p;
            pacc[4 * i + j] = p * (pacc[4 * i + j] - d4[j]);
          }
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const f32x4 l4 = *reinterpret_cast<const f32x4*>(ml + rb * 32 + 8 * i + 4 * hh);
          const f32x4 d4 = *reinterpret_cast<const f32x4*>(md + rb * 32 + 8 * i + 4 * hh);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int t = tb + 8 * i + 4 * hh + j;
            const bool vis = key_ok && t < g.c && my_u <= t;  // my_u < 0 for prior keys
            const float p = __builtin_amdgcn_exp2f(vis ? fmaf(sacc[4 * i + j], a.scale_log2, -l4[j]) : -INFINITY);
            sacc[4 * i + j] = p;
            pacc[4 * i + j] = p * (pacc[4 * i + j] - d4[j]);
          }
        }
      }
      __builtin_amdgcn_s_setprio(0);
#pragma unroll
      for (int s = 0; s < 32 / KS; ++s) {
        const typename M::frag pf = M::pack(sacc, s * KL);
        const typename M::frag sf = M::pack(pacc, s * KL);
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          dvacc[db] = M::mma(td.frag_tr(rb, db, s, lane), pf, dvacc[db]);
          dkacc[db] = M::mma(tq.frag_tr(rb, db, s, lane), sf, dkacc[db]);
        }
      }
    }
  }

  if (!key_ok) return;
  const float sc = g.scale;
  if (sp == 0 && half == 0) {  // the first split adds straight into the pools; the split reduction adds the rest after it
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
          ok[i] += sc * dkacc[db][4 * e4 + i];
          ov[i] += dvacc[db][4 * e4 + i];
        }
        *reinterpret_cast<f32x4*>(dkp + d) = ok;
        *reinterpret_cast<f32x4*>(dvp + d) = ov;
      }
  } else {
    // first halves (and whole shares) of splits 1..: part_k/v [splits-1][Hkv][nkeys][D];
    // second halves: part2_k/v [splits][Hkv][nkeys - key0_sub][D]
    const int slot = half == 0 ? sp - 1 : sp;
    const int key0 = half == 0 ? 0 : a.key0_sub;
    const int nk = nkeys - key0;
    const int64_t base = (((int64_t)slot * g.hkv + h) * nk + (my_key - key0)) * D;
    float* pk_out = half == 0 ? a.part_k : a.part2_k;
    float* pv_out = half == 0 ? a.part_v : a.part2_v;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const int d = db * 32 + 8 * e4 + 4 * hh;
        f32x4 wk, wv;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          wk[i] = sc * dkacc[db][4 * e4 + i];
          wv[i] = dvacc[db][4 * e4 + i];
        }
        *reinterpret_cast<f32x4*>(pk_out + base + d) = wk;
        *reinterpret_cast<f32x4*>(pv_out + base + d) = wv;
      }
  }
}

// dk_pool / dv_pool += sum of the partials of splits 1 .. splits-1, in split
// order, then for the chunk key blocks split in halves those of the second
// halves of shares 0 .. splits-1 (the first half of share 0 has already added
// in place); float4 group i of the [Hkv][keys][D] key list.  Runs after dkdv_kernel has finished (a later
// launch on the same stream).
template <int D>
__device__ __forceinline__ void kv_reduce_group(const BwdArgs& a, int64_t i) {
  const Geo& g = a.g;
  const int nkeys = (g.keff << g.ps_log2) + g.c;
  const int d = (int)(i % (D / 4)) * 4;
  const int64_t hk = i / (D / 4);
  const int h = (int)(hk / nkeys), jj = (int)(hk % nkeys);
  const int64_t stride = (int64_t)g.hkv * nkeys * D;
  const int64_t src = hk * D + d;
  f32x4 sk = *reinterpret_cast<const f32x4*>(a.part_k + src);
  f32x4 sv = *reinterpret_cast<const f32x4*>(a.part_v + src);
  for (int s = 1; s < a.splits - 1; ++s) {
    sk += *reinterpret_cast<const f32x4*>(a.part_k + s * stride + src);
    sv += *reinterpret_cast<const f32x4*>(a.part_v + s * stride + src);
  }
  if (a.sub == 2 && jj >= a.key0_sub) {
    const int nk2 = nkeys - a.key0_sub;
    const int64_t stride2 = (int64_t)g.hkv * nk2 * D;
    const int64_t src2 = ((int64_t)h * nk2 + (jj - a.key0_sub)) * D + d;
    for (int s = 0; s < a.splits; ++s) {
      sk += *reinterpret_cast<const f32x4*>(a.part2_k + s * stride2 + src2);
      sv += *reinterpret_cast<const f32x4*>(a.part2_v + s * stride2 + src2);
    }
  }
  const int64_t dst = key_offset<D>(g, a.pt, a.sel, h, jj) + d;
  f32x4 ok = *reinterpret_cast<f32x4*>(a.dk + dst);
  f32x4 ov = *reinterpret_cast<f32x4*>(a.dv + dst);
  *reinterpret_cast<f32x4*>(a.dk + dst) = ok + sk;
  *reinterpret_cast<f32x4*>(a.dv + dst) = ov + sv;
}

__host__ __device__ inline int64_t kv_reduce_groups(const Geo& g, int d) {
  return (int64_t)g.hkv * ((g.keff << g.ps_log2) + g.c) * (d / 4);
}

// ---------------------------------------------------------------------------
// dQ, query-major.
// ---------------------------------------------------------------------------
template <typename T> constexpr int dq_waves() { return sizeof(T) == 2 ? 8 : 4; }
template <typename T> constexpr int dq_bm() { return 32 * dq_waves<T>(); }  // query rows per workgroup
template <typename T> constexpr int dq_bn() { return sizeof(T) == 2 ? 128 : 32; }  // keys per tile

template <typename T, int D>
__global__ __launch_bounds__(dq_waves<T>() * 64) void dq_kernel(BwdArgs a) {
  typedef Mma<T> M;
  constexpr int BN = dq_bn<T>();
  constexpr int NT = dq_waves<T>() * 64, BM = dq_bm<T>();
  typedef Ring<T, D, BN, NT, 2> KV;  // two slots of 128 keys fill most of the LDS
  typedef typename KV::TL TL;
  constexpr int KS = M::KS, KL = M::KL;
  __shared__ __attribute__((aligned(16))) T lds_k[KV::NS * TL::ELEMS];
  __shared__ __attribute__((aligned(16))) T lds_v[KV::NS * TL::ELEMS];
  __shared__ int page_tab[kPageCache];

  const Geo& g = a.g;
  const int rows_total = g.c * g.G;
  const int nrb = (rows_total + BM - 1) / BM;
  if ((int)blockIdx.x >= nrb * g.hkv) {  // a trailing workgroup: NT float4 groups of the split reduction
    const int64_t i = (int64_t)(blockIdx.x - nrb * g.hkv) * NT + threadIdx.x;
    if (i < kv_reduce_groups(g, D)) kv_reduce_group<D>(a, i);
    return;
  }
  const RowItem it = row_item(blockIdx.x, nrb, g.hkv);
  const int h = it.h;
  const int r0 = (nrb - 1 - it.rank) * BM;  // later (heavier) row blocks first

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, hh = lane >> 5;
  const int my_row = r0 + wave * 32 + col;
  const bool row_ok = my_row < rows_total;
  const int my_t = row_ok ? div_g(g, my_row) : g.c - 1;
  const int my_g = h * g.G + (row_ok ? my_row - div_g(g, my_row) * g.G : 0);
  const int64_t qoff = ((int64_t)my_t * g.hq + my_g) * D;

  typename M::frag qf[D / KS], df[D / KS];
#pragma unroll
  for (int s = 0; s < D / KS; ++s) {
    qf[s] = row_ok ? M::load((const T*)a.q + qoff + s * KS + hh * KL) : M::zero();
    df[s] = row_ok ? M::load((const T*)a.dout + qoff + s * KS + hh * KL) : M::zero();
  }
  const float my_lse = row_ok ? a.lse2[(int64_t)my_g * g.c + my_t] : 0.f;
  const float my_dt = row_ok ? a.dt[(int64_t)my_g * g.c + my_t] : 0.f;

  const int pk = g.keff << g.ps_log2;
  const int last_row = min(r0 + BM, rows_total) - 1;
  const int t_lo = div_g(g, r0);
  const int nkeys = pk + div_g(g, last_row) + 1;
  const int ntiles = (nkeys + BN - 1) / BN;
  PageSlots<kPageCache> pages{(lds_int*)page_tab};
  pages.fill(g, a.pt, a.sel, h, (nkeys + (1 << g.ps_log2) - 1) >> g.ps_log2, tid, NT);
  __syncthreads();

  const T* __restrict__ kp = (const T*)a.k;
  const T* __restrict__ vp = (const T*)a.v;
  KV kv{lds_k, lds_v};
  // one page lookup per tile when the tile lies inside a page (see the forward)
  const bool tile_in_page = BN <= (1 << g.ps_log2);
  const int vm_per_tile = KV::loads_per_tile(wave);

  f32x16 qacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) qacc[db] = zero16();
  vmem_drain();  // the Q and dO fragments and the row statistics are in registers before the key loop

  // The key loop, once per kind of page lookup (see Bool).
  auto run = [&](auto cached_tag) {
  constexpr bool kCached = decltype(cached_tag)::value;
  auto offset = [&](int jj) -> int64_t {
    if constexpr (kCached) return pages.key_offset_cached<D>(g, h, jj);
    else return key_offset<D>(g, a.pt, a.sel, h, jj);
  };
  auto load = [&](int j) {
    if (tile_in_page) {
      const int64_t base = offset(j * BN);
      kv.load(j, kp, vp, tid, [base](int r) -> int64_t { return base + (int64_t)r * D; });
    } else {
      kv.load(j, kp, vp, tid, [&, j](int r) -> int64_t { return offset(min(j * BN + r, nkeys - 1)); });
    }
  };
  for (int j = 0; j < KV::PD && j < ntiles; ++j) load(j);
  for (int it = 0; it < ntiles; ++it) {
    const int j0 = it * BN;
    kv.commit(it, min(KV::PD - 1, ntiles - 1 - it), vm_per_tile, tid);
    __syncthreads();
    if (it + KV::PD < ntiles) load(it + KV::PD);
    const TL tk = kv.ta(it), tv = kv.tb(it);
    const bool masked = j0 + BN - 1 - pk > t_lo || j0 + BN > nkeys;
    // S^T and dP^T of one 32-key block
    auto sdp = [&](int kb, f32x16& sacc, f32x16& pacc) {
      sacc = zero16();
      pacc = zero16();
#pragma unroll
      for (int s = 0; s < D / KS; ++s) {
        sacc = M::mma(tk.frag_rm(kb * 32 + col, s, hh), qf[s], sacc);
        pacc = M::mma(tv.frag_rm(kb * 32 + col, s, hh), df[s], pacc);
      }
    };
    // dS^T in place of dP^T; invisible pairs take exponent -inf (weight 0),
    // so exp2 runs unconditionally
    auto softmax = [&](int kb, const f32x16& sacc, f32x16& pacc) {
      if (masked) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int j = j0 + kb * 32 + acc_row(e, hh);
          const bool vis = j < nkeys && (j < pk || j - pk <= my_t);
          const float p = __builtin_amdgcn_exp2f(vis ? fmaf(sacc[e], a.scale_log2, -my_lse) : -INFINITY);
          pacc[e] = p * (pacc[e] - my_dt);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float p = __builtin_amdgcn_exp2f(fmaf(sacc[e], a.scale_log2, -my_lse));
          pacc[e] = p * (pacc[e] - my_dt);
        }
      }
    };
    auto dq_mma = [&](int kb, const f32x16& pacc) {
#pragma unroll
      for (int s = 0; s < 32 / KS; ++s) {
        const typename M::frag sf = M::pack(pacc, s * KL);
#pragma unroll
        for (int db = 0; db < D / 32; ++db) qacc[db] = M::mma(tk.frag_tr(kb, db, s, lane), sf, qacc[db]);
      }
    };
    // Software-pipelined by one block: the S^T/dP^T MFMAs of block kb+1 are
    // issued before the softmax of block kb, so the matrix core works while
    // the VALU takes the exponentials.
    f32x16 sacc[2], pacc[2];
    sdp(0, sacc[0], pacc[0]);
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb) {
      if (kb + 1 < BN / 32) sdp(kb + 1, sacc[(kb + 1) & 1], pacc[(kb + 1) & 1]);
      softmax(kb, sacc[kb & 1], pacc[kb & 1]);
      dq_mma(kb, pacc[kb & 1]);
    }
  }
  };
  if (pages.cached) run(Bool<true>());
  else run(Bool<false>());

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
  const size_t rowvec = (((size_t)s.hq * s.c * 4) + 255) & ~(size_t)255;
  p.off_dt = 0;
  p.off_lse2 = rowvec;
  p.off_bias = 2 * rowvec;
  size_t off = 2 * rowvec + ((((size_t)s.hq * s.c * 32) + 255) & ~(size_t)255);
  p.splits = kp.splits;
  p.sub = kp.sub;
  p.key0_sub = kp.nprior * (s.bf16 ? kv_keys<__bf16>() : kv_keys<float>());
  p.off_part_k = off;
  const size_t part = kp.splits > 1 ? (size_t)(kp.splits - 1) * s.hkv * nkeys * s.d * 4 : 0;
  off += (part + 255) & ~(size_t)255;
  p.off_part_v = off;
  off += (part + 255) & ~(size_t)255;
  const size_t part2 = kp.sub == 2 ? (size_t)kp.splits * s.hkv * (nkeys - (size_t)p.key0_sub) * s.d * 4 : 0;
  p.off_part2_k = off;
  off += (part2 + 255) & ~(size_t)255;
  p.off_part2_v = off;
  off += (part2 + 255) & ~(size_t)255;
  p.bytes = off;
  return p;
}

template <typename T, int D>
static hipError_t bwd_t(const BwdArgs& a, hipStream_t st) {
  constexpr int LPR = D / (16 / (int)sizeof(T));
  const int rows = a.g.c * a.g.hq;
  {
    Traced tr(st, "dt_kernel");
    const int per_block = (256 / LPR) * kDtRows;
    hipLaunchKernelGGL((dt_kernel<T, D>), dim3((rows + per_block - 1) / per_block), dim3(256), 0, st, a);
  }
  const KvPlan kp = kv_plan(a.g, kv_keys<T>());
  {
    Traced tr(st, "dkdv_kernel");
    hipLaunchKernelGGL((dkdv_kernel<T, D>), dim3(kp.items), dim3(kv_waves<T>() * 64), 0, st, a);
  }
  const int qrows = a.g.c * a.g.G;
  {
    constexpr int NT = dq_waves<T>() * 64;
    const int64_t n_red = kp.splits > 1 ? (kv_reduce_groups(a.g, D) + NT - 1) / NT : 0;
    Traced tr(st, "dq_kernel");
    hipLaunchKernelGGL((dq_kernel<T, D>), dim3((unsigned)(((qrows + dq_bm<T>() - 1) / dq_bm<T>()) * a.g.hkv + n_red)),
                       dim3(NT), 0, st, a);
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
  a.lse2 = (float*)((char*)ws + p.off_lse2);
  a.bias = (__bf16*)((char*)ws + p.off_bias);
  a.part_k = (float*)((char*)ws + p.off_part_k);
  a.part_v = (float*)((char*)ws + p.off_part_v);
  a.part2_k = (float*)((char*)ws + p.off_part2_k);
  a.part2_v = (float*)((char*)ws + p.off_part2_v);
  a.splits = p.splits;
  a.sub = p.sub;
  a.key0_sub = p.key0_sub;
  a.g = make_geo(s);
  a.scale_log2 = s.scale * kLog2e;
  if (s.bf16) return s.d == 128 ? bwd_t<__bf16, 128>(a, st) : bwd_t<__bf16, 64>(a, st);
  return s.d == 128 ? bwd_t<float, 128>(a, st) : bwd_t<float, 64>(a, st);
}

}  // namespace oomb
