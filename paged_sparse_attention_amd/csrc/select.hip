// select.hip -- representative vectors and top-K page selection on gfx950.
//
// Page "Out of the Memory Barrier" (OOMB), technical summary, section 2,
// "Page-level Sparse Attention": a top-K page search over per-page
// representative vectors picks the key pages each chunk attends to.  Readings
// (the page gives no formula): a page's representative vector is the mean of
// its keys per kv-head; its score is the dot product with the chunk's mean
// query over all C tokens and the query heads of the kv-head's group; exact
// ties go to the lower page index; the chosen pages are written ascending.
//
// All four kernels are HBM- or latency-bound; none uses atomics on global
// memory, so every result is bitwise reproducible.
#include <mutex>

#include "common.h"
#include "launch.h"
#include "trace.h"

namespace oomb {

// ---------------------------------------------------------------------------
// rep[first + i][h][:] = mean_r k_pool[pt[first + i]][h][r][:]
// One workgroup per (page, kv-head): 16-byte coalesced loads of the page's
// contiguous ps x D block, per-thread fp32 partial sums, fixed-order LDS
// reduction.
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void rep_update_kernel(const T* __restrict__ k_pool,
                                                         const int32_t* __restrict__ pt, int first,
                                                         int hkv, int ps, float* __restrict__ rep) {
  constexpr int VEC = 16 / sizeof(T);
  constexpr int CPR = D / VEC;          // 16-byte groups per key row
  constexpr int RG = 256 / CPR;         // rows handled in parallel
  __shared__ float red[RG][D + 1];
  const int page = first + blockIdx.x / hkv;
  const int h = blockIdx.x % hkv;
  const int tid = threadIdx.x;
  const int cg = tid % CPR, rg = tid / CPR;
  const int64_t base = ((int64_t)pt[page] * hkv + h) * ps * D;
  float acc[VEC];
#pragma unroll
  for (int i = 0; i < VEC; ++i) acc[i] = 0.f;
  for (int r = rg; r < ps; r += RG) {
    const T* src = k_pool + base + (int64_t)r * D + cg * VEC;
    if constexpr (sizeof(T) == 2) {
      const bf16x8 v = *reinterpret_cast<const bf16x8*>(src);
#pragma unroll
      for (int i = 0; i < VEC; ++i) acc[i] += (float)v[i];
    } else {
      const f32x4 v = *reinterpret_cast<const f32x4*>(src);
#pragma unroll
      for (int i = 0; i < VEC; ++i) acc[i] += v[i];
    }
  }
#pragma unroll
  for (int i = 0; i < VEC; ++i) red[rg][cg * VEC + i] = acc[i];
  __syncthreads();
  if (tid < D) {
    float s = 0.f;
    for (int g = 0; g < RG; ++g) s += red[g][tid];
    rep[((int64_t)page * hkv + h) * D + tid] = s / (float)ps;
  }
}

// ---------------------------------------------------------------------------
// Chunk-mean query, stage 1: partial[b][h][:] = sum over the tokens of block b
// and the G heads of group h of q[t][g][:].
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void qmean_partial_kernel(const T* __restrict__ q, int c, int hq,
                                                            int hkv, int tpb, float* __restrict__ partial) {
  constexpr int VEC = 16 / sizeof(T);
  const int G = hq / hkv;
  const int NC = hkv * D / VEC;   // 16-byte column groups of the [hkv][D] output
  const int TG = 256 / NC;        // token groups
  extern __shared__ float red[];  // [TG][hkv * D]
  const int tid = threadIdx.x;
  const int col = tid % NC, tg = tid / NC;
  const int h = (col * VEC) / D, d0 = (col * VEC) % D;
  const int t0 = blockIdx.x * tpb, t1 = min(c, t0 + tpb);
  float acc[VEC];
#pragma unroll
  for (int i = 0; i < VEC; ++i) acc[i] = 0.f;
  if (tg < TG) {
    // (token, head) pairs of the block, flattened so that the unrolled loop
    // keeps several independent loads in flight
    const int n = (t1 - t0) * G;
#pragma unroll 8
    for (int k = tg; k < n; k += TG) {
      const int t = t0 + k / G, gi = k % G;
      const T* src = q + ((int64_t)t * hq + h * G + gi) * D + d0;
      if constexpr (sizeof(T) == 2) {
        const bf16x8 v = *reinterpret_cast<const bf16x8*>(src);
#pragma unroll
        for (int i = 0; i < VEC; ++i) acc[i] += (float)v[i];
      } else {
        const f32x4 v = *reinterpret_cast<const f32x4*>(src);
#pragma unroll
        for (int i = 0; i < VEC; ++i) acc[i] += v[i];
      }
    }
#pragma unroll
    for (int i = 0; i < VEC; ++i) red[tg * hkv * D + col * VEC + i] = acc[i];
  }
  __syncthreads();
  for (int o = tid; o < hkv * D; o += 256) {
    float s = 0.f;
    for (int g = 0; g < TG; ++g) s += red[g * hkv * D + o];
    partial[(int64_t)blockIdx.x * hkv * D + o] = s;
  }
}

// Stage 2: qbar[h][:] = (sum over blocks of partial) / (C * G).  A workgroup
// takes 64 output columns; its four waves sum every fourth block, then add their
// four sums in a fixed order.
__global__ __launch_bounds__(256) void qmean_final_kernel(const float* __restrict__ partial, int nblk,
                                                          int width, float inv_count,
                                                          float* __restrict__ qbar) {
  __shared__ float red[4][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int o = blockIdx.x * 64 + lane;
  float s = 0.f;
  if (o < width) {
#pragma unroll 8
    for (int b = wave; b < nblk; b += 4) s += partial[(int64_t)b * width + o];
  }
  red[wave][lane] = s;
  __syncthreads();
  if (wave == 0 && o < width) qbar[o] = (((red[0][lane] + red[1][lane]) + red[2][lane]) + red[3][lane]) * inv_count;
}

// ---------------------------------------------------------------------------
// scores[h][n] = qbar[h] . rep[n][h], n < N.  Each thread takes 4 floats of a
// page's [hkv][D] row; the D/4 threads of one head reduce with lane shuffles.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void scores_kernel(const float* __restrict__ rep,
                                                     const float* __restrict__ qbar, int n, int hkv,
                                                     int ppb, float* __restrict__ scores) {
  constexpr int TPH = D / 4;              // threads per head (16 or 32 lanes, aligned)
  const int TPP = hkv * TPH;              // threads per page
  const int PPI = 256 / TPP;              // pages per iteration
  const int tid = threadIdx.x;
  const int slot = tid / TPP, w = tid % TPP;
  const int h = w / TPH;
  const bool lane_ok = slot < PPI;
  f32x4 qv = {0.f, 0.f, 0.f, 0.f};
  if (lane_ok) qv = *reinterpret_cast<const f32x4*>(qbar + w * 4);
  const int p0 = blockIdx.x * ppb, p1 = min(n, p0 + ppb);
  for (int base = p0; base < p1; base += PPI) {
    const int page = base + slot;
    const bool ok = lane_ok && page < p1;
    float s = 0.f;
    if (ok) {
      const f32x4 r = *reinterpret_cast<const f32x4*>(rep + (int64_t)page * hkv * D + w * 4);
      s = qv[0] * r[0] + qv[1] * r[1] + qv[2] * r[2] + qv[3] * r[3];
    }
#pragma unroll
    for (int m = TPH / 2; m >= 1; m >>= 1) s = wave_xor_sum(s, m);
    if (ok && (w % TPH) == 0) scores[(int64_t)h * n + page] = s;
  }
}

// ---------------------------------------------------------------------------
// Top-K per kv-head: MSB-first radix select (4 passes of 8 bits) on
// order-preserving keys of the fp32 scores finds the K-th largest key T and how
// many keys equal to T are taken; a final pass in page order emits every page
// with key > T and the lowest-index pages with key == T, so the output is
// ascending and ties go to the lower page.  One 1024-thread workgroup per head.
// With R > 0 each thread loads its keys (pages tid + 1024 r, r < R) once, all
// loads in flight together, and every pass reads them from registers; R = 0
// re-reads the scores from memory in each pass (N > 1024 * 32).  Each wave
// counts into its own LDS histogram: the leading digits of the scores are
// shared by most pages, and one histogram would make all 16 waves' atomic adds
// wait on the same few bins.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t b = __float_as_uint(f == 0.f ? 0.f : f);  // -0 and +0 are one key
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / 64;

template <int R>
__global__ __launch_bounds__(kTopkThreads) void topk_kernel(const float* __restrict__ scores, int n, int k,
                                                            int32_t* __restrict__ sel) {
  __shared__ uint32_t hist[kTopkWaves][256];
  __shared__ uint32_t sh_digit, sh_krem;
  __shared__ uint32_t wave_tot[2][kTopkWaves];
  const int h = blockIdx.x;
  const float* s = scores + (int64_t)h * n;
  int32_t* out = sel + (int64_t)h * k;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  uint32_t kr[R > 0 ? R : 1];
  if constexpr (R > 0) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int i = tid + kTopkThreads * r;
      kr[r] = i < n ? order_key(s[i]) : 0u;
    }
  }

  uint32_t prefix = 0, mask = 0, krem = (uint32_t)k;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int b = tid; b < kTopkWaves * 256; b += kTopkThreads) (&hist[0][0])[b] = 0;
    __syncthreads();
    if constexpr (R > 0) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int i = tid + kTopkThreads * r;
        if (i < n && (kr[r] & mask) == prefix) atomicAdd(&hist[wave][(kr[r] >> shift) & 255u], 1u);
      }
    } else {
      for (int i = tid; i < n; i += kTopkThreads) {
        const uint32_t key = order_key(s[i]);
        if ((key & mask) == prefix) atomicAdd(&hist[wave][(key >> shift) & 255u], 1u);
      }
    }
    __syncthreads();
    if (wave == 0) {
      // lane L owns bins 255-4L .. 252-4L (descending); inclusive scan from the top
      uint32_t c[4], local = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        c[i] = 0;
#pragma unroll
        for (int w = 0; w < kTopkWaves; ++w) c[i] += hist[w][255 - 4 * lane - i];
        local += c[i];
      }
      uint32_t incl = local;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t v = __shfl_up(incl, off, 64);
        if (lane >= off) incl += v;
      }
      const uint64_t hit = __ballot(incl >= krem);
      const int fl = __ffsll((unsigned long long)hit) - 1;
      if (lane == fl) {
        uint32_t cum = incl - local;
        for (int i = 0; i < 4; ++i) {
          if (cum + c[i] >= krem) {
            sh_digit = 255 - 4 * lane - i;
            sh_krem = krem - cum;
            break;
          }
          cum += c[i];
        }
      }
    }
    __syncthreads();
    prefix |= sh_digit << shift;
    mask |= 255u << shift;
    krem = sh_krem;
    __syncthreads();
  }
  const uint32_t T = prefix;
  // emit in page order
  uint32_t out_base = 0, eq_base = 0;
  const uint64_t below = (1ull << lane) - 1ull;
  auto emit = [&](int i, uint32_t key) {
    const bool gt = i < n && key > T;
    const bool eq = i < n && key == T;
    const uint64_t beq = __ballot(eq);
    if (lane == 0) wave_tot[0][wave] = __popcll(beq);
    __syncthreads();
    uint32_t eq_rank = eq_base + __popcll(beq & below);
    uint32_t eq_all = 0;
    for (int w = 0; w < kTopkWaves; ++w) {
      if (w < wave) eq_rank += wave_tot[0][w];
      eq_all += wave_tot[0][w];
    }
    const bool take = gt || (eq && eq_rank < krem);
    const uint64_t btk = __ballot(take);
    if (lane == 0) wave_tot[1][wave] = __popcll(btk);
    __syncthreads();
    uint32_t pos = out_base + __popcll(btk & below);
    uint32_t tk_all = 0;
    for (int w = 0; w < kTopkWaves; ++w) {
      if (w < wave) pos += wave_tot[1][w];
      tk_all += wave_tot[1][w];
    }
    if (take && pos < (uint32_t)k) out[pos] = i;
    out_base += tk_all;
    eq_base += eq_all;
    __syncthreads();
  };
  if constexpr (R > 0) {
    // With the keys in registers, two barriers in all: page r*1024 + tid
    // belongs to group (r, wave), and the groups in (r, wave) order are the
    // pages in order.  Each wave counts its pages equal to T and above it per
    // group, wave 0 turns the counts into offsets (where a group's taken
    // pages start, and how many pages equal to T come before it), then every
    // thread places its pages.
    constexpr int Q = R * kTopkWaves;
    constexpr int E = (Q + 63) / 64;  // groups per lane of wave 0
    __shared__ uint32_t grp_eq[Q], grp_tk[Q];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int i = r * kTopkThreads + tid;
      const uint64_t bgt = __ballot(i < n && kr[r] > T);
      const uint64_t beq = __ballot(i < n && kr[r] == T);
      if (lane == 0) {
        grp_tk[r * kTopkWaves + wave] = __popcll(bgt);
        grp_eq[r * kTopkWaves + wave] = __popcll(beq);
      }
    }
    __syncthreads();
    if (wave == 0) {
      uint32_t ce[E], cg[E], sum_eq = 0;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int q = lane * E + e;
        ce[e] = q < Q ? grp_eq[q] : 0u;
        cg[e] = q < Q ? grp_tk[q] : 0u;
        sum_eq += ce[e];
      }
      uint32_t incl = sum_eq;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t v = __shfl_up(incl, off, 64);
        if (lane >= off) incl += v;
      }
      uint32_t eq_off = incl - sum_eq, tk[E], sum_tk = 0, eo[E];
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const uint32_t room = krem > eq_off ? krem - eq_off : 0u;  // pages equal to T still to take
        tk[e] = cg[e] + (ce[e] < room ? ce[e] : room);
        eo[e] = eq_off;
        eq_off += ce[e];
        sum_tk += tk[e];
      }
      incl = sum_tk;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t v = __shfl_up(incl, off, 64);
        if (lane >= off) incl += v;
      }
      uint32_t tk_off = incl - sum_tk;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int q = lane * E + e;
        if (q < Q) {
          grp_eq[q] = eo[e];
          grp_tk[q] = tk_off;
        }
        tk_off += tk[e];
      }
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int i = r * kTopkThreads + tid, q = r * kTopkWaves + wave;
      const bool gt = i < n && kr[r] > T;
      const bool eq = i < n && kr[r] == T;
      const uint64_t beq = __ballot(eq);
      const bool take = gt || (eq && grp_eq[q] + __popcll(beq & below) < krem);
      const uint64_t btk = __ballot(take);
      const uint32_t pos = grp_tk[q] + __popcll(btk & below);
      if (take && pos < (uint32_t)k) out[pos] = i;
    }
  } else {
    for (int c0 = 0; c0 < n; c0 += kTopkThreads) {
      const int i = c0 + tid;
      emit(i, i < n ? order_key(s[i]) : 0u);
    }
  }
}

// K >= N: every prior page, in order.
__global__ __launch_bounds__(256) void identity_sel_kernel(int n, int hkv, int32_t* __restrict__ sel) {
  const int64_t total = (int64_t)n * hkv;
  for (int64_t i = blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256)
    sel[i] = (int32_t)(i % n);
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
template <typename T, int D>
static hipError_t rep_update_t(const Shape& s, const void* k_pool, const int32_t* pt, int first, int count,
                               float* rep, hipStream_t st) {
  Traced tr(st, "rep_update_kernel");
  hipLaunchKernelGGL((rep_update_kernel<T, D>), dim3(count * s.hkv), dim3(256), 0, st,
                     (const T*)k_pool, pt, first, s.hkv, s.ps, rep);
  return hipGetLastError();
}

hipError_t launch_rep_update(const Shape& s, const void* k_pool, const int32_t* pt, int first, int count,
                             float* rep, hipStream_t st) {
  if (s.bf16) return s.d == 128 ? rep_update_t<__bf16, 128>(s, k_pool, pt, first, count, rep, st)
                                : rep_update_t<__bf16, 64>(s, k_pool, pt, first, count, rep, st);
  return s.d == 128 ? rep_update_t<float, 128>(s, k_pool, pt, first, count, rep, st)
                    : rep_update_t<float, 64>(s, k_pool, pt, first, count, rep, st);
}

SelectPlan select_plan(const Shape& s) {
  SelectPlan p;
  p.tpb = (s.c + kQmeanBlocks - 1) / kQmeanBlocks;
  p.nblk = (s.c + p.tpb - 1) / p.tpb;
  const size_t width = (size_t)s.hkv * s.d;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += (bytes + 255) & ~(size_t)255;
    return at;
  };
  p.off_partial = take((size_t)p.nblk * width * 4);
  p.off_qbar = take(width * 4);
  p.off_scores = take((size_t)s.hkv * (s.n > 0 ? s.n : 1) * 4);
  p.bytes = off;
  return p;
}

template <typename T, int D>
static hipError_t select_t(const Shape& s, const SelectPlan& p, const void* q, const float* rep, int32_t* sel,
                           float* scores_out, char* ws, hipStream_t st) {
  float* partial = (float*)(ws + p.off_partial);
  float* qbar = (float*)(ws + p.off_qbar);
  float* scores = scores_out ? scores_out : (float*)(ws + p.off_scores);
  const int width = s.hkv * D;
  const int nc = width / (16 / (int)sizeof(T));
  const int tg = 256 / nc;
  {
    Traced tr(st, "qmean_partial_kernel");
    hipLaunchKernelGGL((qmean_partial_kernel<T, D>), dim3(p.nblk), dim3(256), (size_t)tg * width * 4, st,
                       (const T*)q, s.c, s.hq, s.hkv, p.tpb, partial);
  }
  {
    Traced tr(st, "qmean_final_kernel");
    hipLaunchKernelGGL(qmean_final_kernel, dim3((width + 63) / 64), dim3(256), 0, st, (const float*)partial, p.nblk, width,
                       1.0f / ((float)s.c * (float)(s.hq / s.hkv)), qbar);
  }
  const int ppb = 16;
  {
    Traced tr(st, "scores_kernel");
    hipLaunchKernelGGL((scores_kernel<D>), dim3((s.n + ppb - 1) / ppb), dim3(256), 0, st, rep,
                       (const float*)qbar, s.n, s.hkv, ppb, scores);
  }
  if (s.keff >= s.n) {
    const int64_t total = (int64_t)s.n * s.hkv;
    const int grid = (int)((total + 255) / 256 < 4096 ? (total + 255) / 256 : 4096);
    Traced tr(st, "identity_sel_kernel");
    hipLaunchKernelGGL(identity_sel_kernel, dim3(grid), dim3(256), 0, st, s.n, s.hkv, sel);
  } else {
    Traced tr(st, "topk_kernel");
    const dim3 grid(s.hkv), block(kTopkThreads);
    const float* sc = scores;
    if (s.n <= 2 * kTopkThreads) hipLaunchKernelGGL(topk_kernel<2>, grid, block, 0, st, sc, s.n, s.keff, sel);
    else if (s.n <= 8 * kTopkThreads) hipLaunchKernelGGL(topk_kernel<8>, grid, block, 0, st, sc, s.n, s.keff, sel);
    else if (s.n <= 32 * kTopkThreads) hipLaunchKernelGGL(topk_kernel<32>, grid, block, 0, st, sc, s.n, s.keff, sel);
    else hipLaunchKernelGGL(topk_kernel<0>, grid, block, 0, st, sc, s.n, s.keff, sel);
  }
  return hipGetLastError();
}

// Scratch of the allocation-free selection (oomb_select_topk_noalloc): one
// array per device, resident until the process ends.  In host code the name
// `scratch` is only a stand-in for the symbol, not a device address: the
// address is taken once per device with hipGetSymbolAddress, with that device
// current, and only that address is handed to the kernels.
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

hipError_t noalloc_scratch(void** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex lock;
  static void* per_device[kMaxDevices];
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> guard(lock);
  if (!per_device[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    per_device[dev] = p;
  }
  *out = per_device[dev];
  return hipSuccess;
}

hipError_t launch_select(const Shape& s, const void* q, const float* rep, int32_t* sel, float* scores_out,
                         void* ws, hipStream_t st) {
  const SelectPlan p = select_plan(s);
  char* w = (char*)ws;
  if (s.bf16) return s.d == 128 ? select_t<__bf16, 128>(s, p, q, rep, sel, scores_out, w, st)
                                : select_t<__bf16, 64>(s, p, q, rep, sel, scores_out, w, st);
  return s.d == 128 ? select_t<float, 128>(s, p, q, rep, sel, scores_out, w, st)
                    : select_t<float, 64>(s, p, q, rep, sel, scores_out, w, st);
}

}  // namespace oomb
