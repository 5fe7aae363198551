// offload.hip -- page-block copies between the host page pools and a device
// staging pool, for keeping the KV cache and its gradients in CPU memory
// (OOMB page, technical summary, section 2, "Asynchronous CPU Offloading": the
// context-length-dependent KV cache and gradients move between GPU and CPU
// memory asynchronously, overlapped with compute).
//
// The host pools are pinned host memory addressed by the device through its
// mapped view, so one kernel reads or writes them over the host link at full
// link rate whatever the block size, with the block list taken from the page
// table and the selection where they already are, on the device.  Separate
// DMA copies would cost a command each per (page, kv-head) block (32 KB at the
// Qwen2.5-7B shape), and the DMA engines then run far below link rate.
//
// The kernels run on few workgroups (kCopyBlocks of kCopyThreads), so that on
// a second stream they take a small share of the compute units from the
// attention kernels they overlap (a compute unit that holds a copy wave has no
// room left for an attention workgroup, whose waves fill its register files);
// each thread keeps four 16-byte accesses in flight.  Fewer, larger copy
// workgroups were slower: the link rate a compute unit sustains is limited by
// its own outstanding requests.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "launch.h"
#include "trace.h"

namespace oomb {

namespace {

constexpr int kCopyThreads = 512;
constexpr int kCopyUnroll = 4;  // 16-byte accesses in flight per thread

struct CopyArgs {
  // tensor t (0: K or dK, 1: V or dV): host pool and staging pool
  const void* src[2];
  void* dst[2];
  const int32_t* pt;   // logical page -> host slot
  const int32_t* sel;  // [Hkv][K_eff] logical pages
  int hkv, keff, n, n_host_slots;
  int page_lo, page_hi;       // selected blocks of logical pages outside [page_lo, page_hi) are skipped
  int first_block, n_blocks;  // block range: [0, hkv*keff) selected, then (C/ps)*hkv chunk blocks
  int vec_per_block;          // block bytes / 16
  int to_host;                // 0: host -> staging, 1: staging -> host
};

// Block b of the staging layout: head h's block of (host slot, staging slot).
// Returns false for a selection or page-table entry out of range (skipped).
__device__ inline bool block_place(const CopyArgs& a, int b, int& host_slot, int& stage_slot, int& h) {
  const int nsel = a.hkv * a.keff;
  int logical;
  if (b < nsel) {
    h = b / a.keff;
    stage_slot = b;
    logical = a.sel[b];  // sel[h][k], k = b % keff
    if (logical < 0 || logical >= a.n || logical < a.page_lo || logical >= a.page_hi) return false;
  } else {
    const int j = b - nsel;
    h = j % a.hkv;
    stage_slot = nsel + j / a.hkv;
    logical = a.n + j / a.hkv;
  }
  host_slot = a.pt[logical];
  return host_slot >= 0 && host_slot < a.n_host_slots;
}

// Plain copies, in either direction.
__global__ __launch_bounds__(kCopyThreads) void page_copy_kernel(CopyArgs a) {
  const int items = 2 * a.n_blocks;
  for (int it = blockIdx.x; it < items; it += gridDim.x) {
    const int t = it & 1, b = a.first_block + (it >> 1);
    int hs, ss, h;
    if (!block_place(a, b, hs, ss, h)) continue;
    // offsets of the two blocks in 16-byte vectors
    const int64_t vh = ((int64_t)hs * a.hkv + h) * a.vec_per_block;
    const int64_t vs = ((int64_t)ss * a.hkv + h) * a.vec_per_block;
    const int4* __restrict__ s = (const int4*)a.src[t] + (a.to_host ? vs : vh);
    int4* __restrict__ d = (int4*)a.dst[t] + (a.to_host ? vh : vs);
    // four loads in flight per thread, held in named registers: a private
    // array here is placed in LDS by the compiler, and 16 KB of LDS would keep
    // this kernel off the compute units an attention kernel occupies
    const int n = a.vec_per_block;
    for (int i = threadIdx.x; i < n; i += kCopyThreads * kCopyUnroll) {
      int4 r0, r1, r2, r3;
      r0 = s[i];
      if (i + kCopyThreads < n) r1 = s[i + kCopyThreads];
      if (i + 2 * kCopyThreads < n) r2 = s[i + 2 * kCopyThreads];
      if (i + 3 * kCopyThreads < n) r3 = s[i + 3 * kCopyThreads];
      d[i] = r0;
      if (i + kCopyThreads < n) d[i + kCopyThreads] = r1;
      if (i + 2 * kCopyThreads < n) d[i + 2 * kCopyThreads] = r2;
      if (i + 3 * kCopyThreads < n) d[i + 3 * kCopyThreads] = r3;
    }
  }
}

// Gradient flush: host += staging, then staging = 0 (fp32; src = staging,
// dst = host pools).
__global__ __launch_bounds__(kCopyThreads) void grad_flush_kernel(CopyArgs a) {
  const int items = 2 * a.n_blocks;
  for (int it = blockIdx.x; it < items; it += gridDim.x) {
    const int t = it & 1, b = a.first_block + (it >> 1);
    int hs, ss, h;
    if (!block_place(a, b, hs, ss, h)) continue;
    float4* __restrict__ st = (float4*)a.src[t] + ((int64_t)ss * a.hkv + h) * a.vec_per_block;
    float4* __restrict__ ho = (float4*)a.dst[t] + ((int64_t)hs * a.hkv + h) * a.vec_per_block;
    for (int i0 = 0; i0 < a.vec_per_block; i0 += kCopyThreads * kCopyUnroll) {
      float4 x[kCopyUnroll], y[kCopyUnroll];
#pragma unroll
      for (int u = 0; u < kCopyUnroll; ++u) {
        const int i = i0 + u * kCopyThreads + threadIdx.x;
        if (i < a.vec_per_block) {
          x[u] = ho[i];
          y[u] = st[i];
        }
      }
#pragma unroll
      for (int u = 0; u < kCopyUnroll; ++u) {
        const int i = i0 + u * kCopyThreads + threadIdx.x;
        if (i < a.vec_per_block) {
          float4 z;
          z.x = x[u].x + y[u].x;
          z.y = x[u].y + y[u].y;
          z.z = x[u].z + y[u].z;
          z.w = x[u].w + y[u].w;
          ho[i] = z;
          st[i] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
      }
    }
  }
}

// Gradients out: staged block b (the staging layout's block order: selected
// blocks, then the chunk's pages kv-head by kv-head) -> block b of a compact
// buffer (host memory), then the staged block is set to zero.
__global__ __launch_bounds__(kCopyThreads) void grad_out_kernel(CopyArgs a) {
  const int items = 2 * a.n_blocks;
  for (int it = blockIdx.x; it < items; it += gridDim.x) {
    const int t = it & 1, b = it >> 1;
    const int nsel = a.hkv * a.keff;
    int ss, h;
    if (b < nsel) {
      h = b / a.keff;
      ss = b;
    } else {
      h = (b - nsel) % a.hkv;
      ss = nsel + (b - nsel) / a.hkv;
    }
    int4* __restrict__ st = (int4*)a.src[t] + ((int64_t)ss * a.hkv + h) * a.vec_per_block;
    int4* __restrict__ d = (int4*)a.dst[t] + (int64_t)b * a.vec_per_block;
    const int n = a.vec_per_block;
    const int4 z = make_int4(0, 0, 0, 0);
    for (int i = threadIdx.x; i < n; i += kCopyThreads * kCopyUnroll) {
      int4 r0, r1, r2, r3;
      r0 = st[i];
      if (i + kCopyThreads < n) r1 = st[i + kCopyThreads];
      if (i + 2 * kCopyThreads < n) r2 = st[i + 2 * kCopyThreads];
      if (i + 3 * kCopyThreads < n) r3 = st[i + 3 * kCopyThreads];
      d[i] = r0;
      st[i] = z;
      if (i + kCopyThreads < n) {
        d[i + kCopyThreads] = r1;
        st[i + kCopyThreads] = z;
      }
      if (i + 2 * kCopyThreads < n) {
        d[i + 2 * kCopyThreads] = r2;
        st[i + 2 * kCopyThreads] = z;
      }
      if (i + 3 * kCopyThreads < n) {
        d[i + 3 * kCopyThreads] = r3;
        st[i + 3 * kCopyThreads] = z;
      }
    }
  }
}

__global__ void stage_tables_kernel(int32_t* sel_stage, int nsel, int32_t* pt_stage, int n_stage) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < nsel) sel_stage[i] = i;
  if (i < n_stage) pt_stage[i] = i;
}

CopyArgs copy_args(const Shape& s, int eb, const int32_t* pt, const int32_t* sel, int parts) {
  CopyArgs a{};
  a.pt = pt;
  a.sel = sel;
  a.hkv = s.hkv;
  a.keff = s.keff;
  a.n = s.n;
  a.n_host_slots = s.n_slots;
  a.page_lo = 0;
  a.page_hi = s.n;
  const int nsel = s.hkv * s.keff, nchunk = (s.c / s.ps) * s.hkv;
  a.first_block = (parts & kStageSelected) ? 0 : nsel;
  a.n_blocks = ((parts & kStageSelected) ? nsel : 0) + ((parts & kStageChunk) ? nchunk : 0);
  a.vec_per_block = s.ps * s.d * eb / 16;  // ps * D elements of eb bytes
  return a;
}

int copy_grid(const CopyArgs& a) { return std::min(kCopyBlocks, std::max(1, 2 * a.n_blocks)); }

}  // namespace

hipError_t launch_stage_copy(const Shape& s, const void* host_k, const void* host_v, void* stage_k, void* stage_v,
                             const int32_t* pt, const int32_t* sel, int parts, bool to_host, int src_slots,
                             int page_lo, int page_hi, hipStream_t st) {
  CopyArgs a = copy_args(s, s.bf16 ? 2 : 4, pt, sel, parts);
  if (a.n_blocks == 0) return hipSuccess;
  a.n_host_slots = src_slots;
  a.page_lo = page_lo;
  a.page_hi = page_hi;
  a.to_host = to_host ? 1 : 0;
  if (to_host) {
    a.src[0] = stage_k;
    a.src[1] = stage_v;
    a.dst[0] = const_cast<void*>(host_k);
    a.dst[1] = const_cast<void*>(host_v);
  } else {
    a.src[0] = host_k;
    a.src[1] = host_v;
    a.dst[0] = stage_k;
    a.dst[1] = stage_v;
  }
  Traced tr(st, to_host ? "page_offload_kernel" : "page_gather_kernel");
  hipLaunchKernelGGL(page_copy_kernel, dim3(copy_grid(a)), dim3(kCopyThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_grad_flush(const Shape& s, float* stage_dk, float* stage_dv, float* host_dk, float* host_dv,
                             const int32_t* pt, const int32_t* sel, hipStream_t st) {
  CopyArgs a = copy_args(s, 4, pt, sel, kStageSelected | kStageChunk);
  if (a.n_blocks == 0) return hipSuccess;
  a.src[0] = stage_dk;
  a.src[1] = stage_dv;
  a.dst[0] = host_dk;
  a.dst[1] = host_dv;
  Traced tr(st, "grad_flush_kernel");
  hipLaunchKernelGGL(grad_flush_kernel, dim3(copy_grid(a)), dim3(kCopyThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_grads_out(const Shape& s, float* stage_dk, float* stage_dv, float* out_dk, float* out_dv,
                            hipStream_t st) {
  CopyArgs a = copy_args(s, 4, nullptr, nullptr, kStageSelected | kStageChunk);
  if (a.n_blocks == 0) return hipSuccess;
  a.src[0] = stage_dk;
  a.src[1] = stage_dv;
  a.dst[0] = out_dk;
  a.dst[1] = out_dv;
  Traced tr(st, "grad_out_kernel");
  hipLaunchKernelGGL(grad_out_kernel, dim3(copy_grid(a)), dim3(kCopyThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_stage_tables(const Shape& s, int32_t* sel_stage, int32_t* pt_stage, hipStream_t st) {
  const int nsel = s.hkv * s.keff, n_stage = nsel + s.c / s.ps;
  hipLaunchKernelGGL(stage_tables_kernel, dim3((n_stage + 255) / 256), dim3(256), 0, st, sel_stage, nsel, pt_stage,
                     n_stage);
  return hipGetLastError();
}

}  // namespace oomb
