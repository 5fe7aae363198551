// launch.h -- host-side plan of one chunk step and the kernel launchers behind
// the C ABI (include/oomb.h).
#pragma once

#include <hip/hip_runtime.h>

#include <algorithm>
#include <stddef.h>
#include <stdint.h>

#include "common.h"
#include "shape.h"

namespace oomb {

inline Geo make_geo(const Shape& s) {
  Geo g;
  g.hq = s.hq;
  g.hkv = s.hkv;
  g.G = s.hq / s.hkv;
  g.g_magic = ((1ull << 40) + (uint64_t)g.G - 1) / (uint64_t)g.G;
  g.c = s.c;
  g.n = s.n;
  g.keff = s.keff;
  g.ps_log2 = s.ps_log2;
  g.n_slots = s.n_slots;
  g.scale = s.scale;
  return g;
}

constexpr int kQmeanBlocks = 256;  // token blocks of the chunk-mean-query reduction

struct SelectPlan {
  int tpb, nblk;                                   // tokens per block, blocks
  size_t off_partial, off_qbar, off_scores, bytes;  // workspace layout
};
SelectPlan select_plan(const Shape& s);

struct BwdPlan {
  size_t off_dt;                  // Dt = rowsum(dO * O) per (head, token), fp32 [Hq][C]
  size_t off_lse2;                // lse * log2(e) per (head, token), fp32 [Hq][C]
  size_t off_bias;                // dK/dV bias operands per (head, token), bf16 [Hq][C][16]
  size_t off_part_k, off_part_v;  // dK / dV partial sums of row splits 1.., fp32 [splits-1][Hkv][nkeys][D]
  size_t off_part2_k, off_part2_v;  // second halves of the chunk key blocks' shares (sub = 2),
                                    // fp32 [splits][Hkv][nkeys - key0_sub][D]
  int splits;                     // workgroups sharing one key block's query rows
  int sub;                        // 2: each share of a chunk key block is split again in two
  int key0_sub;                   // first key of the chunk key blocks
  size_t bytes;
};
BwdPlan bwd_plan(const Shape& s);

hipError_t launch_rep_update(const Shape& s, const void* k_pool, const int32_t* pt, int first, int count,
                             float* rep, hipStream_t st);
hipError_t launch_select(const Shape& s, const void* q, const float* rep, int32_t* sel, float* scores_out,
                         void* ws, hipStream_t st);
// The allocation-free selection's per-device scratch (kNoAllocScratchBytes,
// 256-byte aligned): its device address on the current device.
constexpr size_t kNoAllocScratchBytes = (size_t)OOMB_NOALLOC_SCRATCH_BYTES;
hipError_t noalloc_scratch(void** out);
hipError_t launch_fwd(const Shape& s, const void* q, const void* k_pool, const void* v_pool, const int32_t* pt,
                      const int32_t* sel, void* o, float* lse, hipStream_t st);
hipError_t launch_bwd(const Shape& s, const void* q, const void* k_pool, const void* v_pool, const int32_t* pt,
                      const int32_t* sel, const void* o, const float* lse, const void* dout, float* dq,
                      float* dk_pool, float* dv_pool, void* ws, hipStream_t st);

// Page-block copies between host page pools and a device staging pool.
constexpr int kStageSelected = 1;  // the selected (kv-head, page) blocks
constexpr int kStageChunk = 2;     // every kv-head of the chunk's own pages
constexpr int kCopyBlocks = 8;     // workgroups of one copy kernel
// host_k / host_v: the pools on the host side of the copy (src_slots slots);
// selected blocks are copied only for logical pages in [page_lo, page_hi).
hipError_t launch_stage_copy(const Shape& s, const void* host_k, const void* host_v, void* stage_k, void* stage_v,
                             const int32_t* pt, const int32_t* sel, int parts, bool to_host, int src_slots,
                             int page_lo, int page_hi, hipStream_t st);
hipError_t launch_grad_flush(const Shape& s, float* stage_dk, float* stage_dv, float* host_dk, float* host_dv,
                             const int32_t* pt, const int32_t* sel, hipStream_t st);
hipError_t launch_grads_out(const Shape& s, float* stage_dk, float* stage_dv, float* out_dk, float* out_dv,
                            hipStream_t st);
hipError_t launch_stage_tables(const Shape& s, int32_t* sel_stage, int32_t* pt_stage, hipStream_t st);
hipError_t launch_check_tables(const Shape& s, const int32_t* pt, const int32_t* sel, int32_t* counts,
                               int32_t* slot_uses, hipStream_t st);
hipError_t launch_probe_mfma(int n_blocks, int iters, float* out, hipStream_t st);

}  // namespace oomb
