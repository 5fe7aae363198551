// abi.hip -- the extern "C" entry points of include/oomb.h: validate the
// descriptor, sizes and pointers on the host (before any HIP call), then
// enqueue the kernels on the caller's stream.  Nothing is allocated, freed or
// synchronised here.
#include <math.h>

#include <algorithm>
#include <stdint.h>

#include "launch.h"
#include "oomb.h"
#include "trace.h"

#define OOMB_API extern "C" __attribute__((visibility("default")))

namespace oomb {
TraceState& trace_state() {
  static TraceState t;
  return t;
}
}  // namespace oomb

namespace {

bool misaligned(const void* p) { return ((uintptr_t)p & 15u) != 0; }

int validate(const oomb_desc* d, oomb::Shape* s) { return oomb::validate_desc(d, s); }

// Every pointer non-NULL and 16-byte aligned.
int check_ptrs(std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if (!p) return OOMB_ERR_NULL_PTR;
  for (const void* p : ps)
    if (misaligned(p)) return OOMB_ERR_MISALIGNED;
  return OOMB_OK;
}

int launched(hipError_t e) { return e == hipSuccess ? OOMB_OK : OOMB_ERR_LAUNCH; }

}  // namespace

OOMB_API int oomb_rep_update(const oomb_desc* desc, const void* k_pool, const int32_t* page_table,
                             int32_t first_page, int32_t n_pages, float* rep, void* stream) {
  oomb::Shape s;
  int rc = validate(desc, &s);
  if (rc) return rc;
  if ((rc = check_ptrs({k_pool, page_table, rep}))) return rc;
  const int64_t pages_total = (int64_t)s.n + s.c / s.ps;
  if (first_page < 0 || n_pages < 0 || (int64_t)first_page + n_pages > pages_total ||
      (int64_t)first_page + n_pages > s.rep_cap)
    return OOMB_ERR_BAD_SHAPE;
  if (n_pages == 0) return OOMB_OK;
  (void)hipGetLastError();
  return launched(oomb::launch_rep_update(s, k_pool, page_table, first_page, n_pages, rep, (hipStream_t)stream));
}

OOMB_API size_t oomb_select_workspace_bytes(const oomb_desc* desc) {
  oomb::Shape s;
  if (validate(desc, &s)) return 0;
  return oomb::select_plan(s).bytes;
}

OOMB_API int oomb_select_topk(const oomb_desc* desc, const void* q, const float* rep, int32_t* sel,
                              float* scores_out, void* workspace, size_t workspace_bytes, void* stream) {
  oomb::Shape s;
  int rc = validate(desc, &s);
  if (rc) return rc;
  if ((rc = check_ptrs({q, rep}))) return rc;
  if (s.keff > 0 && (rc = check_ptrs({sel}))) return rc;
  if (scores_out && misaligned(scores_out)) return OOMB_ERR_MISALIGNED;
  const oomb::SelectPlan p = oomb::select_plan(s);
  if (!workspace || workspace_bytes < p.bytes) return OOMB_ERR_WORKSPACE;
  if (misaligned(workspace)) return OOMB_ERR_MISALIGNED;
  if (s.n == 0) return OOMB_OK;  // no candidate pages: nothing to score or select
  (void)hipGetLastError();
  return launched(oomb::launch_select(s, q, rep, sel, scores_out, workspace, (hipStream_t)stream));
}

OOMB_API int oomb_select_topk_noalloc(const oomb_desc* desc, const void* q, const float* rep, int32_t* sel,
                                      float* scores_out, void* stream) {
  oomb::Shape s;
  int rc = validate(desc, &s);
  if (rc) return rc;
  if ((rc = check_ptrs({q, rep}))) return rc;
  if (s.keff > 0 && (rc = check_ptrs({sel}))) return rc;
  if (scores_out && misaligned(scores_out)) return OOMB_ERR_MISALIGNED;
  const oomb::SelectPlan p = oomb::select_plan(s);
  if (p.bytes > oomb::kNoAllocScratchBytes) return OOMB_ERR_SCRATCH_LIMIT;
  if (s.n == 0) return OOMB_OK;
  (void)hipGetLastError();
  void* ws = nullptr;
  if (oomb::noalloc_scratch(&ws) != hipSuccess) {
    (void)hipGetLastError();
    return OOMB_ERR_LAUNCH;
  }
  return launched(oomb::launch_select(s, q, rep, sel, scores_out, ws, (hipStream_t)stream));
}

OOMB_API int oomb_attn_fwd(const oomb_desc* desc, const void* q, const void* k_pool, const void* v_pool,
                           const int32_t* page_table, const int32_t* sel, void* o, float* lse, void* stream) {
  oomb::Shape s;
  int rc = validate(desc, &s);
  if (rc) return rc;
  if ((rc = check_ptrs({q, k_pool, v_pool, page_table, o, lse}))) return rc;
  if (s.keff > 0 && (rc = check_ptrs({sel}))) return rc;
  (void)hipGetLastError();
  return launched(oomb::launch_fwd(s, q, k_pool, v_pool, page_table, sel, o, lse, (hipStream_t)stream));
}

OOMB_API size_t oomb_bwd_workspace_bytes(const oomb_desc* desc) {
  oomb::Shape s;
  if (validate(desc, &s)) return 0;
  return oomb::bwd_plan(s).bytes;
}

OOMB_API int oomb_attn_bwd(const oomb_desc* desc, const void* q, const void* k_pool, const void* v_pool,
                           const int32_t* page_table, const int32_t* sel, const void* o, const float* lse,
                           const void* dO, float* dq, float* dk_pool, float* dv_pool, void* workspace,
                           size_t workspace_bytes, void* stream) {
  oomb::Shape s;
  int rc = validate(desc, &s);
  if (rc) return rc;
  if ((rc = check_ptrs({q, k_pool, v_pool, page_table, o, lse, dO, dq, dk_pool, dv_pool}))) return rc;
  if (s.keff > 0 && (rc = check_ptrs({sel}))) return rc;
  const oomb::BwdPlan p = oomb::bwd_plan(s);
  if (!workspace || workspace_bytes < p.bytes) return OOMB_ERR_WORKSPACE;
  if (misaligned(workspace)) return OOMB_ERR_MISALIGNED;
  (void)hipGetLastError();
  return launched(oomb::launch_bwd(s, q, k_pool, v_pool, page_table, sel, o, lse, dO, dq, dk_pool, dv_pool,
                                   workspace, (hipStream_t)stream));
}

OOMB_API int oomb_host_view(const void* host_ptr, void** device_view) {
  if (!host_ptr || !device_view) return OOMB_ERR_NULL_PTR;
  void* v = nullptr;
  if (hipHostGetDevicePointer(&v, const_cast<void*>(host_ptr), 0) != hipSuccess || !v) {
    (void)hipGetLastError();
    return OOMB_ERR_NOT_MAPPED;
  }
  *device_view = v;
  return OOMB_OK;
}

namespace {
int stage_shape(const oomb_desc* desc, oomb::Shape* s, oomb_desc* staged) {
  int rc = validate(desc, s);
  if (rc) return rc;
  const int nsel = s->hkv * s->keff, n_stage = nsel + s->c / s->ps;
  *staged = *desc;
  staged->n_prior_pages = nsel;
  staged->top_k = s->keff;
  staged->n_slots = n_stage;
  staged->rep_capacity = n_stage;
  return OOMB_OK;
}
}  // namespace

OOMB_API int oomb_stage_desc(const oomb_desc* desc, oomb_desc* staged) {
  if (!staged) return OOMB_ERR_NULL_PTR;
  oomb::Shape s;
  oomb_desc t;
  int rc = stage_shape(desc, &s, &t);
  if (rc) return rc;
  oomb::Shape check;
  if ((rc = validate(&t, &check))) return rc;
  *staged = t;
  return OOMB_OK;
}

OOMB_API int oomb_stage_tables(const oomb_desc* desc, int32_t* sel_stage, int32_t* pt_stage, void* stream) {
  oomb::Shape s;
  int rc = validate(desc, &s);
  if (rc) return rc;
  if ((rc = check_ptrs({pt_stage}))) return rc;
  if (s.keff > 0 && (rc = check_ptrs({sel_stage}))) return rc;
  (void)hipGetLastError();
  return launched(oomb::launch_stage_tables(s, sel_stage, pt_stage, (hipStream_t)stream));
}

OOMB_API int oomb_stage_gather(const oomb_desc* desc, const void* src_k, const void* src_v, int32_t src_slots,
                               const int32_t* page_table, const int32_t* sel, int32_t parts, int32_t first_page,
                               int32_t n_pages, void* stage_k, void* stage_v, void* stream) {
  oomb::Shape s;
  int rc = validate(desc, &s);
  if (rc) return rc;
  if (parts < 1 || parts > (OOMB_STAGE_SELECTED | OOMB_STAGE_CHUNK)) return OOMB_ERR_BAD_SHAPE;
  if (src_slots <= 0 || first_page < 0 || n_pages < 0) return OOMB_ERR_BAD_SHAPE;
  if ((rc = check_ptrs({src_k, src_v, page_table, stage_k, stage_v}))) return rc;
  if ((parts & OOMB_STAGE_SELECTED) && s.keff > 0 && (rc = check_ptrs({sel}))) return rc;
  const int32_t* sel_used = (parts & OOMB_STAGE_SELECTED) ? sel : nullptr;
  const int64_t hi = std::min<int64_t>((int64_t)first_page + n_pages, s.n);
  (void)hipGetLastError();
  return launched(oomb::launch_stage_copy(s, src_k, src_v, stage_k, stage_v, page_table, sel_used, parts, false,
                                          src_slots, first_page, (int)hi, (hipStream_t)stream));
}

OOMB_API int oomb_stage_offload_chunk(const oomb_desc* desc, const void* stage_k, const void* stage_v,
                                      const int32_t* page_table, void* host_k, void* host_v, void* stream) {
  oomb::Shape s;
  int rc = validate(desc, &s);
  if (rc) return rc;
  if ((rc = check_ptrs({stage_k, stage_v, page_table, host_k, host_v}))) return rc;
  (void)hipGetLastError();
  return launched(oomb::launch_stage_copy(s, host_k, host_v, const_cast<void*>(stage_k), const_cast<void*>(stage_v),
                                          page_table, nullptr, oomb::kStageChunk, true, s.n_slots, 0, s.n,
                                          (hipStream_t)stream));
}

OOMB_API int oomb_stage_flush_grads(const oomb_desc* desc, float* stage_dk, float* stage_dv,
                                    const int32_t* page_table, const int32_t* sel, float* host_dk, float* host_dv,
                                    void* stream) {
  oomb::Shape s;
  int rc = validate(desc, &s);
  if (rc) return rc;
  if ((rc = check_ptrs({stage_dk, stage_dv, page_table, host_dk, host_dv}))) return rc;
  if (s.keff > 0 && (rc = check_ptrs({sel}))) return rc;
  (void)hipGetLastError();
  return launched(
      oomb::launch_grad_flush(s, stage_dk, stage_dv, host_dk, host_dv, page_table, sel, (hipStream_t)stream));
}

OOMB_API int oomb_stage_grads_out(const oomb_desc* desc, float* stage_dk, float* stage_dv, float* out_dk,
                                  float* out_dv, void* stream) {
  oomb::Shape s;
  int rc = validate(desc, &s);
  if (rc) return rc;
  if ((rc = check_ptrs({stage_dk, stage_dv, out_dk, out_dv}))) return rc;
  (void)hipGetLastError();
  return launched(oomb::launch_grads_out(s, stage_dk, stage_dv, out_dk, out_dv, (hipStream_t)stream));
}

OOMB_API int oomb_host_accumulate_grads(const oomb_desc* desc, const float* delta_dk, const float* delta_dv,
                                        const int32_t* page_table, const int32_t* sel, float* host_dk,
                                        float* host_dv, int32_t n_threads) {
  oomb::Shape s;
  int rc = validate(desc, &s);
  if (rc) return rc;
  if (!delta_dk || !delta_dv || !page_table || !host_dk || !host_dv) return OOMB_ERR_NULL_PTR;
  if (s.keff > 0 && !sel) return OOMB_ERR_NULL_PTR;
  if (n_threads < 0 || n_threads > 256) return OOMB_ERR_BAD_SHAPE;
  return oomb::host_accumulate_grads(s, delta_dk, delta_dv, page_table, sel, host_dk, host_dv, n_threads);
}

OOMB_API size_t oomb_check_workspace_bytes(const oomb_desc* desc) {
  oomb::Shape s;
  if (validate(desc, &s)) return 0;
  return (size_t)s.n_slots * 4;
}

OOMB_API int oomb_check_tables(const oomb_desc* desc, const int32_t* page_table, const int32_t* sel,
                               int32_t* counts, void* workspace, size_t workspace_bytes, void* stream) {
  oomb::Shape s;
  int rc = validate(desc, &s);
  if (rc) return rc;
  if ((rc = check_ptrs({page_table, counts}))) return rc;
  if (s.keff > 0 && (rc = check_ptrs({sel}))) return rc;
  if (!workspace || workspace_bytes < (size_t)s.n_slots * 4) return OOMB_ERR_WORKSPACE;
  if (misaligned(workspace)) return OOMB_ERR_MISALIGNED;
  (void)hipGetLastError();
  return launched(
      oomb::launch_check_tables(s, page_table, sel, counts, (int32_t*)workspace, (hipStream_t)stream));
}

OOMB_API int oomb_probe_mfma_peak(int32_t n_blocks, int32_t iters, float* out, void* stream) {
  if (n_blocks < 1 || n_blocks > 65536 || iters < 1 || iters > (1 << 20)) return OOMB_ERR_BAD_SHAPE;
  int rc = check_ptrs({out});
  if (rc) return rc;
  (void)hipGetLastError();
  return launched(oomb::launch_probe_mfma(n_blocks, iters, out, (hipStream_t)stream));
}

OOMB_API const char* oomb_status_string(int status) {
  switch (status) {
    case OOMB_OK: return "ok";
    case OOMB_ERR_NULL_PTR: return "a required pointer is NULL";
    case OOMB_ERR_BAD_SHAPE: return "inconsistent sizes in the descriptor or arguments";
    case OOMB_ERR_UNSUPPORTED: return "shape not supported by the built kernels";
    case OOMB_ERR_BAD_DTYPE: return "dtype is not an oomb_dtype";
    case OOMB_ERR_MISALIGNED: return "a device pointer is not 16-byte aligned";
    case OOMB_ERR_WORKSPACE: return "workspace missing or too small";
    case OOMB_ERR_LAUNCH: return "the HIP runtime rejected a kernel launch";
    case OOMB_ERR_NOT_MAPPED: return "host memory that the device cannot address";
    case OOMB_ERR_SCRATCH_LIMIT: return "the shape needs more scratch than the allocation-free entry point holds";
    default: return "unknown status";
  }
}

OOMB_API int oomb_abi_version(void) { return OOMB_ABI_VERSION; }

OOMB_API int oomb_trace_events(void* const* events, int capacity) {
  if (capacity < 0 || (events && capacity == 0)) return OOMB_ERR_BAD_SHAPE;
  oomb::TraceState& t = oomb::trace_state();
  t.events = events;
  t.capacity = events ? capacity : 0;
  t.count = 0;
  t.error = 0;
  return OOMB_OK;
}

OOMB_API int oomb_trace_only(const char* kernel) {
  oomb::TraceState& t = oomb::trace_state();
  if (!kernel) {
    t.only[0] = 0;
    return OOMB_OK;
  }
  const size_t n = strlen(kernel);
  if (n == 0 || n >= sizeof(t.only)) return OOMB_ERR_BAD_SHAPE;
  memcpy(t.only, kernel, n + 1);
  return OOMB_OK;
}

OOMB_API int oomb_trace_count(void) {
  const oomb::TraceState& t = oomb::trace_state();
  return t.error ? -t.error : t.count;
}

OOMB_API const char* oomb_trace_kernel(int i) {
  const oomb::TraceState& t = oomb::trace_state();
  return (i >= 0 && i < t.count) ? t.names[i] : nullptr;
}
