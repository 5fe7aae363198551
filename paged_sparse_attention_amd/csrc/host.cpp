// host.cpp -- host-only parts of the library: descriptor validation for every
// entry point of include/oomb.h, and the host side of the gradient offload
// (the in-place accumulation of a step's dK/dV blocks into host page pools:
// page "Out of the Memory Barrier", technical summary, section 2, "Paged
// Memory Management" and asynchronous CPU offloading).  Plain C++, no HIP.
#include <math.h>

#include <algorithm>
#include <exception>
#include <thread>
#include <vector>

#include "shape.h"

namespace oomb {

namespace {
int log2_exact(int v) {
  for (int b = 0; b < 31; ++b)
    if (v == (1 << b)) return b;
  return -1;
}
}  // namespace

int validate_desc(const oomb_desc* d, Shape* s) {
  if (!d || !s) return OOMB_ERR_NULL_PTR;
  if (d->dtype != OOMB_F32 && d->dtype != OOMB_BF16) return OOMB_ERR_BAD_DTYPE;
  if (d->n_q_heads <= 0 || d->n_kv_heads <= 0 || d->n_q_heads % d->n_kv_heads != 0) return OOMB_ERR_BAD_SHAPE;
  if (d->head_dim <= 0 || d->page_size <= 0 || d->chunk_len <= 0) return OOMB_ERR_BAD_SHAPE;
  if (d->n_prior_pages < 0 || d->top_k < 0 || d->n_slots <= 0 || d->rep_capacity < 0) return OOMB_ERR_BAD_SHAPE;
  if (d->chunk_len % d->page_size != 0) return OOMB_ERR_BAD_SHAPE;
  if (!(d->softmax_scale >= 0.f) || !isfinite(d->softmax_scale)) return OOMB_ERR_BAD_SHAPE;
  const int64_t pages_total = (int64_t)d->n_prior_pages + d->chunk_len / d->page_size;
  if (d->n_slots < pages_total || d->rep_capacity < pages_total) return OOMB_ERR_BAD_SHAPE;
  if (d->head_dim != 64 && d->head_dim != 128) return OOMB_ERR_UNSUPPORTED;
  const int ps_log2 = log2_exact(d->page_size);
  if (ps_log2 < 4 || ps_log2 > 7) return OOMB_ERR_UNSUPPORTED;
  if ((int64_t)d->n_kv_heads * d->head_dim > 1024) return OOMB_ERR_UNSUPPORTED;
  const int64_t G = d->n_q_heads / d->n_kv_heads;
  if (G >= 1024) return OOMB_ERR_UNSUPPORTED;
  const int64_t keff = d->top_k < d->n_prior_pages ? d->top_k : d->n_prior_pages;
  // 32-bit row and key indices inside the kernels
  if ((int64_t)d->chunk_len * G >= (1ll << 24)) return OOMB_ERR_UNSUPPORTED;
  if (keff * d->page_size + d->chunk_len >= (1ll << 30)) return OOMB_ERR_UNSUPPORTED;
  if ((int64_t)d->chunk_len * d->n_q_heads >= (1ll << 30)) return OOMB_ERR_UNSUPPORTED;
  s->hq = d->n_q_heads;
  s->hkv = d->n_kv_heads;
  s->d = d->head_dim;
  s->ps = d->page_size;
  s->ps_log2 = ps_log2;
  s->c = d->chunk_len;
  s->n = d->n_prior_pages;
  s->keff = (int)keff;
  s->n_slots = d->n_slots;
  s->rep_cap = d->rep_capacity;
  s->bf16 = d->dtype == OOMB_BF16;
  s->scale = d->softmax_scale > 0.f ? d->softmax_scale : 1.0f / sqrtf((float)d->head_dim);
  return OOMB_OK;
}

// Within one call every destination block is distinct (a kv-head's selected
// pages are distinct and none is a chunk page), so the threads never write the
// same element.
int host_accumulate_grads(const Shape& s, const float* delta_dk, const float* delta_dv, const int32_t* pt,
                          const int32_t* sel, float* host_dk, float* host_dv, int n_threads) {
  const int nsel = s.hkv * s.keff, n_blocks = nsel + (s.c / s.ps) * s.hkv;
  const int64_t blk = (int64_t)s.ps * s.d;
  auto work = [&](int b0, int b1) noexcept {
    for (int b = b0; b < b1; ++b) {
      int h, logical;
      if (b < nsel) {
        h = b / s.keff;
        logical = sel[b];
        if (logical < 0 || logical >= s.n) continue;
      } else {
        h = (b - nsel) % s.hkv;
        logical = s.n + (b - nsel) / s.hkv;
      }
      const int slot = pt[logical];
      if (slot < 0 || slot >= s.n_slots) continue;
      const int64_t off = ((int64_t)slot * s.hkv + h) * blk;
      const float* dk = delta_dk + (int64_t)b * blk;
      const float* dv = delta_dv + (int64_t)b * blk;
      float* hk = host_dk + off;
      float* hv = host_dv + off;
      for (int64_t i = 0; i < blk; ++i) hk[i] += dk[i];
      for (int64_t i = 0; i < blk; ++i) hv[i] += dv[i];
    }
  };
  const int nt = std::max(1, std::min(n_threads, n_blocks));
  auto range = [&](int t) { return std::make_pair((int)((int64_t)n_blocks * t / nt), (int)((int64_t)n_blocks * (t + 1) / nt)); };
  // Helper threads take shares 1 .. started; a share whose thread could not be
  // started (allocation or thread-creation failure) is done here instead.
  std::vector<std::thread> pool;
  int started = 0;
  try {
    pool.reserve(nt - 1);
    for (int t = 1; t < nt; ++t) {
      const auto r = range(t);
      pool.emplace_back(work, r.first, r.second);
      ++started;
    }
  } catch (...) {
  }
  for (int t = started + 1; t < nt; ++t) {
    const auto r = range(t);
    work(r.first, r.second);
  }
  const auto r0 = range(0);
  work(r0.first, r0.second);
  for (std::thread& th : pool) th.join();  // join() of a started thread does not throw here
  return OOMB_OK;
}

}  // namespace oomb
