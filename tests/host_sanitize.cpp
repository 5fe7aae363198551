// host_sanitize.cpp -- drives the host-only code of the library
// (paged_sparse_attention_amd/csrc/host.cpp: descriptor validation and the
// threaded host-side gradient add) so that tests/test_sanitize.py can build it
// with g++ under AddressSanitizer + UndefinedBehaviorSanitizer, and under
// ThreadSanitizer.  TEST INFRASTRUCTURE: no GPU, no HIP.
//
// 1. validate_desc on a table of descriptors, each with the status it must
//    return (and the resolved shape for the valid ones).
// 2. host_accumulate_grads against a plain single-threaded loop written here,
//    for 0 .. 300 threads, with out-of-range selection and page-table entries
//    that must be skipped; every element is one fp32 add, so the pools must be
//    bitwise equal.
// Exit status 0 when every check holds; prints one line per section.
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "shape.h"

using oomb::Shape;

static int failures = 0;
#define CHECK(c)                                                      \
  do {                                                                \
    if (!(c)) {                                                       \
      fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); \
      ++failures;                                                     \
    }                                                                 \
  } while (0)

static oomb_desc good() {
  oomb_desc d;
  memset(&d, 0, sizeof d);
  d.n_q_heads = 28;
  d.n_kv_heads = 4;
  d.head_dim = 128;
  d.page_size = 128;
  d.chunk_len = 4096;
  d.n_prior_pages = 2048;
  d.top_k = 64;
  d.n_slots = 2048 + 32;
  d.rep_capacity = 2048 + 32;
  d.dtype = OOMB_BF16;
  d.softmax_scale = 0.f;
  return d;
}

static void validation() {
  Shape s;
  CHECK(oomb::validate_desc(nullptr, &s) == OOMB_ERR_NULL_PTR);
  oomb_desc d = good();
  CHECK(oomb::validate_desc(&d, nullptr) == OOMB_ERR_NULL_PTR);
  CHECK(oomb::validate_desc(&d, &s) == OOMB_OK);
  CHECK(s.hq == 28 && s.hkv == 4 && s.d == 128 && s.ps == 128 && s.ps_log2 == 7 && s.c == 4096);
  CHECK(s.n == 2048 && s.keff == 64 && s.n_slots == 2080 && s.rep_cap == 2080 && s.bf16);
  CHECK(fabsf(s.scale - 1.0f / sqrtf(128.f)) < 1e-7f);
  d.top_k = 5000;  // K >= N: every prior page
  CHECK(oomb::validate_desc(&d, &s) == OOMB_OK && s.keff == 2048);
  d.softmax_scale = 0.25f;
  CHECK(oomb::validate_desc(&d, &s) == OOMB_OK && s.scale == 0.25f);

  struct Case {
    void (*edit)(oomb_desc&);
    int want;
  };
  const Case cases[] = {
      {[](oomb_desc& d) { d.dtype = (oomb_dtype)7; }, OOMB_ERR_BAD_DTYPE},
      {[](oomb_desc& d) { d.n_q_heads = 30; }, OOMB_ERR_BAD_SHAPE},   // Hq % Hkv != 0
      {[](oomb_desc& d) { d.n_kv_heads = 0; }, OOMB_ERR_BAD_SHAPE},
      {[](oomb_desc& d) { d.head_dim = -128; }, OOMB_ERR_BAD_SHAPE},
      {[](oomb_desc& d) { d.chunk_len = 4000; }, OOMB_ERR_BAD_SHAPE},  // C % ps != 0
      {[](oomb_desc& d) { d.n_prior_pages = -1; }, OOMB_ERR_BAD_SHAPE},
      {[](oomb_desc& d) { d.top_k = -1; }, OOMB_ERR_BAD_SHAPE},
      {[](oomb_desc& d) { d.n_slots = 2079; }, OOMB_ERR_BAD_SHAPE},    // fewer slots than pages
      {[](oomb_desc& d) { d.rep_capacity = 100; }, OOMB_ERR_BAD_SHAPE},
      {[](oomb_desc& d) { d.softmax_scale = -1.f; }, OOMB_ERR_BAD_SHAPE},
      {[](oomb_desc& d) { d.softmax_scale = NAN; }, OOMB_ERR_BAD_SHAPE},
      {[](oomb_desc& d) { d.softmax_scale = INFINITY; }, OOMB_ERR_BAD_SHAPE},
      {[](oomb_desc& d) { d.head_dim = 96; }, OOMB_ERR_UNSUPPORTED},
      {[](oomb_desc& d) { d.page_size = 8; d.n_slots = d.rep_capacity = 4096; }, OOMB_ERR_UNSUPPORTED},
      {[](oomb_desc& d) { d.page_size = 256; }, OOMB_ERR_UNSUPPORTED},
      {[](oomb_desc& d) { d.page_size = 96; d.chunk_len = 96 * 40; d.n_slots = d.rep_capacity = 4096; },
       OOMB_ERR_UNSUPPORTED},
      {[](oomb_desc& d) { d.n_q_heads = 16; d.n_kv_heads = 16; }, OOMB_ERR_UNSUPPORTED},   // Hkv * D > 1024
      {[](oomb_desc& d) { d.n_q_heads = 2048; d.n_kv_heads = 1; }, OOMB_ERR_UNSUPPORTED},  // G >= 1024
      {[](oomb_desc& d) {  // C * G >= 2^24
         d.chunk_len = 1 << 22;
         d.n_slots = d.rep_capacity = 2048 + (1 << 15);
       }, OOMB_ERR_UNSUPPORTED},
  };
  int n = 0;
  for (const Case& c : cases) {
    oomb_desc e = good();
    c.edit(e);
    const int got = oomb::validate_desc(&e, &s);
    if (got != c.want) fprintf(stderr, "descriptor case %d: status %d, want %d\n", n, got, c.want);
    CHECK(got == c.want);
    ++n;
  }
  printf("validation: %d cases: %s\n", n + 8, failures ? "FAILED" : "ok");
}

// the plain loop the threaded add must reproduce bit for bit
static void reference(const Shape& s, const float* dk, const float* dv, const int32_t* pt, const int32_t* sel,
                      float* hk, float* hv) {
  const int64_t blk = (int64_t)s.ps * s.d;
  const int nsel = s.hkv * s.keff;
  for (int h = 0; h < s.hkv; ++h)
    for (int i = 0; i < s.keff; ++i) {
      const int b = h * s.keff + i, page = sel[b];
      if (page < 0 || page >= s.n || pt[page] < 0 || pt[page] >= s.n_slots) continue;
      const int64_t off = ((int64_t)pt[page] * s.hkv + h) * blk;
      for (int64_t e = 0; e < blk; ++e) {
        hk[off + e] += dk[b * blk + e];
        hv[off + e] += dv[b * blk + e];
      }
    }
  for (int j = 0; j < s.c / s.ps; ++j)
    for (int h = 0; h < s.hkv; ++h) {
      const int b = nsel + j * s.hkv + h, slot = pt[s.n + j];
      if (slot < 0 || slot >= s.n_slots) continue;
      const int64_t off = ((int64_t)slot * s.hkv + h) * blk;
      for (int64_t e = 0; e < blk; ++e) {
        hk[off + e] += dk[b * blk + e];
        hv[off + e] += dv[b * blk + e];
      }
    }
}

static uint64_t rng_state = 0x9e3779b97f4a7c15ull;
static uint32_t next_u32() {
  rng_state ^= rng_state << 13;
  rng_state ^= rng_state >> 7;
  rng_state ^= rng_state << 17;
  return (uint32_t)(rng_state >> 11);
}
static float next_float() { return (float)(next_u32() % 2001) / 1000.f - 1.f; }

static void accumulate(int hkv, int ps, int d, int c, int n, int k, int extra_slots, bool bad_entries) {
  oomb_desc desc = good();
  desc.n_q_heads = 2 * hkv;
  desc.n_kv_heads = hkv;
  desc.head_dim = d;
  desc.page_size = ps;
  desc.chunk_len = c;
  desc.n_prior_pages = n;
  desc.top_k = k;
  desc.n_slots = n + c / ps + extra_slots;
  desc.rep_capacity = n + c / ps;
  Shape s;
  CHECK(oomb::validate_desc(&desc, &s) == OOMB_OK);
  const int pages = n + c / ps;
  std::vector<int32_t> pt(pages), sel((size_t)hkv * (s.keff > 0 ? s.keff : 1));
  std::vector<int32_t> perm(s.n_slots);
  for (int i = 0; i < s.n_slots; ++i) perm[i] = i;
  for (int i = s.n_slots - 1; i > 0; --i) std::swap(perm[i], perm[next_u32() % (i + 1)]);
  for (int i = 0; i < pages; ++i) pt[i] = perm[i];
  for (int h = 0; h < hkv; ++h) {  // distinct pages per head: every (n / keff)-th, shifted by one on odd heads
    for (int i = 0; i < s.keff; ++i) sel[h * s.keff + i] = (int)(((int64_t)i * n) / s.keff + (h % 2)) % n;
  }
  if (bad_entries && s.keff > 1) {
    sel[0] = -3;                         // selection out of range: skipped
    sel[s.keff - 1] = n + 5;
    pt[sel[hkv > 1 ? s.keff : 1]] = s.n_slots + 9;  // page-table entry out of range: skipped
  }
  const int nb = hkv * s.keff + (c / ps) * hkv;
  const int64_t blk = (int64_t)ps * d, pool = (int64_t)s.n_slots * hkv * blk;
  std::vector<float> dk(nb * blk), dv(nb * blk), hk0(pool), hv0(pool);
  for (auto& v : dk) v = next_float();
  for (auto& v : dv) v = next_float();
  for (auto& v : hk0) v = next_float();
  for (auto& v : hv0) v = next_float();
  std::vector<float> wk = hk0, wv = hv0;
  reference(s, dk.data(), dv.data(), pt.data(), sel.data(), wk.data(), wv.data());
  const int threads[] = {0, 1, 2, 3, 7, 16, 300};
  for (int nt : threads) {
    std::vector<float> gk = hk0, gv = hv0;
    const int rc = oomb::host_accumulate_grads(s, dk.data(), dv.data(), pt.data(), sel.data(), gk.data(),
                                               gv.data(), nt);
    CHECK(rc == OOMB_OK);
    CHECK(memcmp(gk.data(), wk.data(), pool * sizeof(float)) == 0);
    CHECK(memcmp(gv.data(), wv.data(), pool * sizeof(float)) == 0);
  }
}

int main() {
  validation();
  const int before = failures;
  accumulate(4, 16, 64, 64, 40, 7, 3, false);
  accumulate(2, 32, 128, 96, 20, 5, 0, true);
  accumulate(1, 16, 64, 16, 9, 0, 2, false);   // K = 0: chunk pages only
  accumulate(3, 16, 64, 32, 12, 50, 1, false); // K >= N: every prior page
  printf("host_accumulate_grads: %s\n", failures == before ? "ok" : "FAILED");
  return failures ? 1 : 0;
}
