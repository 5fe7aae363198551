/* sanitize_check.c -- runs the whole oracle chain on small seeded problems so
 * that it can be built with AddressSanitizer and UndefinedBehaviorSanitizer
 * (tests/test_sanitize.py builds and runs it; TEST INFRASTRUCTURE, like the
 * oracle itself).  Inputs come from the seeded generator (synth/synth.c).
 *
 * Per problem: rep of every page, chunk-mean query, scores, selection, the
 * forward of every row and the backward of every row; then two properties that
 * hold for any inputs: every output is finite, and the dK of each kv-head sums
 * to zero over its keys (sum_j ds_j = 0 per row).  Exit status 0 when all hold;
 * the sanitizers abort on the first error they find. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "oomb_oracle.h"

/* synth/synth.c */
void synth_tensor(uint64_t seed, uint32_t stream, int64_t start, int64_t count, double scale, int dtype,
                  void* out);
void synth_pool(uint64_t seed, uint32_t tok_stream, uint32_t off_stream, double off_scale, int32_t n_logical,
                int32_t hkv, int32_t ps, int32_t d, const int32_t* page_table, int32_t n_slots, double fill,
                int dtype, void* pool);
void synth_permutation(uint64_t seed, uint32_t stream, int32_t n, int32_t* out);

static int finite_all(const double* a, int64_t n) {
  for (int64_t i = 0; i < n; ++i)
    if (!isfinite(a[i])) return 0;
  return 1;
}

static int run(ora_shape s, uint64_t seed) {
  const int32_t pages = s.n + s.c / s.ps;
  const size_t eb = s.dtype == ORA_BF16 ? 2 : (s.dtype == ORA_F32 ? 4 : 8);
  const int64_t rows = (int64_t)s.c * s.hq;
  const int64_t pool_elems = (int64_t)s.n_slots * s.hkv * s.ps * s.d;
  int32_t* perm = malloc(sizeof(int32_t) * (size_t)s.n_slots);
  synth_permutation(seed, 6, s.n_slots, perm);  /* first `pages` entries: the page table */
  void* q = malloc(eb * (size_t)(rows * s.d));
  void* dout = malloc(eb * (size_t)(rows * s.d));
  void* kp = malloc(eb * (size_t)pool_elems);
  void* vp = malloc(eb * (size_t)pool_elems);
  synth_tensor(seed, 1, 0, rows * s.d, 1.0, s.dtype, q);
  synth_tensor(seed, 4, 0, rows * s.d, 1.0, s.dtype, dout);
  synth_pool(seed, 2, 5, 0.5, pages, s.hkv, s.ps, s.d, perm, s.n_slots, 64.0, s.dtype, kp);
  synth_pool(seed, 3, 5, 0.0, pages, s.hkv, s.ps, s.d, perm, s.n_slots, 64.0, s.dtype, vp);

  const int32_t keff = ora_keff(&s);
  const int64_t nkeys = ora_nkeys(&s);
  double* rep = malloc(sizeof(double) * (size_t)((int64_t)pages * s.hkv * s.d));
  double* qbar = malloc(sizeof(double) * (size_t)(s.hkv * s.d));
  double* scores = malloc(sizeof(double) * (size_t)((int64_t)s.hkv * (s.n > 0 ? s.n : 1)));
  int32_t* sel = malloc(sizeof(int32_t) * (size_t)(s.hkv * (keff > 0 ? keff : 1)));
  ora_rep(&s, kp, perm, 0, pages, rep);
  ora_qmean(&s, q, qbar);
  ora_scores(&s, qbar, rep, scores);
  if (ora_select(&s, scores, sel) != keff) return 0;

  int64_t* all = malloc(sizeof(int64_t) * (size_t)rows);
  for (int64_t i = 0; i < rows; ++i) all[i] = i;
  double* o = malloc(sizeof(double) * (size_t)(rows * s.d));
  double* lse = malloc(sizeof(double) * (size_t)rows);
  double* dq = malloc(sizeof(double) * (size_t)(rows * s.d));
  double* dk = malloc(sizeof(double) * (size_t)(s.hkv * nkeys * s.d));
  double* dv = malloc(sizeof(double) * (size_t)(s.hkv * nkeys * s.d));
  ora_fwd(&s, q, kp, vp, perm, sel, rows, all, o, lse);
  ora_bwd(&s, q, kp, vp, perm, sel, dout, rows, all, dq, dk, dv);

  int ok = finite_all(rep, (int64_t)pages * s.hkv * s.d) && finite_all(o, rows * s.d) &&
           finite_all(lse, rows) && finite_all(dq, rows * s.d) && finite_all(dk, s.hkv * nkeys * s.d) &&
           finite_all(dv, s.hkv * nkeys * s.d);
  for (int32_t h = 0; ok && h < s.hkv; ++h)
    for (int32_t d = 0; d < s.d; ++d) {
      double sum = 0.0, mag = 0.0;
      for (int64_t j = 0; j < nkeys; ++j) {
        const double x = dk[((int64_t)h * nkeys + j) * s.d + d];
        sum += x;
        mag += fabs(x);
      }
      if (fabs(sum) > 1e-9 * (mag + 1.0)) ok = 0;
    }
  printf("hq %d hkv %d d %d ps %d c %d n %d k %d dtype %d: %s\n", s.hq, s.hkv, s.d, s.ps, s.c, s.n, s.k, s.dtype,
         ok ? "ok" : "FAILED");
  free(perm); free(q); free(dout); free(kp); free(vp); free(rep); free(qbar); free(scores); free(sel);
  free(all); free(o); free(lse); free(dq); free(dk); free(dv);
  return ok;
}

int main(void) {
  const ora_shape shapes[] = {
      {4, 2, 64, 16, 64, 12, 3, 20, ORA_F32, 0.0},   /* GQA, sparse, extra slots */
      {7, 1, 64, 16, 32, 5, 9, 7, ORA_BF16, 0.0},    /* K >= N: dense */
      {2, 2, 128, 32, 64, 0, 4, 2, ORA_F32, 0.3},    /* no prior pages, scale given */
      {4, 2, 64, 16, 48, 6, 0, 9, ORA_BF16, 0.0},    /* K = 0: the chunk only */
  };
  int ok = 1;
  for (unsigned i = 0; i < sizeof(shapes) / sizeof(shapes[0]); ++i) ok &= run(shapes[i], 11 + i);
  return ok ? 0 : 1;
}
