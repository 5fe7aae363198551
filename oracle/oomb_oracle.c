/* oomb_oracle.c -- plain fp64 CPU oracle for paged top-K chunk attention.
 *
 * TEST INFRASTRUCTURE, NOT PRODUCT CODE: only the test suite, the smoke check
 * and the CPU-baseline leg of the benchmark may load or run it.  It shares no
 * code with the HIP library.
 *
 * Source of the method: page "Out of the Memory Barrier: A Highly Memory
 * Efficient Training System for LLMs with Million-Token Contexts" (OOMB),
 * technical summary, section 2 (Methodology):
 *   - "Paged Memory Management": the KV cache and its gradients are held in
 *     page-granular buffers and gradients are accumulated in place, with no
 *     concatenated tensors and outside the autograd graph.
 *   - "Page-level Sparse Attention": a top-K page search over representative
 *     vectors picks the most relevant key pages in the forward pass; the same
 *     pages are reused in the backward pass.
 * The pages print no formula.  The readings taken here, each repeated where it
 * is used:
 *   (a) the representative vector of a page is the mean of its stored keys,
 *       per kv-head;
 *   (b) a page's score is the dot product of that vector with the mean query of
 *       the chunk (over all chunk tokens and all query heads of the kv-head's
 *       group); one selection per (chunk, kv-head);
 *   (c) only the n prior pages are candidates; the chunk's own tokens are always
 *       attended, causally (token u is visible to query t iff u <= t);
 *   (d) exact score ties go to the lower page index; the selection is written
 *       in ascending page order;
 *   (e) query head g reads kv-head g / (Hq/Hkv);
 *   (f) softmax over scale * q.k with scale 1/sqrt(D) unless given; LSE is the
 *       natural log of the softmax denominator, scale included;
 *   (g) the backward treats the selection as a constant and differentiates
 *       O with respect to Q, K and V only.
 * Arithmetic is fp64 throughout; inputs are the stored (bf16/fp32/fp64) values
 * widened exactly.  Parallel loops (OpenMP) only split independent rows or keys.
 */
#include "oomb_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int ora_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

static double widen(const void* base, int32_t dtype, int64_t i) {
  if (dtype == ORA_F64) return ((const double*)base)[i];
  if (dtype == ORA_F32) return (double)((const float*)base)[i];
  /* bf16: the upper 16 bits of an IEEE binary32 */
  uint32_t bits = (uint32_t)((const uint16_t*)base)[i] << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

static double softmax_scale(const ora_shape* s) {
  return s->scale > 0.0 ? s->scale : 1.0 / sqrt((double)s->d);
}

int32_t ora_keff(const ora_shape* s) {
  if (s->k <= 0) return 0;
  return s->k < s->n ? s->k : s->n;
}

int64_t ora_nkeys(const ora_shape* s) {
  return (int64_t)ora_keff(s) * s->ps + s->c;
}

/* Element offset of (slot, kv-head h, row r, dim 0) in a pool. */
static int64_t pool_offset(const ora_shape* s, int64_t slot, int32_t h, int32_t r) {
  return ((slot * s->hkv + h) * s->ps + r) * (int64_t)s->d;
}

int64_t ora_key_offset(const ora_shape* s, const int32_t* page_table, const int32_t* sel,
                       int32_t h, int64_t jj) {
  const int32_t keff = ora_keff(s);
  const int64_t n_prior_keys = (int64_t)keff * s->ps;
  int64_t page;
  int32_t row;
  if (jj < n_prior_keys) {                 /* a token of a selected prior page */
    page = sel[(int64_t)h * keff + jj / s->ps];
    row = (int32_t)(jj % s->ps);
  } else {                                 /* chunk token u lives in page n + u / ps */
    const int64_t u = jj - n_prior_keys;
    page = s->n + u / s->ps;
    row = (int32_t)(u % s->ps);
  }
  return pool_offset(s, page_table[page], h, row);
}

/* Reading (a): rep = mean of the page's ps stored keys, per kv-head. */
void ora_rep(const ora_shape* s, const void* k_pool, const int32_t* page_table,
             int32_t first, int32_t count, double* rep) {
  const int32_t D = s->d;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < count; ++i) {
    const int64_t slot = page_table[first + i];
    for (int32_t h = 0; h < s->hkv; ++h) {
      double* out = rep + (i * s->hkv + h) * D;
      for (int32_t x = 0; x < D; ++x) out[x] = 0.0;
      for (int32_t r = 0; r < s->ps; ++r) {
        const int64_t off = pool_offset(s, slot, h, r);
        for (int32_t x = 0; x < D; ++x) out[x] += widen(k_pool, s->dtype, off + x);
      }
      for (int32_t x = 0; x < D; ++x) out[x] /= (double)s->ps;
    }
  }
}

/* Reading (b): the chunk-mean query of kv-head h, over all C tokens and the
 * G = Hq/Hkv query heads g with g / G == h (reading (e)). */
void ora_qmean(const ora_shape* s, const void* q, double* qbar) {
  const int32_t D = s->d, G = s->hq / s->hkv;
  for (int32_t h = 0; h < s->hkv; ++h) {
    double* out = qbar + (int64_t)h * D;
    for (int32_t x = 0; x < D; ++x) out[x] = 0.0;
    for (int32_t t = 0; t < s->c; ++t)
      for (int32_t g = h * G; g < (h + 1) * G; ++g) {
        const int64_t off = ((int64_t)t * s->hq + g) * D;
        for (int32_t x = 0; x < D; ++x) out[x] += widen(q, s->dtype, off + x);
      }
    for (int32_t x = 0; x < D; ++x) out[x] /= (double)s->c * (double)G;
  }
}

/* Reading (b): score = plain dot product of the chunk-mean query and the
 * page's representative vector (no scale, no normalisation). */
void ora_scores(const ora_shape* s, const double* qbar, const double* rep, double* scores) {
  const int32_t D = s->d;
  for (int32_t h = 0; h < s->hkv; ++h)
    for (int32_t n = 0; n < s->n; ++n) {
      const double* a = qbar + (int64_t)h * D;
      const double* b = rep + ((int64_t)n * s->hkv + h) * D;
      double acc = 0.0;
      for (int32_t x = 0; x < D; ++x) acc += a[x] * b[x];
      scores[(int64_t)h * s->n + n] = acc;
    }
}

/* Order used by the top-K: higher score first, then lower page index
 * (reading (d)). */
typedef struct { double score; int32_t page; } ranked;

static int by_rank(const void* pa, const void* pb) {
  const ranked* a = (const ranked*)pa;
  const ranked* b = (const ranked*)pb;
  if (a->score > b->score) return -1;
  if (a->score < b->score) return 1;
  return (a->page > b->page) - (a->page < b->page);
}

static int by_int(const void* pa, const void* pb) {
  const int32_t a = *(const int32_t*)pa, b = *(const int32_t*)pb;
  return (a > b) - (a < b);
}

/* Top-K page search: sort every prior page by rank, keep the first K_eff,
 * write them in ascending page order. */
int32_t ora_select(const ora_shape* s, const double* scores, int32_t* sel) {
  const int32_t keff = ora_keff(s);
  ranked* all = (ranked*)malloc(sizeof(ranked) * (size_t)(s->n > 0 ? s->n : 1));
  for (int32_t h = 0; h < s->hkv; ++h) {
    for (int32_t n = 0; n < s->n; ++n) {
      all[n].score = scores[(int64_t)h * s->n + n];
      all[n].page = n;
    }
    qsort(all, (size_t)s->n, sizeof(ranked), by_rank);
    int32_t* out = sel + (int64_t)h * keff;
    for (int32_t i = 0; i < keff; ++i) out[i] = all[i].page;
    qsort(out, (size_t)keff, sizeof(int32_t), by_int);
  }
  free(all);
  return keff;
}

/* The key list J(h) widened to fp64: kk[jj][:] and vv[jj][:]. */
typedef struct { double* k; double* v; int64_t nkeys; } keyset;

static keyset gather_keys(const ora_shape* s, const void* k_pool, const void* v_pool,
                          const int32_t* page_table, const int32_t* sel, int32_t h) {
  keyset ks;
  ks.nkeys = ora_nkeys(s);
  const int32_t D = s->d;
  ks.k = (double*)malloc(sizeof(double) * (size_t)(ks.nkeys * D + 1));
  ks.v = (double*)malloc(sizeof(double) * (size_t)(ks.nkeys * D + 1));
#pragma omp parallel for schedule(static)
  for (int64_t jj = 0; jj < ks.nkeys; ++jj) {
    const int64_t off = ora_key_offset(s, page_table, sel, h, jj);
    for (int32_t x = 0; x < D; ++x) {
      ks.k[jj * D + x] = widen(k_pool, s->dtype, off + x);
      ks.v[jj * D + x] = widen(v_pool, s->dtype, off + x);
    }
  }
  return ks;
}

static void free_keys(keyset* ks) {
  free(ks->k);
  free(ks->v);
}

/* Keys of J(h) visible to chunk token t: all K_eff*ps prior keys, then chunk
 * tokens u = 0..t (reading (c)). */
static int64_t visible_keys(const ora_shape* s, int32_t t) {
  return (int64_t)ora_keff(s) * s->ps + t + 1;
}

static double dot(const double* a, const double* b, int32_t n) {
  double acc = 0.0;
  for (int32_t x = 0; x < n; ++x) acc += a[x] * b[x];
  return acc;
}

/* Softmax attention of one query row over its visible keys, exactly as
 * defined: s_j = scale q.k_j, m = max s, LSE = m + ln sum exp(s_j - m),
 * p_j = exp(s_j - LSE), o = sum p_j v_j.  sbuf holds nvis scores. */
static void attend_row(const ora_shape* s, const keyset* ks, const double* qrow, int64_t nvis,
                       double* sbuf, double* o, double* lse) {
  const int32_t D = s->d;
  const double sc = softmax_scale(s);
  double m = -INFINITY;
  for (int64_t j = 0; j < nvis; ++j) {
    sbuf[j] = sc * dot(qrow, ks->k + j * D, D);
    if (sbuf[j] > m) m = sbuf[j];
  }
  double denom = 0.0;
  for (int64_t j = 0; j < nvis; ++j) denom += exp(sbuf[j] - m);
  const double L = m + log(denom);
  for (int32_t x = 0; x < D; ++x) o[x] = 0.0;
  for (int64_t j = 0; j < nvis; ++j) {
    const double p = exp(sbuf[j] - L);
    for (int32_t x = 0; x < D; ++x) o[x] += p * ks->v[j * D + x];
  }
  *lse = L;
}

static void load_row(const ora_shape* s, const void* src, int64_t row, double* out) {
  const int64_t off = row * s->d;
  for (int32_t x = 0; x < s->d; ++x) out[x] = widen(src, s->dtype, off + x);
}

void ora_fwd(const ora_shape* s, const void* q, const void* k_pool, const void* v_pool,
             const int32_t* page_table, const int32_t* sel,
             int64_t nrows, const int64_t* rows, double* o, double* lse) {
  const int32_t D = s->d, G = s->hq / s->hkv;
  for (int32_t h = 0; h < s->hkv; ++h) {
    keyset ks = gather_keys(s, k_pool, v_pool, page_table, sel, h);
#pragma omp parallel
    {
      double* sbuf = (double*)malloc(sizeof(double) * (size_t)ks.nkeys);
      double* qrow = (double*)malloc(sizeof(double) * (size_t)D);
#pragma omp for schedule(dynamic, 16)
      for (int64_t i = 0; i < nrows; ++i) {
        const int64_t row = rows[i];
        const int32_t t = (int32_t)(row / s->hq), g = (int32_t)(row % s->hq);
        if (g / G != h) continue;                        /* reading (e) */
        load_row(s, q, row, qrow);
        attend_row(s, &ks, qrow, visible_keys(s, t), sbuf, o + i * D, lse + i);
      }
      free(sbuf);
      free(qrow);
    }
    free_keys(&ks);
  }
}

/* Backward of o = softmax(scale q K^T) V for the listed rows, selection held
 * fixed (reading (g)):
 *   Dt = dO . o,  dp_j = dO . v_j,  ds_j = p_j (dp_j - Dt)
 *   dq = scale sum_j ds_j k_j
 *   dk_j += scale ds_j q,  dv_j += p_j dO   (summed over the rows that see key j)
 * Pass 1 walks rows (forward, Dt, dq); pass 2 walks keys and sums over rows, so
 * no two threads ever write the same output. */
void ora_bwd(const ora_shape* s, const void* q, const void* k_pool, const void* v_pool,
             const int32_t* page_table, const int32_t* sel, const void* dout,
             int64_t nrows, const int64_t* rows, double* dq, double* dk, double* dv) {
  const int32_t D = s->d, G = s->hq / s->hkv;
  const double sc = softmax_scale(s);
  const int64_t nkeys = ora_nkeys(s);
  double* lse = (double*)malloc(sizeof(double) * (size_t)(nrows + 1));
  double* dt = (double*)malloc(sizeof(double) * (size_t)(nrows + 1));
  if (dk) memset(dk, 0, sizeof(double) * (size_t)(s->hkv * nkeys * D));
  if (dv) memset(dv, 0, sizeof(double) * (size_t)(s->hkv * nkeys * D));

  for (int32_t h = 0; h < s->hkv; ++h) {
    keyset ks = gather_keys(s, k_pool, v_pool, page_table, sel, h);
    /* pass 1: per row */
#pragma omp parallel
    {
      double* sbuf = (double*)malloc(sizeof(double) * (size_t)ks.nkeys);
      double* qrow = (double*)malloc(sizeof(double) * (size_t)D);
      double* drow = (double*)malloc(sizeof(double) * (size_t)D);
      double* orow = (double*)malloc(sizeof(double) * (size_t)D);
#pragma omp for schedule(dynamic, 16)
      for (int64_t i = 0; i < nrows; ++i) {
        const int64_t row = rows[i];
        const int32_t t = (int32_t)(row / s->hq), g = (int32_t)(row % s->hq);
        if (g / G != h) continue;
        load_row(s, q, row, qrow);
        load_row(s, dout, row, drow);
        const int64_t nvis = visible_keys(s, t);
        attend_row(s, &ks, qrow, nvis, sbuf, orow, &lse[i]);
        dt[i] = dot(drow, orow, D);
        if (dq) {
          double* out = dq + i * D;
          for (int32_t x = 0; x < D; ++x) out[x] = 0.0;
          for (int64_t j = 0; j < nvis; ++j) {
            const double p = exp(sbuf[j] - lse[i]);
            const double ds = p * (dot(drow, ks.v + j * D, D) - dt[i]);
            for (int32_t x = 0; x < D; ++x) out[x] += sc * ds * ks.k[j * D + x];
          }
        }
      }
      free(sbuf);
      free(qrow);
      free(drow);
      free(orow);
    }
    /* pass 2: per key of J(h) */
    if (dk || dv) {
#pragma omp parallel
      {
        double* qrow = (double*)malloc(sizeof(double) * (size_t)D);
        double* drow = (double*)malloc(sizeof(double) * (size_t)D);
#pragma omp for schedule(dynamic, 4)
        for (int64_t jj = 0; jj < nkeys; ++jj) {
          const double* kj = ks.k + jj * D;
          const double* vj = ks.v + jj * D;
          double* dkj = dk ? dk + ((int64_t)h * nkeys + jj) * D : NULL;
          double* dvj = dv ? dv + ((int64_t)h * nkeys + jj) * D : NULL;
          for (int64_t i = 0; i < nrows; ++i) {
            const int64_t row = rows[i];
            const int32_t t = (int32_t)(row / s->hq), g = (int32_t)(row % s->hq);
            if (g / G != h) continue;
            if (jj >= visible_keys(s, t)) continue;         /* causal: u > t */
            load_row(s, q, row, qrow);
            load_row(s, dout, row, drow);
            const double p = exp(sc * dot(qrow, kj, D) - lse[i]);
            const double ds = p * (dot(drow, vj, D) - dt[i]);
            for (int32_t x = 0; x < D; ++x) {
              if (dkj) dkj[x] += sc * ds * qrow[x];
              if (dvj) dvj[x] += p * drow[x];
            }
          }
        }
        free(qrow);
        free(drow);
      }
    }
    free_keys(&ks);
  }
  free(lse);
  free(dt);
}
