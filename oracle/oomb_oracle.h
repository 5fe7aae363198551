/* oomb_oracle.h -- plain fp64 CPU oracle for paged top-K chunk attention.
 *
 * TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the smoke check
 * and the CPU-baseline leg of the benchmark may load or run it.  It shares no
 * code, header, table or helper with the HIP library; the two meet only in the
 * seeded input generator (synth/), which holds none of the method's arithmetic.
 *
 * Method: "Out of the Memory Barrier: A Highly Memory Efficient Training System
 * for LLMs with Million-Token Contexts" (OOMB), technical summary, section 2
 * (Methodology), items "Paged Memory Management" and "Page-level Sparse
 * Attention".  The pages state the method in prose only; every concrete rule the
 * oracle needs beyond that prose is a stated reading, repeated at the function
 * that takes it.
 *
 * Tensor layouts (all row-major, element type given by ora_shape.dtype unless
 * noted; every output is fp64):
 *   q, o, dO        [C][Hq][D]
 *   k_pool, v_pool  [n_slots][Hkv][ps][D]     physical page slots
 *   page_table      [N + C/ps] int32           logical page -> physical slot
 *   rep             [pages][Hkv][D]            indexed by logical page
 *   scores          [Hkv][N]
 *   sel             [Hkv][K_eff] int32         logical page indices, ascending
 * A "row" is one (chunk token t, query head g) pair with id t*Hq + g.
 * The key list of kv-head h is J(h): the tokens of the selected pages, page by
 * page in sel order and row order inside a page (K_eff*ps keys), then the C
 * chunk tokens 0..C-1 (the local causal chunk).  Key index jj runs over J(h).
 */
#ifndef OOMB_ORACLE_H
#define OOMB_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORA_F32 = 0, ORA_BF16 = 1, ORA_F64 = 2 };

typedef struct {
  int32_t hq, hkv;      /* query heads, kv heads; hq % hkv == 0 */
  int32_t d;            /* head dimension */
  int32_t ps;           /* tokens per page */
  int32_t c;            /* chunk length (multiple of ps) */
  int32_t n;            /* prior (candidate) logical pages 0..n-1 */
  int32_t k;            /* top-K; K_eff = min(k, n) */
  int32_t n_slots;      /* physical page slots in the pools */
  int32_t dtype;        /* ORA_F32, ORA_BF16 or ORA_F64: element type of q, pools, dO */
  double scale;         /* softmax scale; <= 0 selects 1/sqrt(d) */
} ora_shape;

/* Host threads the parallel loops use (OpenMP). */
int ora_threads(void);

/* Number of selected pages per kv-head, min(k, n). */
int32_t ora_keff(const ora_shape* s);
/* Keys in J(h): K_eff*ps + C. */
int64_t ora_nkeys(const ora_shape* s);

/* rep[i][h][:] = mean over the ps rows of the keys of logical page first+i. */
void ora_rep(const ora_shape* s, const void* k_pool, const int32_t* page_table,
             int32_t first, int32_t count, double* rep);

/* qbar[h][:] = mean over all chunk tokens and all query heads of group h. */
void ora_qmean(const ora_shape* s, const void* q, double* qbar);

/* scores[h][n] = qbar[h] . rep[n][h] for the n prior pages. */
void ora_scores(const ora_shape* s, const double* qbar, const double* rep, double* scores);

/* sel[h][:] = the K_eff best pages by (score desc, page asc), written ascending.
 * Returns K_eff. */
int32_t ora_select(const ora_shape* s, const double* scores, int32_t* sel);

/* Forward for the listed rows: o[i][:] and lse[i] of row rows[i]. */
void ora_fwd(const ora_shape* s, const void* q, const void* k_pool, const void* v_pool,
             const int32_t* page_table, const int32_t* sel,
             int64_t nrows, const int64_t* rows, double* o, double* lse);

/* Backward driven by the listed rows (their own forward is recomputed here):
 *   dq[i][:]       gradient of row rows[i]
 *   dk[h][jj][:]   sum over the listed rows of their contribution to key jj of J(h)
 *   dv[h][jj][:]   same for V
 * dk / dv are overwritten (zeroed first); either may be NULL to skip it. */
void ora_bwd(const ora_shape* s, const void* q, const void* k_pool, const void* v_pool,
             const int32_t* page_table, const int32_t* sel, const void* dout,
             int64_t nrows, const int64_t* rows, double* dq, double* dk, double* dv);

/* Physical element offset (into k_pool / v_pool) of key jj of J(h), row 0 of D. */
int64_t ora_key_offset(const ora_shape* s, const int32_t* page_table, const int32_t* sel,
                       int32_t h, int64_t jj);

#ifdef __cplusplus
}
#endif
#endif
