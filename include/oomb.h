/* oomb.h -- C ABI of the MI355X (gfx950) paged top-K chunk attention library.
 *
 * One chunk step of chunk-recurrent attention over a paged KV cache, as the
 * page "Out of the Memory Barrier: A Highly Memory Efficient Training System
 * for LLMs with Million-Token Contexts" (OOMB) describes it in its technical
 * summary, section 2 (Methodology):
 *   - "Paged Memory Management": the KV cache and its gradients live in
 *     page-granular buffers (the pools below, addressed through a page table);
 *     gradients are accumulated into them in place, outside any autograd graph,
 *     with no concatenated tensors.
 *   - "Page-level Sparse Attention": in the forward pass a top-K page search
 *     over per-page representative vectors picks the most relevant key pages;
 *     the backward pass reuses that choice.
 *   - "Specialized Kernels": KV-cache operations are kept out of the autograd
 *     graph.
 * A chunk of C query tokens attends causally to itself and to the K selected
 * prior pages of its kv-head.
 *
 * Readings taken where the page is silent (the page gives prose only):
 *   - representative vector of a page = mean of its stored keys, per kv-head;
 *   - page score = (mean query of the chunk over its C tokens and the query
 *     heads of the kv-head's group) . (representative vector); one selection per
 *     (chunk, kv-head); exact score ties go to the lower page index;
 *   - only the N prior pages are candidates; the chunk's own C/ps pages are
 *     always attended, causally (chunk token u is visible to query token t iff
 *     u <= t);
 *   - query head g reads kv-head g / (Hq / Hkv) (contiguous GQA groups);
 *   - softmax scale 1/sqrt(D) unless given; the backward holds the selection
 *     fixed and differentiates with respect to Q, K and V.
 *
 * Conventions for every entry point
 *   - Pointers are DEVICE pointers unless marked host; the caller owns every
 *     buffer.  The library never allocates, frees or synchronises; all work is
 *     enqueued on `stream` (a hipStream_t passed as void*, NULL = the default
 *     stream) and returns before it runs.  Kernel launches are the only work
 *     enqueued (no memset or copy), so a caller may capture whole chunk steps
 *     in a HIP graph; replays produce the same bytes as the eager calls.
 *   - Every device pointer must be 16-byte aligned.
 *   - Element type "T" is the descriptor's dtype (fp32 or bf16); dq, lse, rep,
 *     scores and the gradient pools are always fp32.
 *   - Layouts (row-major):
 *       q, o, dO          T     [C][Hq][D]
 *       k_pool, v_pool    T     [n_slots][Hkv][ps][D]
 *       dk_pool, dv_pool  fp32  [n_slots][Hkv][ps][D]
 *       page_table        int32 [N + C/ps]      logical page -> physical slot;
 *                                               the chunk's tokens are logical
 *                                               pages N .. N + C/ps - 1
 *       rep               fp32  [rep_capacity][Hkv][D]   by logical page
 *       sel               int32 [Hkv][K_eff]    logical pages, ascending,
 *                                               K_eff = min(top_k, N)
 *       lse               fp32  [Hq][C]         natural log, scale included
 *   - Errors: every check on the host descriptor, sizes and pointers runs
 *     before any HIP call; on failure the call returns a negative status,
 *     launches nothing and writes nothing.  Device-resident contents
 *     (page_table, sel) are trusted: entries out of range are undefined
 *     behaviour.  A launch error maps to OOMB_ERR_LAUNCH; faults inside a
 *     kernel surface at the caller's next synchronisation.  No C++ exception
 *     crosses this interface.
 *   - Calls on one stream run in order; calls on different streams that write
 *     the same buffer race.
 */
#ifndef OOMB_H
#define OOMB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define OOMB_ABI_VERSION 2

typedef enum { OOMB_F32 = 0, OOMB_BF16 = 1 } oomb_dtype;

typedef enum {
  OOMB_OK = 0,
  OOMB_ERR_NULL_PTR = -1,    /* a required pointer is NULL */
  OOMB_ERR_BAD_SHAPE = -2,   /* inconsistent sizes (e.g. Hq % Hkv != 0, C % ps != 0) */
  OOMB_ERR_UNSUPPORTED = -3, /* valid but not built (D not in {64,128}, ps not in {16,32,64,128}, ...) */
  OOMB_ERR_BAD_DTYPE = -4,   /* dtype not an oomb_dtype */
  OOMB_ERR_MISALIGNED = -5,  /* a device pointer is not 16-byte aligned */
  OOMB_ERR_WORKSPACE = -6,   /* workspace NULL or smaller than the *_workspace_bytes query */
  OOMB_ERR_LAUNCH = -7,      /* the HIP runtime rejected a launch */
  OOMB_ERR_NOT_MAPPED = -8,  /* host memory the device cannot address (oomb_host_view) */
  OOMB_ERR_SCRATCH_LIMIT = -9 /* the shape needs more scratch than oomb_select_topk_noalloc holds */
} oomb_status;

/* Host-side descriptor of one chunk step. */
typedef struct {
  int32_t n_q_heads;      /* Hq > 0 */
  int32_t n_kv_heads;     /* Hkv > 0, Hq % Hkv == 0, Hkv * D <= 1024 */
  int32_t head_dim;       /* D in {64, 128} */
  int32_t page_size;      /* ps in {16, 32, 64, 128} */
  int32_t chunk_len;      /* C > 0, C % ps == 0, C * Hq < 2^30,
                             C * Hq / Hkv < 2^24, Hq / Hkv < 1024 */
  int32_t n_prior_pages;  /* N >= 0: candidate logical pages 0 .. N-1 */
  int32_t top_k;          /* >= 0; K_eff = min(top_k, N); top_k >= N attends every prior page;
                             K_eff * ps + C < 2^30 */
  int32_t n_slots;        /* physical pages in each pool, >= N + C/ps */
  int32_t rep_capacity;   /* rows of the rep table, >= N + C/ps */
  int32_t dtype;          /* oomb_dtype of q, k/v pools, o, dO */
  float softmax_scale;    /* > 0, or 0 for 1/sqrt(D) */
} oomb_desc;

/* Representative-vector update (OOMB, section 2, "Page-level Sparse Attention":
 * pages are ranked by representative vectors; reading: the mean of the page's
 * keys).  For i < n_pages and every kv-head h:
 *     rep[first_page + i][h][:] = (1/ps) * sum_r k_pool[page_table[first_page + i]][h][r][:]
 * accumulated in fp32.  Needs 0 <= first_page, first_page + n_pages <= N + C/ps
 * and <= rep_capacity.  n_pages == 0 is a no-op.  Other rep rows are untouched. */
int oomb_rep_update(const oomb_desc* desc, const void* k_pool, const int32_t* page_table,
                    int32_t first_page, int32_t n_pages, float* rep, void* stream);

/* Bytes of device workspace oomb_select_topk needs (0 if desc is invalid). */
size_t oomb_select_workspace_bytes(const oomb_desc* desc);

/* Top-K page selection (OOMB, section 2, "Page-level Sparse Attention": a
 * top-K page search over representative vectors, made in the forward pass).
 *   qbar[h]   = mean of q[t][g] over t < C and the heads g of group h (fp32)
 *   score[h][n] = qbar[h] . rep[n][h]                    for n < N
 *   sel[h]    = the K_eff pages of highest score, exact ties to the lower page,
 *               written in ascending page order; top_k >= N gives 0..N-1.
 * scores_out (fp32 [Hkv][N]) receives the scores when not NULL.
 * Deterministic: the only atomics are integer adds into LDS histograms (their
 * order cannot change a count), and every floating-point sum has a fixed
 * order, so repeated calls give identical bits. */
int oomb_select_topk(const oomb_desc* desc, const void* q, const float* rep, int32_t* sel,
                     float* scores_out, void* workspace, size_t workspace_bytes, void* stream);

/* oomb_select_topk without a workspace, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation.  Same arguments, results and determinism as
 * oomb_select_topk (the same kernels); the workspace is instead a scratch
 * array that the library holds on each device it runs on, of
 * OOMB_NOALLOC_SCRATCH_BYTES (4 MiB), resident until the process ends.  No
 * device memory is allocated or freed by the call.
 * Every call on one device uses that device's one scratch array: calls that
 * can overlap on one device (unordered streams, several host threads) race
 * and must be ordered by the caller.  The scratch holds the previous call's
 * partial sums and scores; each call overwrites what it reads, so nothing
 * needs clearing.
 * Errors: the checks of oomb_select_topk, then OOMB_ERR_SCRATCH_LIMIT when
 * oomb_select_workspace_bytes(desc) exceeds the scratch (Hkv * N up to about
 * 917,000 at Hkv * D = 512, 785,000 at Hkv * D = 1024), all before any HIP
 * call;
 * OOMB_ERR_LAUNCH if the scratch's address cannot be obtained on the current
 * device or a launch fails. */
#define OOMB_NOALLOC_SCRATCH_BYTES (4u << 20)
int oomb_select_topk_noalloc(const oomb_desc* desc, const void* q, const float* rep, int32_t* sel,
                             float* scores_out, void* stream);

/* Fused forward (OOMB, section 2: attention over the selected pages plus the
 * local chunk).  For chunk token t and query head g, h = g / (Hq/Hkv), the key
 * set J is every token of the pages sel[h][:] and chunk tokens u <= t:
 *   s_j = scale * q[t][g] . k_j,  lse[g][t] = ln sum_j exp(s_j),
 *   o[t][g] = sum_j exp(s_j - lse[g][t]) v_j.
 * bf16: q.k and p.v on bf16 MFMA with fp32 accumulation; p rounded to bf16.
 * o and lse are overwritten. */
int oomb_attn_fwd(const oomb_desc* desc, const void* q, const void* k_pool, const void* v_pool,
                  const int32_t* page_table, const int32_t* sel, void* o, float* lse, void* stream);

/* Bytes of device workspace oomb_attn_bwd needs (0 if desc is invalid). */
size_t oomb_bwd_workspace_bytes(const oomb_desc* desc);

/* Fused backward (OOMB, section 2, "Paged Memory Management": gradients of the
 * KV cache are accumulated in place into paged buffers; "Page-level Sparse
 * Attention": the forward's page choice is reused).  With the same J and the
 * forward's o and lse:
 *   p_j = exp(s_j - lse),  Dt = dO . o,  ds_j = p_j (dO . v_j - Dt)
 *   dq[t][g]            = scale * sum_j ds_j k_j                  (overwritten)
 *   dk_pool[slot(j)]   += scale * sum over rows seeing j of ds_j q
 *   dv_pool[slot(j)]   += sum over rows seeing j of p_j dO
 * Only the slots of the selected pages and of the chunk's pages change; every
 * other byte of the gradient pools is left as it was.  Deterministic (no
 * atomics).  workspace: oomb_bwd_workspace_bytes(desc) bytes. */
int oomb_attn_bwd(const oomb_desc* desc, const void* q, const void* k_pool, const void* v_pool,
                  const int32_t* page_table, const int32_t* sel, const void* o, const float* lse,
                  const void* dO, float* dq, float* dk_pool, float* dv_pool, void* workspace,
                  size_t workspace_bytes, void* stream);

/* ---- Checking the device tables -------------------------------------------
 * The calls above trust the contents of page_table and sel (an entry out of
 * range is an out-of-bounds access inside a kernel).  A caller that builds
 * them itself can check them first; this call only reads them, so any
 * contents are safe.  counts (int32 [4], device) receives:
 *   counts[0]  selection entries outside [0, N)
 *   counts[1]  adjacent selection entries of a kv-head not strictly ascending
 *   counts[2]  page-table entries (logical pages 0 .. N + C/ps - 1) outside
 *              [0, n_slots)
 *   counts[3]  page-table entries that repeat an earlier entry's slot (two
 *              logical pages sharing a slot would add their gradients into
 *              one page)
 * All zero means the tables are valid for this descriptor.  workspace:
 * oomb_check_workspace_bytes(desc) bytes (one counter per slot), cleared by
 * the call itself. */
size_t oomb_check_workspace_bytes(const oomb_desc* desc);
int oomb_check_tables(const oomb_desc* desc, const int32_t* page_table, const int32_t* sel, int32_t* counts,
                      void* workspace, size_t workspace_bytes, void* stream);

/* ---- CPU offloading of the KV cache and its gradients -------------------
 * (OOMB, section 2, "Asynchronous CPU Offloading": the KV cache and its
 * gradients, which grow with the context, live in CPU memory and move to and
 * from the GPU asynchronously, overlapped with compute.)
 *
 * HOST POOLS have the device pools' layout, [n_slots][Hkv][ps][D] (T for K/V,
 * fp32 for dK/dV), in pinned host memory that the device addresses; the calls
 * below take the device view of a host buffer (oomb_host_view) where they say
 * "host pool".  page_table maps logical pages to host-pool slots.
 *
 * A chunk step then runs on a device STAGING POOL that holds only what the
 * step touches: n_stage = Hkv*K_eff + C/ps slots of [Hkv][ps][D],
 *   slot h*K_eff + k      kv-head h's block of page sel[h][k] (the other heads'
 *                         blocks of that slot are not used);
 *   slot Hkv*K_eff + j    every kv-head of the chunk's page N + j.
 * The four calls above run on it unchanged with the STAGED descriptor
 * (oomb_stage_desc), the staged selection sel'[h][k] = h*K_eff + k and the
 * identity page table of length n_stage (oomb_stage_tables).  Every kv-head
 * then visits the same keys in the same order as on the full pools, so the
 * forward, dQ and the staged dK/dV blocks are bitwise those of the full-pool
 * call; gradients go back to the host pools with oomb_stage_flush_grads.
 *
 * These calls are asynchronous on `stream` like the others; a copy on one
 * stream overlaps attention on another (each copy kernel occupies only a few
 * compute units).  Selection and page-table entries out of range are skipped
 * (no copy); device pointers must be 16-byte aligned. */
#define OOMB_STAGE_SELECTED 1 /* the selected (kv-head, page) blocks */
#define OOMB_STAGE_CHUNK 2    /* every kv-head of the chunk's own pages */

/* Device view of pinned host memory (hipHostMalloc or torch pin_memory), for
 * the host-pool arguments below (host).  OOMB_ERR_NOT_MAPPED if the device
 * cannot address host_ptr. */
int oomb_host_view(const void* host_ptr, void** device_view);

/* Staged descriptor (host, no HIP call): desc with n_prior_pages = Hkv*K_eff,
 * top_k = K_eff and n_slots = rep_capacity = n_stage. */
int oomb_stage_desc(const oomb_desc* desc, oomb_desc* staged);

/* sel_stage[i] = i for i < Hkv*K_eff (NULL allowed when K_eff = 0) and
 * pt_stage[i] = i for i < n_stage (int32, device). */
int oomb_stage_tables(const oomb_desc* desc, int32_t* sel_stage, int32_t* pt_stage, void* stream);

/* Pools -> staging pool: the parts (OOMB_STAGE_SELECTED and/or
 * OOMB_STAGE_CHUNK) of K and V, from slots page_table[sel[h][k]] and
 * page_table[N + j] of the source pools src_k / src_v ([src_slots][Hkv][ps][D];
 * the device view of the host pools, or device pools such as another staging
 * pool).  Selected blocks are copied only for logical pages in
 * [first_page, first_page + n_pages); pass 0 and N for all of them.  Entries
 * that map outside the src_slots slots are skipped. */
int oomb_stage_gather(const oomb_desc* desc, const void* src_k, const void* src_v, int32_t src_slots,
                      const int32_t* page_table, const int32_t* sel, int32_t parts, int32_t first_page,
                      int32_t n_pages, void* stage_k, void* stage_v, void* stream);

/* Staging pool -> host pools: every kv-head of the chunk's pages N .. N+C/ps-1
 * (the chunk's keys and values once it has run), to host slots page_table[N + j]. */
int oomb_stage_offload_chunk(const oomb_desc* desc, const void* stage_k, const void* stage_v,
                             const int32_t* page_table, void* host_k, void* host_v, void* stream);

/* Gradient flush (fp32): for the selected blocks and the chunk's pages,
 * host_dk[block] += stage_dk[block] and host_dv[block] += stage_dv[block], then
 * those staging blocks are set to zero, ready for the next step's in-place
 * accumulation.  Flushes that may touch the same host blocks must run in order
 * (one stream). */
int oomb_stage_flush_grads(const oomb_desc* desc, float* stage_dk, float* stage_dv,
                           const int32_t* page_table, const int32_t* sel, float* host_dk, float* host_dv,
                           void* stream);

/* Gradients out (fp32): the staged gradient blocks of the step, in the
 * staging layout's block order -- block b < Hkv*K_eff is kv-head b / K_eff's
 * block of slot b, block Hkv*K_eff + j*Hkv + h is kv-head h of the chunk's
 * page j -- are written to out_dk / out_dv as n_blocks = Hkv*K_eff + (C/ps)*Hkv
 * consecutive blocks of ps*D floats (normally the device view of pinned host
 * buffers), and those staged blocks are then set to zero.  With
 * oomb_host_accumulate_grads this replaces oomb_stage_flush_grads: the link
 * carries the gradients one way instead of there and back. */
int oomb_stage_grads_out(const oomb_desc* desc, float* stage_dk, float* stage_dv, float* out_dk, float* out_dv,
                         void* stream);

/* Host accumulation (host memory only, no HIP call, returns when done): for
 * each block b of oomb_stage_grads_out's order, host_dk[slot][h] += delta_dk[b]
 * and host_dv[slot][h] += delta_dv[b], where (slot, h) is the host-pool block
 * that b stands for: page_table[sel[h][k]] or page_table[N + j].  page_table
 * and sel are HOST arrays.  Entries out of range are skipped.  Runs on
 * n_threads host threads (0 or 1: the calling thread only); each element gets
 * one fp32 add, so the result equals oomb_stage_flush_grads'.  If a helper
 * thread cannot be started, the calling thread adds that share itself: the
 * result is the same, and no exception leaves the call.
 * OOMB_ERR_NULL_PTR, OOMB_ERR_BAD_SHAPE (n_threads outside 0..256) from the
 * checks; otherwise OOMB_OK. */
int oomb_host_accumulate_grads(const oomb_desc* desc, const float* delta_dk, const float* delta_dv,
                               const int32_t* page_table, const int32_t* sel, float* host_dk, float* host_dv,
                               int32_t n_threads);

/* ---- The decoder block around the attention (not steps of the method) ---
 * Qwen2-style block pieces, so that a layer around the path runs chunk by
 * chunk without chains of small framework kernels: RMSNorm, rotary positions
 * (rotate-half pairing), SwiGLU, forward and backward.  All device pointers,
 * row-major, asynchronous on `stream`; fp32 accumulation, bf16 outputs rounded
 * once (RNE).  Host checks run before any HIP call: OOMB_ERR_NULL_PTR,
 * OOMB_ERR_BAD_SHAPE, OOMB_ERR_MISALIGNED (fp32 row buffers 16-byte aligned,
 * bf16 buffers 8-byte aligned), OOMB_ERR_BAD_DTYPE.
 *
 * oomb_rmsnorm_fwd: h[r][:] = x[r][:] * rstd[r] * gain, with rstd[r] =
 *   1/sqrt(mean(x[r][:]^2) + eps).  x fp32 [rows][hidden], gain bf16
 *   [hidden], h bf16 [rows][hidden], rstd fp32 [rows] (out).  hidden % 4 == 0,
 *   hidden <= 8192.
 * oomb_rmsnorm_bwd: dx = rstd*gain*dh - x*rstd^3*mean(gain*dh*x) (+ dres if
 *   not NULL), per row.  dh bf16, dres/dx fp32 [rows][hidden]; rstd from the
 *   forward.
 * oomb_rmsnorm_gain_grad: partial[s][j] = sum over the rows r of segment s of
 *   dh[r][j]*x[r][j]*rstd[r]; the gain gradient is the sum over s of
 *   partial[s][:] (fp32 [segments][hidden], out).  Rows are split into
 *   `segments` equal contiguous ranges.
 * oomb_rotary: out = in with pair (j, j + D/2) of each head of token r turned
 *   by the angle of position first_position + r: cos_table/sin_table fp32
 *   [positions][D/2]; inverse != 0 turns the other way (the transpose, for
 *   gradients).  in [rows][heads][D] of in_dtype (OOMB_F32 or OOMB_BF16), out
 *   bf16 of the same shape (not aliasing in).
 * oomb_swiglu_fwd: out = silu(gate) * up, bf16, n elements (n % 4 == 0).
 * oomb_swiglu_bwd: dgate = dout*up*silu'(gate), dup = dout*silu(gate), bf16. */
int oomb_rmsnorm_fwd(const float* x, const void* gain, int32_t rows, int32_t hidden, float eps, void* h, float* rstd,
                     void* stream);
int oomb_rmsnorm_bwd(const float* x, const void* gain, const float* rstd, const void* dh, const float* dres,
                     int32_t rows, int32_t hidden, float* dx, void* stream);
int oomb_rmsnorm_gain_grad(const float* x, const float* rstd, const void* dh, int32_t rows, int32_t hidden,
                           int32_t segments, float* partial, void* stream);
int oomb_rotary(const void* in, int32_t in_dtype, void* out, const float* cos_table, const float* sin_table,
                int32_t rows, int32_t heads, int32_t head_dim, int32_t first_position, int32_t inverse, void* stream);
int oomb_swiglu_fwd(const void* gate, const void* up, void* out, int64_t n, void* stream);
int oomb_swiglu_bwd(const void* gate, const void* up, const void* dout, void* dgate, void* dup, int64_t n,
                    void* stream);

/* ---- Measurement helper (not a step of the attention path) --------------
 * Sustained bf16 MFMA rate of the device: launches n_blocks workgroups of 4
 * waves on `stream`; every wave issues 4 * iters v_mfma_f32_32x32x16_bf16
 * (32768 flop each) on register operands, in four independent accumulation
 * chains, and writes one float, out[wave] = 4 * iters exactly (a check that
 * the work ran), to out[n_blocks * 4] (device, caller-owned).  Time it with
 * events on `stream`: flop = n_blocks * 4 * 4 * iters * 32768.  Returns
 * OOMB_ERR_BAD_SHAPE unless 1 <= n_blocks <= 65536 and 1 <= iters <= 2^20,
 * OOMB_ERR_NULL_PTR / OOMB_ERR_MISALIGNED for `out`, before any HIP call. */
int oomb_probe_mfma_peak(int32_t n_blocks, int32_t iters, float* out, void* stream);

/* Static text for a status code (host). */
const char* oomb_status_string(int status);

/* OOMB_ABI_VERSION of the built library. */
int oomb_abi_version(void);

/* Kernel tracing, for profiling (host).  `events` holds `capacity` hipEvent_t
 * handles that the caller created; while set, the i-th kernel launched by the
 * entry points above (counting from this call) records events[2i] on its
 * stream just before it and events[2i+1] just after it, for 2i+1 < capacity;
 * later launches record nothing.  events == NULL switches tracing off.
 * Returns OOMB_ERR_BAD_SHAPE for capacity < 0 or a non-NULL list of capacity 0.
 * Process-wide state: not for concurrent use from several host threads. */
int oomb_trace_events(void* const* events, int capacity);

/* Restrict kernel tracing to the launches of one kernel, named as
 * oomb_trace_kernel reports them (for example "dkdv_kernel"); other launches
 * record no events and take no slots.  NULL lifts the restriction.  The name
 * is copied.  Returns OOMB_ERR_BAD_SHAPE for an empty name or one of 64 bytes
 * or more.  Process-wide, like oomb_trace_events. */
int oomb_trace_only(const char* kernel);

/* Launches recorded since the last oomb_trace_events call, or minus the
 * hipError_t of the first event record that failed. */
int oomb_trace_count(void);

/* Static name of the kernel of recorded launch i, or NULL if i is out of range. */
const char* oomb_trace_kernel(int i);

#ifdef __cplusplus
}
#endif
#endif /* OOMB_H */
