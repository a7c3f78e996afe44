/*
 * paged_mqa_logits.h -- C ABI of the paged MQA-logits indexer library
 * (libidx_paged_mqa.so, HIP kernels for gfx950).
 *
 * What is computed.  The DSA indexer scores one query row against every
 * cached c4-position of that row's paged key cache.  The pages describe it as
 * attention scores between the current query and all cached positions, with
 * a ReLU, a per-head weighting and a position-specific scale ("The Dispatch
 * Wire: Connecting a Triton Indexer Kernel to Production Inference",
 * section "The Road to This Message"), the fallback's op chain being a batched
 * QK product, ReLU, weight scaling and a sum over heads (same section).  With
 * H = 64 heads, D = 128 and pages of 64 c4-positions:
 *
 *   L_b          = clamp(seqlens[b], 0, table_width * 64)
 *   out[b][p]    = sum_h w[b][h] * ReLU( s_p * <q[b][h][:], k_p[:]> )   p <  L_b
 *   out[b][p]    = -inf                                                 p >= L_b
 *
 * where position p = 64*j + i lives in physical page g = page_table_b[j] at
 * slot i, k_p is its 128-value key and s_p its scale (1 for bf16 keys).
 * ReLU propagates NaN.  Positions at or past the row's length are -inf
 * ("The Final Gate: Validating a Custom Triton Indexer Kernel Before Production
 * Deployment", section "What the Test Output Reveals").
 *
 * Launch model.  One fixed grid whose shape depends only on the scalar
 * arguments; a work unit whose pages all start at or past L_b writes -inf and
 * exits without reading the page table or the keys, so the cost follows the
 * actual lengths while the grid and the output shape stay fixed and the call
 * can be captured into a HIP graph ("The Moment the Context-Length Tax
 * Vanished: Committing the O(actual) Triton Indexer", section "The Commit:
 * Engineering as Narrative").  Pages are read through the page table on the
 * fly; no gathered copy of the cache is ever made (the bf16 prefill failure in
 * "The Dispatch Decision: Wiring a Triton Kernel into Production", section
 * "The Problem That Led Here").
 *
 * Ownership and threading.  Every pointer argument is a DEVICE pointer owned by
 * the caller.  The library holds no state, allocates no memory, never
 * synchronises the host and enqueues its work on `stream` (NULL = the null
 * stream).  Calls are thread-safe; calls that write the same `out` race.
 *
 * Errors.  Every entry point validates its arguments on the host and returns
 * an idx_status; it never aborts, prints or throws.  Nothing is launched when
 * the return value is not IDX_OK.  Device data is never inspected on the host:
 *  - seqlens are clamped to [0, table_width*64] on the device;
 *  - a page-table entry that is read (its page holds a live position) and lies
 *    outside [0, num_pages) is never dereferenced: that page's live positions
 *    are written as NaN (its masked positions still get -inf);
 *  - page-table entries of slots past a row's live pages are never read and
 *    may hold anything (e.g. -1 padding).
 */
#ifndef IDX_PAGED_MQA_LOGITS_H
#define IDX_PAGED_MQA_LOGITS_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Version of this ABI; bumped on any incompatible change. */
#define IDX_ABI_VERSION 1

/* Fixed shape of the indexer: heads, head dimension, positions per page. */
#define IDX_NUM_HEADS 64
#define IDX_HEAD_DIM 128
#define IDX_PAGE_POSITIONS 64

typedef enum {
  IDX_OK = 0,
  IDX_ERR_NULL = -1,        /* a required pointer is NULL (or kscale given for bf16) */
  IDX_ERR_UNSUPPORTED = -2, /* num_heads != 64 or head_dim != 128 */
  IDX_ERR_SHAPE = -3,       /* negative or oversized dimension, stride too small */
  IDX_ERR_ALIGN = -4,       /* pointer or stride misaligned */
  IDX_ERR_LAUNCH = -5       /* the HIP launch reported an error */
} idx_status;

/*
 * fp8-key variant.  Keys are OCP e4m3fn bytes with one fp32 scale per
 * position; the cache block of the pages holds 64 positions x 128 e4m3 values
 * followed by 64 fp32 scales, 8,448 bytes in all ("The Dispatch Wire ...",
 * section "The Reasoning and Decision-Making"; "The Final Gate ...", section
 * "Assumptions and Knowledge Required").
 *
 *   q          bf16 [rows][64][128], contiguous, 16-byte aligned.
 *   kv_pages   key pool.  Page g starts at (const char*)kv_pages +
 *              g*kv_page_stride and holds [64][128] e4m3fn bytes, position
 *              major.  16-byte aligned.
 *   kscale     scale of slot i of page g is the fp32 at
 *              (const char*)kscale + g*kscale_page_stride + 4*i.  For the
 *              fused block layout pass kv_pages + 8192 and a stride of 8448.
 *              4-byte aligned.
 *   page_table int32; row b's table is page_table + b*page_table_row_stride,
 *              table_width entries of physical page ids.  A stride of 0 makes
 *              every row share one table (the prefill case: T query tokens of
 *              one request).  4-byte aligned.
 *   seqlens    int32 [rows], valid c4-positions per row.  4-byte aligned.
 *   weights    fp32 [rows][64] per-head weights, 16-byte aligned.
 *   out        fp32 [rows][table_width*64], 16-byte aligned.  Every element is
 *              written (finite, NaN for an invalid page id, or -inf).
 *   rows, table_width       >= 0; 0 returns IDX_OK with no launch.
 *                           table_width <= 16,777,216.
 *   num_heads, head_dim     must be 64 and 128.
 *   num_pages               pages in the pool (bound for page ids), >= 0.
 *   kv_page_stride          bytes, >= 8192, multiple of 16.
 *   kscale_page_stride      bytes, >= 256, multiple of 4.
 *   page_table_row_stride   int32 elements, >= 0.
 *   stream                  HIP stream the kernel is enqueued on.
 */
int idx_paged_mqa_logits_fp8(const void* q, const void* kv_pages, const float* kscale,
                             const int32_t* page_table, const int32_t* seqlens,
                             const float* weights, float* out, int32_t rows, int32_t num_heads,
                             int32_t head_dim, int32_t table_width, int64_t num_pages,
                             int64_t kv_page_stride, int64_t kscale_page_stride,
                             int64_t page_table_row_stride, hipStream_t stream);

/*
 * bf16-key variant: keys stored as bf16, 256 bytes per position and no scale
 * (s_p = 1), the layout of the bf16 indexer store in "The Dispatch Decision:
 * Wiring a Triton Kernel into Production", section "The Problem That Led Here".
 * Same arguments as the fp8 variant except:
 *   kv_pages            page g holds [64][128] bf16; kv_page_stride >= 16384,
 *                       multiple of 16.
 *   kscale              must be NULL (else IDX_ERR_NULL); kscale_page_stride
 *                       is ignored.
 */
int idx_paged_mqa_logits_bf16(const void* q, const void* kv_pages, const float* kscale,
                              const int32_t* page_table, const int32_t* seqlens,
                              const float* weights, float* out, int32_t rows, int32_t num_heads,
                              int32_t head_dim, int32_t table_width, int64_t num_pages,
                              int64_t kv_page_stride, int64_t kscale_page_stride,
                              int64_t page_table_row_stride, hipStream_t stream);

/*
 * Multi-request prefill: the query rows of several requests in one call, each
 * request with its own page table and every row with its own causal length.
 * The pages show a prefill of one request; a batch of several is the reading
 * taken for serving ("The Dispatch Decision: Wiring a Triton Kernel into
 * Production", section "The Problem That Led Here": the prefill path scores
 * the query tokens of a request against its cached keys).
 * Arguments as idx_paged_mqa_logits_fp8 except:
 *   page_table   int32 tables, table t at page_table + t*page_table_row_stride
 *                (table_width entries each).
 *   row_table    int32 [rows], 4-byte aligned: the table (request) of each
 *                row.  Rows of one request should be contiguous: a block of 4
 *                consecutive rows reads each key page once per distinct table
 *                among its rows.  A row whose index lies outside
 *                [0, num_tables) scores NaN at its live positions.
 *   num_tables   >= 0.
 *   seqlens      per row: the positions that row sees (its causal limit).
 * Every output element is written.
 */
int idx_paged_mqa_logits_varlen_fp8(const void* q, const void* kv_pages, const float* kscale,
                                    const int32_t* page_table, const int32_t* row_table,
                                    int32_t num_tables, const int32_t* seqlens, const float* weights,
                                    float* out, int32_t rows, int32_t num_heads, int32_t head_dim,
                                    int32_t table_width, int64_t num_pages, int64_t kv_page_stride,
                                    int64_t kscale_page_stride, int64_t page_table_row_stride,
                                    hipStream_t stream);

/* bf16-key counterpart of idx_paged_mqa_logits_varlen_fp8 (kscale must be NULL). */
int idx_paged_mqa_logits_varlen_bf16(const void* q, const void* kv_pages, const float* kscale,
                                     const int32_t* page_table, const int32_t* row_table,
                                     int32_t num_tables, const int32_t* seqlens, const float* weights,
                                     float* out, int32_t rows, int32_t num_heads, int32_t head_dim,
                                     int32_t table_width, int64_t num_pages, int64_t kv_page_stride,
                                     int64_t kscale_page_stride, int64_t page_table_row_stride,
                                     hipStream_t stream);

/*
 * Top-k over logits rows: the selection the -inf-masked logits feed ("The
 * Final Gate: Validating a Custom Triton Indexer Kernel Before Production
 * Deployment", section "What the Test Output Reveals").  The pages give
 * neither k nor a tie rule; this library's rule:
 *
 *   candidates  positions p < L_b of row b, L_b = clamp(seqlens[b], 0, ncols)
 *   order       larger value first; equal values (+0 equals -0) by lower
 *               position; NaN after every number
 *   result      the first min(k, L_b) candidates of that order, written in
 *               ascending position order to topk_idx[b][0..), then -1 up to k
 *
 *   logits      fp32 rows; row b starts at logits + b*row_stride (elements).
 *               16-byte aligned, row_stride a multiple of 4 and >= ncols.
 *               Only positions p < L_b are read.  May be NULL if ncols == 0.
 *   seqlens     int32 [rows], 4-byte aligned.
 *   rows, ncols, k   >= 0; rows == 0 or k == 0 returns IDX_OK with no launch.
 *   topk_idx    int32 [rows][k], 4-byte aligned.
 *   topk_val    optional (NULL: not written) fp32 [rows][k], 4-byte aligned:
 *               the selected logits, bit for bit, and -inf for padding.
 * One workgroup per row; the result is deterministic.
 */
int idx_topk_logits(const float* logits, int64_t row_stride, const int32_t* seqlens, int32_t rows,
                    int32_t ncols, int32_t k, int32_t* topk_idx, float* topk_val,
                    hipStream_t stream);

/*
 * Logits followed by their top-k, in one call on one stream: the arguments of
 * idx_paged_mqa_logits_fp8 (q ... page_table_row_stride), then k, topk_idx and
 * topk_val as in idx_topk_logits over the logits rows (ncols = row_stride =
 * table_width*64).  `logits` is the caller's buffer [rows][table_width*64]
 * for the intermediate scores.  Unlike idx_paged_mqa_logits_fp8 the -inf
 * stores past each row's live pages are skipped where the kernel can skip
 * them: after the call only positions p < L_b are defined, the rest hold
 * their old contents or -inf.  Errors as both functions; nothing is launched
 * on an error.
 */
int idx_paged_mqa_topk_fp8(const void* q, const void* kv_pages, const float* kscale,
                           const int32_t* page_table, const int32_t* seqlens, const float* weights,
                           float* logits, int32_t rows, int32_t num_heads, int32_t head_dim,
                           int32_t table_width, int64_t num_pages, int64_t kv_page_stride,
                           int64_t kscale_page_stride, int64_t page_table_row_stride, int32_t k,
                           int32_t* topk_idx, float* topk_val, hipStream_t stream);

/* bf16-key counterpart of idx_paged_mqa_topk_fp8 (kscale must be NULL). */
int idx_paged_mqa_topk_bf16(const void* q, const void* kv_pages, const float* kscale,
                            const int32_t* page_table, const int32_t* seqlens, const float* weights,
                            float* logits, int32_t rows, int32_t num_heads, int32_t head_dim,
                            int32_t table_width, int64_t num_pages, int64_t kv_page_stride,
                            int64_t kscale_page_stride, int64_t page_table_row_stride, int32_t k,
                            int32_t* topk_idx, float* topk_val, hipStream_t stream);

/*
 * Paged key store, fp8: the write side of the cache block above.  Each of n
 * keys (128 values) is quantised and written to one slot of the pool.  The
 * pages give the block (64 positions x 128 fp8 values, then 64 fp32 scales;
 * "The Dispatch Wire ...", section "The Reasoning and Decision-Making") and a
 * per-position scale; the quantiser is the amax/448 rule, computed in float32
 * in this order (bit-exact, so every caller gets the same bytes):
 *
 *   scale   = amax > 0 ? amax / 448 : 1        amax = max_d |k_d|
 *   code_d  = e4m3fn(clamp(k_d / scale, -448, 448)), round to nearest even;
 *             a value that rounds to zero keeps its sign (0x80 for -0).
 *
 *   keys        bf16 [n][128], 16-byte aligned.
 *   slots       int64 [n], 8-byte aligned: key t goes to page slots[t] / 64,
 *               position slots[t] % 64.  A slot outside [0, 64*num_pages) --
 *               e.g. -1 for a padding token -- skips the key.  Two keys with
 *               the same slot race.
 *   kv_pages    pool as in idx_paged_mqa_logits_fp8 (codes at page*stride +
 *               128*position), 16-byte aligned; kv_page_stride >= 8192,
 *               multiple of 16.
 *   kscale      scales as in idx_paged_mqa_logits_fp8 (at page*kscale_page_stride
 *               + 4*position), 4-byte aligned; kscale_page_stride >= 256,
 *               multiple of 4.
 *   n, num_pages  >= 0; n == 0 returns IDX_OK with no launch.
 * Keys holding NaN or Inf give unspecified codes.
 */
int idx_store_keys_fp8(const void* keys, const int64_t* slots, int64_t n, void* kv_pages,
                       float* kscale, int64_t num_pages, int64_t kv_page_stride,
                       int64_t kscale_page_stride, hipStream_t stream);

/*
 * Paged key store, bf16: key t is copied to its slot of 16,384-byte bf16 pages
 * (256 bytes per position, the bf16 store of "The Dispatch Decision ...",
 * section "The Problem That Led Here").  Arguments as idx_store_keys_fp8
 * without the scales; kv_page_stride >= 16384, multiple of 16.
 */
int idx_store_keys_bf16(const void* keys, const int64_t* slots, int64_t n, void* kv_pages,
                        int64_t num_pages, int64_t kv_page_stride, hipStream_t stream);

/* Static, human-readable text for an idx_status value (never NULL). */
const char* idx_status_string(int status);

/* IDX_ABI_VERSION of the loaded library. */
int idx_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* IDX_PAGED_MQA_LOGITS_H */
