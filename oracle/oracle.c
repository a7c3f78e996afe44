/*
 * oracle.c -- TEST INFRASTRUCTURE ONLY.  A plain, slow CPU definition of the
 * paged MQA-logits indexer, used to check the HIP library.  Nothing in the
 * library links, includes or calls this file; only the tests, the smoke check
 * and the benchmark's CPU-baseline leg load it.
 *
 * Arithmetic is float64 throughout, in a fixed order: for each output the dot
 * product runs over d = 0..127 ascending, then heads h = 0..63 ascending.
 * Parallelism (OpenMP) is only over independent outputs, so it never changes
 * any result.
 *
 * Sources (the pages' titles and sections):
 *  - the computation: a per-head QK score, scaled per position, passed through
 *    ReLU, weighted per head and summed over heads -- "The Dispatch Wire:
 *    Connecting a Triton Indexer Kernel to Production Inference", section
 *    "The Road to This Message", and the fp8-to-bf16 cast / ReLU / weighted
 *    head sum / per-position scale listed in its section "Assumptions and
 *    Risks";
 *  - keys stored per cache block as 64 positions of 128 fp8 values followed
 *    by 64 fp32 scales -- same page, section "The Reasoning and
 *    Decision-Making";
 *  - bf16 keys at 256 bytes per position with no quantisation -- "The Dispatch
 *    Decision: Wiring a Triton Kernel into Production", section "The Problem
 *    That Led Here";
 *  - positions at or past the row's length are -inf -- "The Final Gate:
 *    Validating a Custom Triton Indexer Kernel Before Production Deployment",
 *    section "What the Test Output Reveals".
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *  - fp8 means OCP e4m3fn (bias 7, no infinities, S.1111.111 is NaN, largest
 *    finite 448); the pages only say "fp8";
 *  - ReLU(x) = max(x, 0) with NaN propagated (the fallback's clamp_min);
 *  - the scale multiplies the dot product before the ReLU;
 *  - L = clamp(seqlen, 0, table_width*64);
 *  - a page id that must be read and lies outside [0, num_pages) yields NaN at
 *    that page's live positions.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* OCP 8-bit floating point, E4M3 ("fn": finite, no infinities).
 * sign s, 4-bit exponent e (bias 7), 3-bit mantissa m:
 *   e == 0            : (-1)^s * 2^-6 * (m / 8)        (subnormal)
 *   e == 15 && m == 7 : NaN
 *   otherwise         : (-1)^s * 2^(e-7) * (1 + m / 8)                      */
double oracle_e4m3fn_value(uint32_t code) {
  const uint32_t s = (code >> 7) & 1u, e = (code >> 3) & 15u, m = code & 7u;
  double mag;
  if (e == 15u && m == 7u) return NAN;
  if (e == 0u)
    mag = ldexp((double)m / 8.0, -6);
  else
    mag = ldexp(1.0 + (double)m / 8.0, (int)e - 7);
  return s ? -mag : mag;
}

/* bfloat16: the upper 16 bits of an IEEE binary32. */
double oracle_bf16_value(uint16_t bits) {
  const uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

static double relu(double x) { return isnan(x) ? x : (x > 0.0 ? x : 0.0); }

enum { NH = 64, HD = 128, PG = 64 };

/*
 * Full definition over host buffers laid out exactly as the library's
 * arguments (see the library header).  key_kind 0 = e4m3fn keys with scales,
 * 1 = bf16 keys with s = 1.
 *
 *   q_bits      bf16 bits [rows][64][128]
 *   kv          key pool bytes; page g at kv + g*kv_stride
 *   ks          scale bytes (fp8 only); scale (g, i) at ks + g*ks_stride + 4*i
 *   page_table  int32; row b's table at page_table + t*pt_stride with
 *               t = row_table[b] (a request's table; its rows are that
 *               request's query tokens), or t = b when row_table is NULL
 *   row_table   NULL, or int32 [rows]: table index of each row, valid in
 *               [0, num_tables); a row with an index outside it scores NaN at
 *               its live positions (as an invalid page id does)
 *   seqlens     int32 [rows]
 *   weights     fp32 [rows][64]
 *   row_ids     rows to evaluate (n_out of them); NULL = all rows in order
 *   out         float64 [n_out][table_width*64]
 */
void oracle_paged_mqa_logits(int key_kind, const uint16_t* q_bits, const uint8_t* kv,
                             int64_t kv_stride, const uint8_t* ks, int64_t ks_stride,
                             int64_t num_pages, const int32_t* page_table, int64_t pt_stride,
                             const int32_t* row_table, int32_t num_tables,
                             const int32_t* seqlens, const float* weights, int32_t rows,
                             int32_t table_width, const int32_t* row_ids, int32_t n_out,
                             double* out) {
  const int64_t ncols = (int64_t)table_width * PG;
  if (row_ids == NULL) n_out = rows;
  const int64_t total = (int64_t)n_out * table_width;

#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t t = 0; t < total; ++t) {
    const int32_t r = (int32_t)(t / table_width);
    const int32_t j = (int32_t)(t % table_width);
    const int32_t b = row_ids ? row_ids[r] : r;
    double* o = out + (int64_t)r * ncols + (int64_t)j * PG;

    int64_t L = seqlens[b];
    if (L < 0) L = 0;
    if (L > ncols) L = ncols;

    if ((int64_t)j * PG >= L) {            /* whole page past the length */
      for (int i = 0; i < PG; ++i) o[i] = -INFINITY;
      continue;
    }
    const int64_t tr = row_table ? (int64_t)row_table[b] : (int64_t)b;
    const int table_ok = row_table == NULL || (tr >= 0 && tr < num_tables);
    const int32_t g = table_ok ? page_table[tr * pt_stride + j] : -1;
    const int page_ok = (g >= 0 && (int64_t)g < num_pages);

    for (int i = 0; i < PG; ++i) {
      const int64_t p = (int64_t)j * PG + i;
      if (p >= L) { o[i] = -INFINITY; continue; }
      if (!page_ok) { o[i] = NAN; continue; }

      double k[HD];
      double s;
      if (key_kind == 0) {
        const uint8_t* kp = kv + (int64_t)g * kv_stride + (int64_t)i * HD;
        for (int d = 0; d < HD; ++d) k[d] = oracle_e4m3fn_value(kp[d]);
        float sf;
        memcpy(&sf, ks + (int64_t)g * ks_stride + 4 * i, sizeof sf);
        s = (double)sf;
      } else {
        const uint8_t* kp = kv + (int64_t)g * kv_stride + (int64_t)i * HD * 2;
        for (int d = 0; d < HD; ++d) {
          uint16_t bits;
          memcpy(&bits, kp + 2 * d, sizeof bits);
          k[d] = oracle_bf16_value(bits);
        }
        s = 1.0;
      }

      double acc = 0.0;
      for (int h = 0; h < NH; ++h) {
        const uint16_t* qh = q_bits + ((int64_t)b * NH + h) * HD;
        double dot = 0.0;
        for (int d = 0; d < HD; ++d) dot += oracle_bf16_value(qh[d]) * k[d];
        acc += (double)weights[(int64_t)b * NH + h] * relu(s * dot);
      }
      o[i] = acc;
    }
  }
}

/*
 * Paged key store, fp8 (the write side of the cache block above): each key of
 * 128 values gets one scale and 128 e4m3fn codes.  The pages give the block
 * (64 positions x 128 fp8 values, then 64 fp32 scales) and a per-position
 * scale; the quantiser itself is the reading taken for it -- scale = amax/448,
 * the largest e4m3fn magnitude -- and every step is done in float32, in this
 * order, so that a float32 implementation can match it bit for bit:
 *
 *   k_d    = the bf16 key value as float32 (exact)
 *   amax   = max_d |k_d|
 *   scale  = amax > 0 ? amax / 448 : 1                (float32 division)
 *   y_d    = clamp(k_d / scale, -448, 448)            (float32 division)
 *   code_d = e4m3fn nearest to y_d, ties to the even code; the sign of y_d is
 *            kept when the nearest value is 0
 */

/* e4m3fn code nearest to y (|y| <= 448), ties to the code with mantissa LSB 0. */
uint32_t oracle_e4m3fn_encode(float y) {
  const double a = fabs((double)y);
  uint32_t best = 0;
  double best_d = INFINITY;
  for (uint32_t c = 0; c <= 0x7Eu; ++c) {  /* the non-negative finite codes, ascending */
    const double d = fabs(oracle_e4m3fn_value(c) - a);
    if (d < best_d || (d == best_d && (c & 1u) == 0u)) {
      best_d = d;
      best = c;
    }
  }
  return signbit(y) ? (best | 0x80u) : best;
}

void oracle_quantize_keys_fp8(const uint16_t* keys_bits, int64_t n, uint8_t* codes, float* scales) {
  for (int64_t t = 0; t < n; ++t) {
    float k[HD];
    float amax = 0.0f;
    for (int d = 0; d < HD; ++d) {
      const uint32_t u = (uint32_t)keys_bits[t * HD + d] << 16;
      memcpy(&k[d], &u, sizeof(float));
      const float m = fabsf(k[d]);
      if (m > amax) amax = m;
    }
    const float scale = amax > 0.0f ? amax / 448.0f : 1.0f;
    scales[t] = scale;
    for (int d = 0; d < HD; ++d) {
      float y = k[d] / scale;
      if (y > 448.0f) y = 448.0f;
      if (y < -448.0f) y = -448.0f;
      codes[t * HD + d] = (uint8_t)oracle_e4m3fn_encode(y);
    }
  }
}

/*
 * Top-k selection over logits rows, the consumer of the -inf-masked output
 * ("The Final Gate: Validating a Custom Triton Indexer Kernel Before
 * Production Deployment", section "What the Test Output Reveals": the masking
 * matters because the logits feed a downstream top-k).  The pages give no k
 * and no tie rule; the readings taken:
 *
 *   candidates   positions p < L, L = clamp(seqlen, 0, ncols)
 *   order        larger value first; equal values (-0 equals +0) by lower
 *                position; NaN after every number
 *   output       the first min(k, L) candidates of that order, written in
 *                ascending position order, then -1 up to k
 *
 * The values are given as float64 (float32 logits convert exactly, with the
 * same order).
 */
struct topk_cand {
  double v;
  int32_t p;
};

static int topk_rank_cmp(const void* a, const void* b) {
  const struct topk_cand* x = (const struct topk_cand*)a;
  const struct topk_cand* y = (const struct topk_cand*)b;
  const int xn = isnan(x->v) ? 1 : 0, yn = isnan(y->v) ? 1 : 0;
  if (xn != yn) return xn - yn;
  if (!xn && x->v != y->v) return x->v > y->v ? -1 : 1;
  return (x->p > y->p) - (x->p < y->p);
}

static int topk_pos_cmp(const void* a, const void* b) {
  const int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
  return (x > y) - (x < y);
}

void oracle_topk(const double* vals, int64_t row_stride, const int32_t* seqlens, int32_t rows,
                 int32_t ncols, int32_t k, int32_t* idx) {
#pragma omp parallel for schedule(dynamic)
  for (int32_t b = 0; b < rows; ++b) {
    int32_t L = seqlens[b];
    if (L < 0) L = 0;
    if (L > ncols) L = ncols;
    const int32_t m = L < k ? L : k;
    int32_t* o = idx + (int64_t)b * k;
    if (m > 0) {
      struct topk_cand* c = (struct topk_cand*)malloc(sizeof(struct topk_cand) * (size_t)L);
      for (int32_t p = 0; p < L; ++p) {
        c[p].v = vals[(int64_t)b * row_stride + p];
        c[p].p = p;
      }
      qsort(c, (size_t)L, sizeof(struct topk_cand), topk_rank_cmp);
      for (int32_t t = 0; t < m; ++t) o[t] = c[t].p;
      free(c);
      qsort(o, (size_t)m, sizeof(int32_t), topk_pos_cmp);
    }
    for (int32_t t = m; t < k; ++t) o[t] = -1;
  }
}

/* Number of OpenMP threads the oracle runs with (1 when built without it). */
int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Set the OpenMP thread count used by later calls (no-op without OpenMP). */
void oracle_set_num_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}
