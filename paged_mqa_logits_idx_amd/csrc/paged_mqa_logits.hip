// paged_mqa_logits.hip -- gfx950 kernels and C-ABI entry points of the paged
// MQA-logits indexer (declared in include/paged_mqa_logits.h).
//
// The computation, per query row b and cached c4-position p = 64*j + i:
//   out[b][p] = sum_h w[b][h] * ReLU(s_p * <q[b][h], k_p>)   if p < L_b, else -inf
// ("The Dispatch Wire: Connecting a Triton Indexer Kernel to Production
// Inference", sections "The Road to This Message" and "Assumptions and Risks").
//
// Work decomposition.  One wave (64 lanes) scores one 64-position page of one
// row: a 64-head x 64-position x 128 contraction done as 64 MFMAs
// v_mfma_f32_16x16x32_bf16, then the epilogue (scale, ReLU, head weights, sum
// over heads) on the accumulators and one 256-byte store.  The grid is fixed by
// (rows, table_width); a page that starts at or past the row length is written
// as -inf without touching the page table or the cache ("The Moment the
// Context-Length Tax Vanished: Committing the O(actual) Triton Indexer",
// section "The Commit: Engineering as Narrative").
//
// Two kernels share that per-page core:
//  * rowwise  -- rows with their own page tables (decode).  Each wave owns a run
//    of page slots of one row, keeps the row's query in registers across them
//    and streams key bytes from HBM straight into the MFMA operand layout,
//    prefetching the next page while the current one is multiplied.
//  * shared   -- rows that share one page table (page_table_row_stride == 0:
//    the query tokens of one prefill request).  A workgroup owns 4 rows x a
//    chunk of pages; each page is loaded once into LDS (XOR-swizzled) and all
//    4 waves multiply it against their own row's query, so key bytes are
//    fetched once per 4 rows and the query stays in registers for the chunk.
//
// MFMA fragment layout (16x16x32 bf16, lane l, n = l % 16, g = l / 16):
//   A (query)  row  h = 16*mb + n,  8 k-values,
//   B (keys)   col  i = 16*nb + n,  8 k-values (same k-set as A for lane l),
//   D          D[4*g + r][n] in accumulator element r.
// The contraction is invariant under any permutation of k applied to both
// operands, so lane group g takes the contiguous k-range [32g, 32g+32) and
// MFMA kb in 0..3 takes its 8-value slice 32g + 8kb .. +8.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "paged_mqa_logits.h"

namespace {

constexpr int kHeads = IDX_NUM_HEADS;     // 64
constexpr int kDim = IDX_HEAD_DIM;        // 128
constexpr int kPage = IDX_PAGE_POSITIONS; // 64
constexpr int kFp8 = 0;
constexpr int kBf16 = 1;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct Params {
  const uint8_t* q;   // bf16 [rows][64][128]
  const uint8_t* kv;  // key pool
  const uint8_t* ks;  // scale bytes (fp8 only)
  const int32_t* pt;  // page tables
  const int32_t* sl;  // seqlens
  const float* w;     // [rows][64]
  float* out;         // [rows][width*64]
  int64_t num_pages, kv_stride, ks_stride, pt_stride;
  int32_t rows, width;
};

// Raw key bytes of one page for one lane, already in B-fragment order:
// 4 position blocks (nb) x 32 k-values.  fp8: 32 bytes per nb; bf16: 64.
template <int KEY>
struct PageKeys {
  static constexpr int kVec = (KEY == kFp8) ? 2 : 4;  // u32x4 per nb
  u32x4 v[4][kVec];
  float s[4];  // scale of position 16*nb + n (1 for bf16)
};

__device__ __forceinline__ uint32_t bits_of(bf16x2 x) { return __builtin_bit_cast(uint32_t, x); }

// 8 e4m3fn bytes -> 8 bf16 (exact: every e4m3fn value is a bf16 value).
__device__ __forceinline__ bf16x8 fp8x8_to_bf16x8(uint32_t lo, uint32_t hi) {
  u32x4 r;
  r.x = bits_of(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false));
  r.y = bits_of(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true));
  r.z = bits_of(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false));
  r.w = bits_of(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true));
  return __builtin_bit_cast(bf16x8, r);
}

// Query fragments of row b (A operand) and the lane's 16 head weights.
struct RowQuery {
  bf16x8 a[4][4];  // [mb][kb]
  f32x4 w[4];      // w[mb][r] = weight of head 16*mb + 4*g + r
};

__device__ __forceinline__ void load_row_query(const Params& p, int32_t b, int lane, RowQuery& rq) {
  const int n = lane & 15, g = lane >> 4;
  const uint8_t* qrow = p.q + (int64_t)b * (kHeads * kDim * 2);
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    const u32x4* src = reinterpret_cast<const u32x4*>(qrow + ((16 * mb + n) * kDim + 32 * g) * 2);
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) rq.a[mb][kb] = __builtin_bit_cast(bf16x8, src[kb]);
    rq.w[mb] = *reinterpret_cast<const f32x4*>(p.w + (int64_t)b * kHeads + 16 * mb + 4 * g);
  }
}

// Global -> registers, B-fragment order (rowwise kernel).
template <int KEY>
__device__ __forceinline__ void load_page_global(const Params& p, int32_t gp, int lane, PageKeys<KEY>& pk) {
  const int n = lane & 15, g = lane >> 4;
  const uint8_t* base = p.kv + (int64_t)gp * p.kv_stride;
  constexpr int kRowBytes = (KEY == kFp8) ? kDim : 2 * kDim;
  constexpr int kSlice = (KEY == kFp8) ? 32 : 64;  // bytes of 32 k-values
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    const u32x4* src = reinterpret_cast<const u32x4*>(base + (16 * nb + n) * kRowBytes + kSlice * g);
#pragma unroll
    for (int v = 0; v < PageKeys<KEY>::kVec; ++v) pk.v[nb][v] = __builtin_nontemporal_load(src + v);
  }
  if constexpr (KEY == kFp8) {
    const float* sc = reinterpret_cast<const float*>(p.ks + (int64_t)gp * p.ks_stride);
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) pk.s[nb] = sc[16 * nb + n];
  } else {
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) pk.s[nb] = 1.0f;
  }
}

// Score one page: returns the logit of position 64*j + lane (before masking).
//   x[h][i]  = <q[h], k_i>                       (MFMA, fp32 accumulate)
//   logit_i  = |s_i| * sum_h w[h] * ReLU(x')      with x' = x for s_i >= 0 and
//              x' = -x (keys negated, exact) for s_i < 0, which equals
//              sum_h w[h] * ReLU(s_i * x) in exact arithmetic.
template <int KEY>
__device__ __forceinline__ float score_page(const RowQuery& rq, const PageKeys<KEY>& pk, int lane) {
  const int g = lane >> 4;
  float res[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    bf16x8 kop[4];
    if constexpr (KEY == kFp8) {
      const uint32_t flip = (__builtin_bit_cast(uint32_t, pk.s[nb]) >> 31) * 0x80808080u;
      kop[0] = fp8x8_to_bf16x8(pk.v[nb][0].x ^ flip, pk.v[nb][0].y ^ flip);
      kop[1] = fp8x8_to_bf16x8(pk.v[nb][0].z ^ flip, pk.v[nb][0].w ^ flip);
      kop[2] = fp8x8_to_bf16x8(pk.v[nb][1].x ^ flip, pk.v[nb][1].y ^ flip);
      kop[3] = fp8x8_to_bf16x8(pk.v[nb][1].z ^ flip, pk.v[nb][1].w ^ flip);
    } else {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) kop[kb] = __builtin_bit_cast(bf16x8, pk.v[nb][kb]);
    }
    f32x4 acc[4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) acc[mb] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
        acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(rq.a[mb][kb], kop[kb], acc[mb], 0, 0, 0);
    float part = 0.f;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        part = fmaf(rq.w[mb][r], __builtin_elementwise_maximum(acc[mb][r], 0.0f), part);
    part += __shfl_xor(part, 16);
    part += __shfl_xor(part, 32);
    res[nb] = (KEY == kFp8) ? fabsf(pk.s[nb]) * part : part;
  }
  // Lane l = 16*g + n owns position 16*g + n, i.e. block nb = g, column n.
  return g == 0 ? res[0] : g == 1 ? res[1] : g == 2 ? res[2] : res[3];
}

__device__ __forceinline__ void store_page(float* orow, int32_t j, int32_t L, int lane, float v) {
  const int32_t pos = j * kPage + lane;
  __builtin_nontemporal_store(pos < L ? v : -INFINITY, orow + pos);
}

__device__ __forceinline__ void store_bad_page(float* orow, int32_t j, int32_t L, int lane) {
  const int32_t pos = j * kPage + lane;
  __builtin_nontemporal_store(pos < L ? __builtin_nanf("") : -INFINITY, orow + pos);
}

// -inf over npages whole pages starting at page slot j (16-byte stores).
__device__ __forceinline__ void fill_neg_inf(float* orow, int32_t j, int32_t npages, int lane) {
  f32x4* dst = reinterpret_cast<f32x4*>(orow + (int64_t)j * kPage);
  const f32x4 ninf = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
  for (int32_t t = lane; t < npages * (kPage / 4); t += 64) __builtin_nontemporal_store(ninf, dst + t);
}

__device__ __forceinline__ int32_t clamp_len(int32_t L, int32_t width) {
  return min(max(L, 0), width * kPage);
}

__device__ __forceinline__ bool page_ok(int32_t gp, int64_t num_pages) {
  return gp >= 0 && (int64_t)gp < num_pages;
}

// ---------------------------------------------------------------------------
// rowwise kernel: unit = (row b, WAVES*PPW consecutive page slots); wave w of
// the unit owns PPW slots.
template <int KEY, int PPW, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void rowwise_kernel(Params p, int32_t units_per_row,
                                                              int64_t total_units) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int32_t width = p.width;
  for (int64_t unit = blockIdx.x; unit < total_units; unit += gridDim.x) {
    const int32_t b = (int32_t)(unit / units_per_row);
    const int32_t u = (int32_t)(unit % units_per_row);
    const int32_t j0 = (u * WAVES + wave) * PPW;
    if (j0 >= width) continue;
    const int32_t jend = min(j0 + PPW, width);
    const int32_t L = clamp_len(p.sl[b], width);
    const int32_t live = (L + kPage - 1) / kPage;
    const int32_t jl = max(j0, min(jend, live));  // [j0, jl) live, [jl, jend) dead
    float* orow = p.out + (int64_t)b * width * kPage;

    if (j0 < jl) {
      RowQuery rq;
      load_row_query(p, b, lane, rq);
      const int32_t* tab = p.pt + (int64_t)b * p.pt_stride;
      PageKeys<KEY> buf[2];
      int32_t gcur = tab[j0];
      bool okcur = page_ok(gcur, p.num_pages);
      if (okcur) load_page_global<KEY>(p, gcur, lane, buf[0]);
#pragma unroll
      for (int t = 0; t < PPW; ++t) {
        const int32_t j = j0 + t;
        if (j < jl) {
          int32_t gnxt = 0;
          bool oknxt = false;
          if (t + 1 < PPW && j + 1 < jl) {
            gnxt = tab[j + 1];
            oknxt = page_ok(gnxt, p.num_pages);
            if (oknxt) load_page_global<KEY>(p, gnxt, lane, buf[(t + 1) & 1]);
          }
          if (okcur)
            store_page(orow, j, L, lane, score_page<KEY>(rq, buf[t & 1], lane));
          else
            store_bad_page(orow, j, L, lane);
          gcur = gnxt;
          okcur = oknxt;
        }
      }
    }
    if (jl < jend) fill_neg_inf(orow, jl, jend - jl, lane);
  }
}

// ---------------------------------------------------------------------------
// shared kernel: rows share one page table.  Unit = (block of 4 rows, chunk of
// CHUNK page slots); wave w scores row 4*rb + w.  Pages go through LDS.
constexpr int kSharedRows = 4;

template <int KEY>
struct LdsPage {
  static constexpr int kRowBytes = (KEY == kFp8) ? kDim : 2 * kDim;  // 128 / 256
  static constexpr int kChunks = kRowBytes / 16;                       // 8 / 16 per row
  static constexpr int kKeyBytes = kPage * kRowBytes;                  // 8192 / 16384
  static constexpr int kBytes = kKeyBytes + ((KEY == kFp8) ? kPage * 4 : 0);
  // 16-byte chunk c of key row i lives at row i, chunk c ^ (i % kChunks') where
  // the XOR spreads the 16 rows a B-fragment read touches over distinct banks.
  static __device__ __forceinline__ int chunk_off(int i, int c) {
    return i * kRowBytes + ((c ^ (i & (kChunks - 1))) << 4);
  }
};

// Per-thread share of one page copy: 16-byte chunks (plus scale chunks).
template <int KEY>
struct Stage {
  static constexpr int kKeyChunks = LdsPage<KEY>::kKeyBytes / 16 / (64 * kSharedRows);  // 2 / 4
  u32x4 v[kKeyChunks];
  u32x4 sc;  // threads 0..15 carry the 256 scale bytes (fp8)
};

template <int KEY>
__device__ __forceinline__ void stage_load(const Params& p, int32_t gp, int tid, Stage<KEY>& st) {
  const uint8_t* base = p.kv + (int64_t)gp * p.kv_stride;
#pragma unroll
  for (int c = 0; c < Stage<KEY>::kKeyChunks; ++c)
    st.v[c] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(base) + tid + c * 64 * kSharedRows);
  if constexpr (KEY == kFp8) {
    if (tid < 16)
      st.sc = *reinterpret_cast<const u32x4*>(p.ks + (int64_t)gp * p.ks_stride + 16 * tid);
  }
}

template <int KEY>
__device__ __forceinline__ void stage_store(uint8_t* lds, int tid, const Stage<KEY>& st) {
  constexpr int kChunks = LdsPage<KEY>::kChunks;
#pragma unroll
  for (int c = 0; c < Stage<KEY>::kKeyChunks; ++c) {
    const int ci = tid + c * 64 * kSharedRows;
    *reinterpret_cast<u32x4*>(lds + LdsPage<KEY>::chunk_off(ci / kChunks, ci % kChunks)) = st.v[c];
  }
  if constexpr (KEY == kFp8) {
    if (tid < 16) *reinterpret_cast<u32x4*>(lds + LdsPage<KEY>::kKeyBytes + 16 * tid) = st.sc;
  }
}

template <int KEY>
__device__ __forceinline__ void load_page_lds(const uint8_t* lds, int lane, PageKeys<KEY>& pk) {
  const int n = lane & 15, g = lane >> 4;
  constexpr int kVec = PageKeys<KEY>::kVec;
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    const int i = 16 * nb + n;
#pragma unroll
    for (int v = 0; v < kVec; ++v)
      pk.v[nb][v] = *reinterpret_cast<const u32x4*>(lds + LdsPage<KEY>::chunk_off(i, kVec * g + v));
    if constexpr (KEY == kFp8)
      pk.s[nb] = reinterpret_cast<const float*>(lds + LdsPage<KEY>::kKeyBytes)[i];
    else
      pk.s[nb] = 1.0f;
  }
}

template <int KEY, int CHUNK>
__global__ __launch_bounds__(64 * kSharedRows) void shared_kernel(Params p, int32_t row_blocks,
                                                                  int32_t chunks, int32_t rb_per_xcd,
                                                                  int64_t total_slots) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][LdsPage<KEY>::kBytes];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int32_t width = p.width;
  const int32_t* tab = p.pt;  // shared table (row stride 0)

  for (int64_t slot = blockIdx.x; slot < total_slots; slot += gridDim.x) {
    // Workgroup ids are dealt to the 8 XCDs round-robin; keep all chunks of a
    // row block on one XCD (its query rows stay in that L2) and hand out row
    // blocks longest-first (largest index first).
    const int32_t xcd = (int32_t)(slot % 8);
    const int64_t seq = slot / 8;
    const int32_t rb_local = (int32_t)(seq / chunks);
    const int32_t c = (int32_t)(seq % chunks);
    const int32_t rb_rev = rb_local * 8 + xcd;
    if (rb_local >= rb_per_xcd || rb_rev >= row_blocks) continue;
    const int32_t rb = row_blocks - 1 - rb_rev;

    const int32_t j0 = c * CHUNK;
    const int32_t jend = min(j0 + CHUNK, width);
    const int32_t b = rb * kSharedRows + wave;
    const bool row_ok = b < p.rows;
    float* orow = p.out + (int64_t)b * width * kPage;

    // Longest live prefix over the block's rows decides which pages to load.
    int32_t Lmax = 0;
#pragma unroll
    for (int r = 0; r < kSharedRows; ++r) {
      const int32_t br = rb * kSharedRows + r;
      if (br < p.rows) Lmax = max(Lmax, clamp_len(p.sl[br], width));
    }
    const int32_t L = row_ok ? clamp_len(p.sl[b], width) : 0;
    const int32_t live_w = (L + kPage - 1) / kPage;
    const int32_t jl = max(j0, min(jend, (Lmax + kPage - 1) / kPage));  // pages any row needs

    if (j0 < jl) {
      RowQuery rq;
      if (row_ok && j0 < live_w) load_row_query(p, b, lane, rq);
      Stage<KEY> st;
      int32_t gcur = tab[j0];
      bool okcur = page_ok(gcur, p.num_pages);
      if (okcur) stage_load<KEY>(p, gcur, tid, st);
      for (int32_t j = j0; j < jl; ++j) {
        uint8_t* buf = lds[(j - j0) & 1];
        if (okcur) stage_store<KEY>(buf, tid, st);
        __syncthreads();
        int32_t gnxt = 0;
        bool oknxt = false;
        if (j + 1 < jl) {
          gnxt = tab[j + 1];
          oknxt = page_ok(gnxt, p.num_pages);
          if (oknxt) stage_load<KEY>(p, gnxt, tid, st);
        }
        if (row_ok) {
          if (j >= live_w) {
            store_page(orow, j, 0, lane, 0.f);  // whole page past this row's length
          } else if (okcur) {
            PageKeys<KEY> pk;
            load_page_lds<KEY>(buf, lane, pk);
            store_page(orow, j, L, lane, score_page<KEY>(rq, pk, lane));
          } else {
            store_bad_page(orow, j, L, lane);
          }
        }
        okcur = oknxt;
        gcur = gnxt;
      }
      __syncthreads();  // LDS is reused by this workgroup's next slot
    }
    if (row_ok && jl < jend) fill_neg_inf(orow, jl, jend - jl, lane);
  }
}

// ---------------------------------------------------------------------------
// Host side.

constexpr int kRowwisePPW = 2;
constexpr int kRowwiseWaves = 4;
constexpr int kSharedChunk = 8;
constexpr int64_t kMaxGrid = (int64_t)1 << 20;  // larger grids loop (grid-stride)
constexpr int32_t kMaxWidth = 1 << 24;

inline bool aligned(const void* ptr, uintptr_t a) { return ((uintptr_t)ptr & (a - 1)) == 0; }

int validate(int key, const void* q, const void* kv_pages, const float* kscale,
             const int32_t* page_table, const int32_t* seqlens, const float* weights,
             const float* out, int32_t rows, int32_t num_heads, int32_t head_dim,
             int32_t table_width, int64_t num_pages, int64_t kv_page_stride,
             int64_t kscale_page_stride, int64_t page_table_row_stride) {
  if (num_heads != kHeads || head_dim != kDim) return IDX_ERR_UNSUPPORTED;
  if (rows < 0 || table_width < 0 || table_width > kMaxWidth || num_pages < 0 ||
      page_table_row_stride < 0)
    return IDX_ERR_SHAPE;
  const int64_t min_kv = (key == kFp8) ? (int64_t)kPage * kDim : (int64_t)kPage * kDim * 2;
  if (kv_page_stride < min_kv || kv_page_stride > ((int64_t)1 << 32)) return IDX_ERR_SHAPE;
  if (key == kFp8 && (kscale_page_stride < kPage * 4 || kscale_page_stride > ((int64_t)1 << 32)))
    return IDX_ERR_SHAPE;
  if (rows == 0 || table_width == 0) return IDX_OK;
  if (!q || !kv_pages || !page_table || !seqlens || !weights || !out) return IDX_ERR_NULL;
  if (key == kFp8 ? (kscale == nullptr) : (kscale != nullptr)) return IDX_ERR_NULL;
  if (!aligned(q, 16) || !aligned(kv_pages, 16) || !aligned(weights, 16) || !aligned(out, 16) ||
      (kv_page_stride % 16) != 0 || !aligned(page_table, 4) || !aligned(seqlens, 4))
    return IDX_ERR_ALIGN;
  if (key == kFp8 && (!aligned(kscale, 4) || (kscale_page_stride % 4) != 0)) return IDX_ERR_ALIGN;
  return IDX_OK;
}

template <int KEY>
int launch(const void* q, const void* kv_pages, const float* kscale, const int32_t* page_table,
           const int32_t* seqlens, const float* weights, float* out, int32_t rows,
           int32_t num_heads, int32_t head_dim, int32_t table_width, int64_t num_pages,
           int64_t kv_page_stride, int64_t kscale_page_stride, int64_t page_table_row_stride,
           hipStream_t stream) {
  const int st = validate(KEY, q, kv_pages, kscale, page_table, seqlens, weights, out, rows,
                          num_heads, head_dim, table_width, num_pages, kv_page_stride,
                          kscale_page_stride, page_table_row_stride);
  if (st != IDX_OK || rows == 0 || table_width == 0) return st;

  Params p;
  p.q = static_cast<const uint8_t*>(q);
  p.kv = static_cast<const uint8_t*>(kv_pages);
  p.ks = reinterpret_cast<const uint8_t*>(kscale);
  p.pt = page_table;
  p.sl = seqlens;
  p.w = weights;
  p.out = out;
  p.num_pages = num_pages;
  p.kv_stride = kv_page_stride;
  p.ks_stride = (KEY == kFp8) ? kscale_page_stride : 0;
  p.pt_stride = page_table_row_stride;
  p.rows = rows;
  p.width = table_width;

  (void)hipGetLastError();  // start from a clean error state
  if (page_table_row_stride == 0 && rows > 1) {
    const int32_t row_blocks = (rows + kSharedRows - 1) / kSharedRows;
    const int32_t chunks = (table_width + kSharedChunk - 1) / kSharedChunk;
    const int32_t rb_per_xcd = (row_blocks + 7) / 8;
    const int64_t total = (int64_t)8 * rb_per_xcd * chunks;
    const int64_t grid = total < kMaxGrid ? total : kMaxGrid;
    shared_kernel<KEY, kSharedChunk><<<dim3((uint32_t)grid), dim3(64 * kSharedRows), 0, stream>>>(
        p, row_blocks, chunks, rb_per_xcd, total);
  } else {
    constexpr int per_unit = kRowwisePPW * kRowwiseWaves;
    const int32_t units_per_row = (table_width + per_unit - 1) / per_unit;
    const int64_t total = (int64_t)rows * units_per_row;
    const int64_t grid = total < kMaxGrid ? total : kMaxGrid;
    rowwise_kernel<KEY, kRowwisePPW, kRowwiseWaves>
        <<<dim3((uint32_t)grid), dim3(64 * kRowwiseWaves), 0, stream>>>(p, units_per_row, total);
  }
  return hipGetLastError() == hipSuccess ? IDX_OK : IDX_ERR_LAUNCH;
}

}  // namespace

extern "C" {

int idx_paged_mqa_logits_fp8(const void* q, const void* kv_pages, const float* kscale,
                             const int32_t* page_table, const int32_t* seqlens,
                             const float* weights, float* out, int32_t rows, int32_t num_heads,
                             int32_t head_dim, int32_t table_width, int64_t num_pages,
                             int64_t kv_page_stride, int64_t kscale_page_stride,
                             int64_t page_table_row_stride, hipStream_t stream) {
  return launch<kFp8>(q, kv_pages, kscale, page_table, seqlens, weights, out, rows, num_heads,
                      head_dim, table_width, num_pages, kv_page_stride, kscale_page_stride,
                      page_table_row_stride, stream);
}

int idx_paged_mqa_logits_bf16(const void* q, const void* kv_pages, const float* kscale,
                              const int32_t* page_table, const int32_t* seqlens,
                              const float* weights, float* out, int32_t rows, int32_t num_heads,
                              int32_t head_dim, int32_t table_width, int64_t num_pages,
                              int64_t kv_page_stride, int64_t kscale_page_stride,
                              int64_t page_table_row_stride, hipStream_t stream) {
  return launch<kBf16>(q, kv_pages, kscale, page_table, seqlens, weights, out, rows, num_heads,
                       head_dim, table_width, num_pages, kv_page_stride, kscale_page_stride,
                       page_table_row_stride, stream);
}

const char* idx_status_string(int status) {
  switch (status) {
    case IDX_OK: return "ok";
    case IDX_ERR_NULL: return "null pointer (or kscale passed to the bf16 variant)";
    case IDX_ERR_UNSUPPORTED: return "unsupported num_heads/head_dim (need 64 and 128)";
    case IDX_ERR_SHAPE: return "invalid dimension or stride";
    case IDX_ERR_ALIGN: return "misaligned pointer or stride";
    case IDX_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}

int idx_abi_version(void) { return IDX_ABI_VERSION; }

}  // extern "C"
