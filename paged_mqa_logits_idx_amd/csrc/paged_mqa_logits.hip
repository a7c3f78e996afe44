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
// over heads) on the accumulators, leaving one logit per lane.  The balanced
// and shared kernels collect a run of pages' logits in LDS and store them
// after the run's key DMAs; the rowwise kernel stores each page's 256 bytes at
// once.  The grid is fixed by
// (rows, table_width); a page that starts at or past the row length is written
// as -inf without touching the page table or the cache ("The Moment the
// Context-Length Tax Vanished: Committing the O(actual) Triton Indexer",
// section "The Commit: Engineering as Narrative").
//
// Three kernels share that per-page core:
//  * balanced -- rows with their own page tables (decode, up to 1024 rows).  A
//    fixed grid whose waves take equal shares of all rows' live pages and of
//    the -inf slots; each wave keeps its row's query in registers and streams
//    pages HBM -> LDS by DMA, the next pages in flight while one is multiplied.
//  * rowwise  -- rows with their own page tables beyond 1024 rows.  Each wave
//    owns a run of page slots of one row and streams key bytes from HBM
//    straight into the MFMA operand layout, one page ahead.
//  * shared   -- rows that share page tables: the query tokens of one
//    prefill request (page_table_row_stride == 0), or of several requests
//    with a row -> request table map.  A workgroup owns 4 rows x a chunk of
//    pages; each page is loaded once into LDS (XOR-swizzled) and the waves
//    whose rows use that table multiply it against their own row's query, so
//    key bytes are fetched once per 4 rows and the query stays in registers
//    for the chunk.  A block of 4 rows that straddles requests runs once per
//    table.
// Beside them: the paged key store (quantise / copy keys into pool slots) and
// the top-k over logits rows.
//
// MFMA fragment layout (16x16x32 bf16, lane l, n = l % 16, g = l / 16):
//   A (query)  row  h = 16*mb + n,  8 k-values,
//   B (keys)   col  i = 16*nb + n,  8 k-values (same k-set as A for lane l),
//   D          D[4*g + r][n] in accumulator element r.
// The contraction is invariant under any permutation of k applied to both
// operands.  MFMA kb in 0..3 gives lane group g the 8 k-values
//   k(kb, g) = 64*(kb/2) + 16*g + 8*(kb%2) .. +8,
// so that
//   * a query load (one kb, 16 bytes per lane) touches one 128-byte line per
//     head row: the four lane groups read 16 bytes at 32-byte steps inside
//     the same 128 bytes (16 lines per instruction, not the 32 of a layout
//     with each lane group's k-range 64 bytes away from the next);
//   * a lane's fp8 key bytes of one position are two 16-byte chunks, g and
//     4 + g of the 128-byte row: chunk g holds kb = 0, 1 and chunk 4 + g
//     kb = 2, 3 (bf16 keys: 16-byte chunks 2g, 2g+1, 8+2g, 9+2g of the
//     256-byte row for kb = 0..3).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <atomic>
#include <type_traits>

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
typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((address_space(3))) void* lds_ptr;
typedef __attribute__((address_space(1))) const void* global_ptr;

struct Params {
  const uint8_t* q;   // bf16 [rows][64][128]
  const uint8_t* kv;  // key pool
  const uint8_t* ks;  // scale bytes (fp8 only)
  const int32_t* pt;  // page tables
  const int32_t* sl;  // seqlens
  const float* w;     // [rows][64]
  float* out;         // [rows][width*64]
  int64_t num_pages, kv_stride, ks_stride, pt_stride;
  uint32_t pages_lim;  // min(num_pages, 2^31): page ids below it are in the pool (a 32-bit scalar compare)
  int32_t rows, width;
  int32_t fill;       // 0: page slots past a row's live pages are left unwritten
  const int32_t* rt;  // shared kernel: table index of each row (NULL: table 0 for all)
  int32_t num_tables; // valid table indices [0, num_tables) when rt is set
};

// Raw key bytes of one page for one lane, already in B-fragment order:
// 4 position blocks (nb) x 32 k-values (fp8: 32 bytes per nb; bf16: 64), and
// the scale of position `lane` of the page (1 for bf16).
template <int KEY>
struct PageKeys {
  static constexpr int kVec = (KEY == kFp8) ? 2 : 4;  // u32x4 per nb
  u32x4 v[4][kVec];
  float s;
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
    // k(kb, g) = 64*(kb/2) + 16*g + 8*(kb%2): byte offset 128*(kb/2) + 32*g + 16*(kb%2)
    const uint8_t* hrow = qrow + (16 * mb + n) * (kDim * 2) + 32 * g;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
      rq.a[mb][kb] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(hrow + 128 * (kb >> 1) + 16 * (kb & 1)));
    rq.w[mb] = *reinterpret_cast<const f32x4*>(p.w + (int64_t)b * kHeads + 16 * mb + 4 * g);
  }
}

// Global -> registers, B-fragment order (rowwise kernel).
template <int KEY>
__device__ __forceinline__ void load_page_global(const Params& p, int32_t gp, int lane, PageKeys<KEY>& pk) {
  const int n = lane & 15, g = lane >> 4;
  const uint8_t* base = p.kv + (int64_t)gp * p.kv_stride;
  constexpr int kRowBytes = (KEY == kFp8) ? kDim : 2 * kDim;
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    const uint8_t* row = base + (16 * nb + n) * kRowBytes;
#pragma unroll
    for (int v = 0; v < PageKeys<KEY>::kVec; ++v) {
      // fp8: 16-byte chunks g and 4 + g; bf16: chunks 2g, 2g+1, 8+2g, 9+2g
      const int c = (KEY == kFp8) ? g + 4 * v : 8 * (v >> 1) + 2 * g + (v & 1);
      pk.v[nb][v] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(row + 16 * c));
    }
  }
  if constexpr (KEY == kFp8)
    pk.s = reinterpret_cast<const float*>(p.ks + (int64_t)gp * p.ks_stride)[lane];
  else
    pk.s = 1.0f;
}

// Score one page: returns the logit of position 64*j + lane (before masking).
//   x[h][i]  = <q[h], k_i>                       (MFMA, fp32 accumulate)
//   logit_i  = |s_i| * sum_h w[h] * ReLU(x')      with x' = x for s_i >= 0 and
//              x' = -x (keys negated, exact) for s_i < 0, which equals
//              sum_h w[h] * ReLU(s_i * x) in exact arithmetic.
// Lane l = 16*g + n holds, per position block nb, the partial sum over its 16
// heads of position 16*nb + n; a two-step butterfly (xor 16, xor 32) leaves lane
// l with the full head sum of position 16*g + n = l.
// B operands of position block nb (8 bf16 per k-slice), keys negated when
// FLIP says the position's scale is negative.
template <int KEY, bool FLIP>
__device__ __forceinline__ void block_operands(const PageKeys<KEY>& pk, int nb, int n,
                                               bf16x8 (&kop)[4]) {
  if constexpr (KEY == kFp8) {
    uint32_t flip = 0;
    if constexpr (FLIP) flip = (__shfl(pk.s, 16 * nb + n) < 0.0f) ? 0x80808080u : 0u;
    kop[0] = fp8x8_to_bf16x8(pk.v[nb][0].x ^ flip, pk.v[nb][0].y ^ flip);
    kop[1] = fp8x8_to_bf16x8(pk.v[nb][0].z ^ flip, pk.v[nb][0].w ^ flip);
    kop[2] = fp8x8_to_bf16x8(pk.v[nb][1].x ^ flip, pk.v[nb][1].y ^ flip);
    kop[3] = fp8x8_to_bf16x8(pk.v[nb][1].z ^ flip, pk.v[nb][1].w ^ flip);
  } else {
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) kop[kb] = __builtin_bit_cast(bf16x8, pk.v[nb][kb]);
  }
}

// sum over the lane's 16 heads of w[h] * ReLU(x[h]) for one position block
__device__ __forceinline__ float block_epilogue(const RowQuery& rq, const f32x4 (&acc)[4]) {
  float sum = 0.f;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      sum = fmaf(rq.w[mb][r], __builtin_elementwise_maximum(acc[mb][r], 0.0f), sum);
  return sum;
}

// part[nb] of lane (g, n) -> sum over g of part[g] of lanes (., n), in lane (g, n).
// permlane16_swap(x, y) trades rows 1, 3 of x with rows 0, 2 of y (a row is 16
// lanes), so x' + y' holds, per row pair {0,1} / {2,3}, the pair sums of x
// (rows 0 and 2) and of y (rows 1 and 3); permlane32_swap then trades the upper
// half of one such sum with the lower half of the other.
__device__ __forceinline__ float reduce_heads(const float (&part)[4]) {
  // (elements of the returned pairs go through __uint_as_float: a bit_cast of
  // an ext-vector element is folded to element 0 by this compiler)
  const auto s01 = __builtin_amdgcn_permlane16_swap(__float_as_uint(part[0]), __float_as_uint(part[1]),
                                                    false, false);
  const auto s23 = __builtin_amdgcn_permlane16_swap(__float_as_uint(part[2]), __float_as_uint(part[3]),
                                                    false, false);
  const float t = __uint_as_float(s01[0]) + __uint_as_float(s01[1]);
  const float u = __uint_as_float(s23[0]) + __uint_as_float(s23[1]);
  const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(t), __float_as_uint(u), false, false);
  return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

// Score one page: returns the logit of position 64*j + lane (before masking).
//   x[h][i]  = <q[h], k_i>                       (MFMA, fp32 accumulate)
//   logit_i  = |s_i| * sum_h w[h] * ReLU(x')      with x' = x for s_i >= 0 and
//              x' = -x (keys negated, exact) for s_i < 0, which equals
//              sum_h w[h] * ReLU(s_i * x) in exact arithmetic.
// The four position blocks are software-pipelined: while the 16 MFMAs of
// block nb run, the VALU converts block nb+1 and reduces block nb-1.
// Lane l = 16*g + n then holds, per block nb, the partial sum over its 16 heads
// of position 16*nb + n; a two-step butterfly (xor 16, xor 32) leaves lane l
// with the full head sum of position 16*g + n = l.
template <int KEY, bool FLIP>
__device__ __forceinline__ float score_page_impl(const RowQuery& rq, const PageKeys<KEY>& pk,
                                                 int lane) {
  const int n = lane & 15, g = lane >> 4;
  bf16x8 kop[2][4];
  f32x4 acc[2][4];
  float part[4];
  block_operands<KEY, FLIP>(pk, 0, n, kop[0]);
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    const int cur = nb & 1;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) acc[cur][mb] = (f32x4){0.f, 0.f, 0.f, 0.f};
    // Issue order of the 16 MFMAs of a block (each mb chain adds kb = 0..3 in
    // turn either way, so the sums are the same).  bf16 keys: chain by chain,
    // the VALU work that fills the gaps is the epilogue alone.  e4m3 keys:
    // k-slice by k-slice, so the first four MFMAs need only the first
    // converted slice.  Measured on the prefill: 1-3% faster than the other
    // order for each key type.
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int mb = (KEY == kFp8) ? (i & 3) : (i >> 2), kb = (KEY == kFp8) ? (i >> 2) : (i & 3);
      acc[cur][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(rq.a[mb][kb], kop[cur][kb], acc[cur][mb], 0, 0, 0);
    }
    if (nb + 1 < 4) block_operands<KEY, FLIP>(pk, nb + 1, n, kop[cur ^ 1]);
    if (nb > 0) part[nb - 1] = block_epilogue(rq, acc[cur ^ 1]);
    // interleave: each MFMA followed by up to 3 VALU ops (bf16) or 2 (e4m3:
    // the conversion of the next block, the epilogue of the previous one);
    // the ratios are the measured best of 1-4 for each key type
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                      // 1 MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, KEY == kFp8 ? 2 : 3, 0);  // VALU
    }
  }
  part[3] = block_epilogue(rq, acc[1]);
  const float total = reduce_heads(part);
  return (KEY == kFp8) ? fabsf(pk.s) * total : total;
}

template <int KEY>
__device__ __forceinline__ float score_page(const RowQuery& rq, const PageKeys<KEY>& pk, int lane) {
  if constexpr (KEY == kFp8) {
    if (__ballot(pk.s < 0.0f) != 0) return score_page_impl<KEY, true>(rq, pk, lane);
  }
  return score_page_impl<KEY, false>(rq, pk, lane);
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

__device__ __forceinline__ bool page_ok(int32_t gp, uint32_t pages_lim) {
  return gp >= 0 && (uint32_t)gp < pages_lim;
}

// Wave-uniform values kept in scalar registers.
__device__ __forceinline__ int32_t uniform(int32_t x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ int64_t uniform(int64_t x) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)(uint64_t)x);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)x >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Read of an int32 table (page tables, lengths) at a wave-uniform index
// through the constant address space: a scalar load, counted by lgkmcnt, so it
// never waits behind the key streams counted by vmcnt.  The tables are never
// written by the kernels.
__device__ __forceinline__ int32_t load_uniform(const int32_t* base, int64_t idx) {
  typedef __attribute__((address_space(4))) const int32_t* const_i32;
  return ((const_i32)(uintptr_t)base)[uniform(idx)];
}

// Logits of a wave's consecutive pages of one row wait in a per-wave LDS
// buffer and go to memory in runs of up to `cap` pages (16-byte stores), at
// the end of the run or when the buffer is full.  Vector-memory operations
// retire in issue order, so a store issued between two page DMAs makes the
// wait for the later page also wait for that store's acknowledgement;
// buffered, the stores issue after the run's last DMA.
// Cache policy: with the -inf fill on, the logits are streamed out
// (non-temporal, like the fill); with it off -- the fused top-k call, whose
// top-k reads the rows right after -- they are ordinary stores, which the
// top-k then finds in the caches (decode fused call 47.6 -> 46.2 us; the same
// ordinary stores with the fill on cost 4 us).
constexpr int kScoreBufPages = 12;        // decode: 3 KiB of LDS per wave
constexpr int kSharedScoreBufPages = 24;  // prefill: 6 KiB of LDS per wave
typedef __attribute__((address_space(3))) float lds_f32;
typedef __attribute__((address_space(3))) f32x4 lds_f32x4;

struct ScoreBuffer {
  lds_f32* buf;  // [cap][64]
  float* orow;   // output row
  int32_t j0;    // page slot of buf[0]
  int32_t n;     // pages held
  int32_t cap;   // pages the buffer holds
  bool nt;       // non-temporal stores (see the call sites)
};

__device__ __forceinline__ void score_buffer_flush(ScoreBuffer& sb, int lane) {
  // The 16-byte reads below take values other lanes wrote as floats: keep
  // them after those writes (a wave's LDS operations execute in order).
  __asm__ volatile("" ::: "memory");
  const lds_f32x4* src = reinterpret_cast<const lds_f32x4*>(sb.buf);
  f32x4* dst = reinterpret_cast<f32x4*>(sb.orow + (int64_t)sb.j0 * kPage);
  if (sb.nt) {
    for (int32_t i = lane; i < sb.n * (kPage / 4); i += 64) __builtin_nontemporal_store(src[i], dst + i);
  } else {
    for (int32_t i = lane; i < sb.n * (kPage / 4); i += 64) dst[i] = src[i];
  }
  sb.j0 = uniform(sb.j0 + sb.n);
  sb.n = 0;
}

// Logit v of position 64*j + lane (NaN for a page id outside the pool), -inf
// from the row length L on.
__device__ __forceinline__ void score_buffer_put(ScoreBuffer& sb, bool page_valid, float v, int32_t L,
                                                 int lane) {
  const int32_t pos = (sb.j0 + sb.n) * kPage + lane;
  sb.buf[sb.n * kPage + lane] = pos < L ? (page_valid ? v : __builtin_nanf("")) : -INFINITY;
  sb.n = uniform(sb.n + 1);
  if (sb.n == sb.cap) score_buffer_flush(sb, lane);
}

// ---------------------------------------------------------------------------
// rowwise kernel: unit = (row b, WAVES*PPW consecutive page slots); wave w of
// the unit owns PPW slots.
template <int KEY, int PPW, int WAVES>
__global__ __launch_bounds__(64 * WAVES) __attribute__((amdgpu_waves_per_eu(KEY == kFp8 ? 2 : 1, 2))) void rowwise_kernel(Params p, int32_t units_per_row,
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
    const int32_t L = clamp_len(load_uniform(p.sl, b), width);
    const int32_t live = (L + kPage - 1) / kPage;
    const int32_t jl = max(j0, min(jend, live));  // [j0, jl) live, [jl, jend) dead
    float* orow = p.out + (int64_t)b * width * kPage;

    if (j0 < jl) {
      RowQuery rq;
      load_row_query(p, b, lane, rq);
      const int32_t* tab = p.pt + (int64_t)b * p.pt_stride;
      PageKeys<KEY> buf[2];
      int32_t gcur = load_uniform(tab, j0);
      bool okcur = page_ok(gcur, p.pages_lim);
      if (okcur) load_page_global<KEY>(p, gcur, lane, buf[0]);
#pragma unroll
      for (int t = 0; t < PPW; ++t) {
        const int32_t j = j0 + t;
        if (j < jl) {
          int32_t gnxt = 0;
          bool oknxt = false;
          if (t + 1 < PPW && j + 1 < jl) {
            gnxt = load_uniform(tab, j + 1);
            oknxt = page_ok(gnxt, p.pages_lim);
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
    if (p.fill && jl < jend) fill_neg_inf(orow, jl, jend - jl, lane);
  }
}

// ---------------------------------------------------------------------------
// balanced kernel: a fixed grid (about two workgroups per CU, set by the
// scalar arguments and the device) in which every wave takes
//   (1) an equal share of the row-major sequence of all rows' live pages,
//       located from an in-wave prefix sum over the row lengths, and
//   (2) an equal share of the (row, page slot) grid, of which it writes the
//       slots past each row's live pages as -inf.
// Dead slots cost no dispatch and the live work is spread evenly over the
// SIMDs whatever the length mix.  Rows are scanned 64 at a time, so the
// kernel serves batches of up to kBalancedMaxRows rows.
constexpr int32_t kBalancedMaxRows = 1024;

__device__ __forceinline__ int32_t live_pages_of(int32_t L) { return (L + kPage - 1) / kPage; }

__device__ __forceinline__ int64_t wave_sum(int64_t v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d);
  return v;
}

__device__ __forceinline__ int32_t wave_inclusive_scan(int32_t v, int lane) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int32_t t = __shfl_up(v, d);
    if (lane >= d) v += t;
  }
  return v;
}

// ---- fp8 pages streamed HBM -> LDS with global_load_lds_dwordx4 ----------
// Each wave owns two LDS slots of 8448 bytes.  DMA instruction t (0..7) copies
// the contiguous kilobyte of key rows 8t..8t+7 (lane l: row 8t + l/8, 16-byte
// chunk position l%8), so every instruction reads whole 128-byte lines.  The
// slot keeps the rows in order but XOR-swizzles the chunks inside a row:
// position c of row i holds key chunk c ^ (i % 8).  A B fragment then reads row
// i = 16 nb + n, chunks g and 4+g, at positions (g+4h) ^ (n % 8): the eight
// lanes n = 0..7 of a lane group hit distinct banks.  The scales land at
// slot + 8192 (lane l: scale of position l).  Per page: wait for the page's
// DMA group, copy the slot into registers, refill the slot with the page two
// ahead, multiply -- two pages are in flight during every multiply without
// holding them in VGPRs.
constexpr int kSlotBytes = 8448;
constexpr int kDmaOps = 9;  // VMEM instructions per page (8 x 16 B + 1 x 4 B)
// Cache policy of the decode key DMAs: non-temporal.  In decode every key byte
// is read once per launch, so the pages stream past the L2 and the last-level
// cache instead of displacing lines that are reused (queries, tables, the
// output).  Measured on the 4097-wide decode: 41.2 -> 37.2 us.
constexpr int kDmaStreaming = 2;  // the nt bit of the load's cache-policy operand
// s_waitcnt immediate (gfx9 layout: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] |
// vmcnt[5:4] << 14) waiting on vmcnt only.
constexpr int wait_vm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x70 | 0xF00; }

__device__ __forceinline__ void dma_page(const uint8_t* keys, const uint8_t* scales, lds_u8* slot,
                                         int lane) {
  const int rsub = lane >> 3, c = lane & 7;
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const int i = 8 * t + rsub;
    const uint8_t* src = keys + i * kDim + 16 * (c ^ (i & 7));
    __builtin_amdgcn_global_load_lds((global_ptr)src, (lds_ptr)(slot + 1024 * t), 16, 0, kDmaStreaming);
  }
  __builtin_amdgcn_global_load_lds((global_ptr)(scales + 4 * lane), (lds_ptr)(slot + 8192), 4, 0,
                                   kDmaStreaming);
}

// Lane's LDS byte offsets (within a slot) of its two 16-byte B chunks of
// position block 0 (chunks g and 4 + g of row n); block nb adds 2048 nb.
__device__ __forceinline__ uint32_t slot_chunk_offset(int lane, int h) {
  const int n = lane & 15, g = lane >> 4;
  return (uint32_t)(n * kDim + 16 * ((g + 4 * h) ^ (n & 7)));
}

// Wait until at most N vector-memory operations are outstanding (the page's
// DMA group is then complete), then copy the slot into the lane's registers.
// The compiler does not see these LDS reads, so it adds no conservative wait
// for the other slot's DMA, which stays in flight.
template <int N>
__device__ __forceinline__ void read_slot(uint32_t a0, uint32_t a1, uint32_t a4, PageKeys<kFp8>& pk) {
  asm volatile(
      "s_waitcnt vmcnt(%12)\n\t"
      "ds_read_b128 %0, %8\n\t"
      "ds_read_b128 %1, %9\n\t"
      "ds_read_b128 %2, %8 offset:2048\n\t"
      "ds_read_b128 %3, %9 offset:2048\n\t"
      "ds_read_b128 %4, %8 offset:4096\n\t"
      "ds_read_b128 %5, %9 offset:4096\n\t"
      "ds_read_b128 %6, %8 offset:6144\n\t"
      "ds_read_b128 %7, %9 offset:6144\n\t"
      "ds_read_b32 %10, %11\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(pk.v[0][0]), "=&v"(pk.v[0][1]), "=&v"(pk.v[1][0]), "=&v"(pk.v[1][1]),
        "=&v"(pk.v[2][0]), "=&v"(pk.v[2][1]), "=&v"(pk.v[3][0]), "=&v"(pk.v[3][1]), "+v"(a0),
        "+v"(a1), "=&v"(pk.s)
      : "v"(a4), "n"(N)
      : "memory");
}

// Wait until at most `groups` page DMA groups (kDmaOps operations each) are
// outstanding, then read the slot.  groups < NS, so the wait is one of NS
// immediates: one scalar compare per page (a switch over every possible count
// compiled to a branch tree).
template <int NS>
__device__ __forceinline__ void read_slot_after(int groups, uint32_t a0, uint32_t a1, uint32_t a4,
                                                PageKeys<kFp8>& pk) {
  static_assert(NS >= 1 && NS <= 3, "one to three DMA slots");
  if (NS > 2 && groups == 2) read_slot<2 * kDmaOps>(a0, a1, a4, pk);
  else if (NS > 1 && groups == 1) read_slot<kDmaOps>(a0, a1, a4, pk);
  else read_slot<0>(a0, a1, a4, pk);
}

// Boundary of wave wid's share of `total` units when the first h waves weigh
// wa each and the other nw - h waves wb each.
__device__ __forceinline__ int64_t share_bound(int64_t wid, int64_t nw, int64_t h, int64_t wa, int64_t wb,
                                               int64_t total) {
  const int64_t W = min(wid, h) * wa + max((int64_t)0, wid - h) * wb;
  return total * W / (h * wa + (nw - h) * wb);
}

// -inf fill work of one wave: its share [a, z) of the row-major (row, page
// slot) grid, of which only slots past each row's live pages are written.
struct FillCursor {
  int64_t a, z;          // share not yet scanned
  int32_t r, j, jend;    // current row r: dead pages [j, jend) still to write
};

__device__ __forceinline__ FillCursor fill_cursor(const Params& p, int64_t wid, int64_t nw) {
  const int64_t slots = (int64_t)p.rows * p.width;
  FillCursor fc;
  fc.a = uniform(wid * slots / nw);
  fc.z = uniform((wid + 1) * slots / nw);
  fc.r = 0;
  fc.j = 0;
  fc.jend = 0;
  return fc;
}

__device__ __forceinline__ bool fill_next_segment(const Params& p, FillCursor& fc) {
  const int32_t width = p.width;
  while (fc.a < fc.z) {
    const int32_t r = uniform((int32_t)(fc.a / width)), j = uniform((int32_t)(fc.a % width));
    const int32_t jend = uniform((int32_t)min<int64_t>(width, j + (fc.z - fc.a)));
    const int32_t d0 = max(j, live_pages_of(clamp_len(load_uniform(p.sl, r), width)));
    fc.a = uniform(fc.a + (jend - j));
    if (d0 < jend) {
      fc.r = r;
      fc.j = uniform(d0);
      fc.jend = jend;
      return true;
    }
  }
  return false;
}

__device__ __forceinline__ void fill_rest(const Params& p, FillCursor& fc, int lane) {
  do {
    if (fc.j < fc.jend) {
      fill_neg_inf(p.out + (int64_t)fc.r * p.width * kPage, fc.j, fc.jend - fc.j, lane);
      fc.j = fc.jend;
    }
  } while (fill_next_segment(p, fc));
}

// bf16 page from its LDS slot into the lane's B fragments (rows of 256 B,
// 16-byte chunk c of row i at chunk c ^ (i % 16)): lane (g, n) reads chunks
// 2g, 2g+1, 8+2g, 9+2g of rows n, 16+n, 32+n, 48+n.  Waits
// until at most N vector-memory operations are outstanding first (the
// compiler does not see these reads, so it adds no wait for the DMAs still in
// flight into other slots).
template <int N>
__device__ __forceinline__ void read_slot_bf16(uint32_t sb, int lane, PageKeys<kBf16>& pk) {
  const int n = lane & 15, g = lane >> 4;
  uint32_t a[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) a[v] = sb + (uint32_t)(n * 256 + 16 * ((8 * (v >> 1) + 2 * g + (v & 1)) ^ n));
  asm volatile(
      "s_waitcnt vmcnt(%20)\n\t"
      "ds_read_b128 %0, %16\n\t"
      "ds_read_b128 %1, %17\n\t"
      "ds_read_b128 %2, %18\n\t"
      "ds_read_b128 %3, %19\n\t"
      "ds_read_b128 %4, %16 offset:4096\n\t"
      "ds_read_b128 %5, %17 offset:4096\n\t"
      "ds_read_b128 %6, %18 offset:4096\n\t"
      "ds_read_b128 %7, %19 offset:4096\n\t"
      "ds_read_b128 %8, %16 offset:8192\n\t"
      "ds_read_b128 %9, %17 offset:8192\n\t"
      "ds_read_b128 %10, %18 offset:8192\n\t"
      "ds_read_b128 %11, %19 offset:8192\n\t"
      "ds_read_b128 %12, %16 offset:12288\n\t"
      "ds_read_b128 %13, %17 offset:12288\n\t"
      "ds_read_b128 %14, %18 offset:12288\n\t"
      "ds_read_b128 %15, %19 offset:12288\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(pk.v[0][0]), "=&v"(pk.v[0][1]), "=&v"(pk.v[0][2]), "=&v"(pk.v[0][3]),
        "=&v"(pk.v[1][0]), "=&v"(pk.v[1][1]), "=&v"(pk.v[1][2]), "=&v"(pk.v[1][3]),
        "=&v"(pk.v[2][0]), "=&v"(pk.v[2][1]), "=&v"(pk.v[2][2]), "=&v"(pk.v[2][3]),
        "=&v"(pk.v[3][0]), "=&v"(pk.v[3][1]), "=&v"(pk.v[3][2]), "=&v"(pk.v[3][3])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "n"(N)
      : "memory");
  pk.s = 1.0f;
}

// One bf16 page into a wave's 16 KiB slot by DMA: 16 operations of 1 KiB
// (4 rows of 256 B each), the chunk swizzle applied on the source side since
// the DMA destination is lane-linear.
constexpr int kBf16SlotBytes = 16384;
constexpr int kBf16DmaOps = 16;
__device__ __forceinline__ void dma_page_bf16(const uint8_t* keys, lds_u8* slot, int lane) {
  const int r = lane >> 4, c = lane & 15;
#pragma unroll
  for (int t = 0; t < kBf16DmaOps; ++t) {
    const int i = 4 * t + r;
    __builtin_amdgcn_global_load_lds((global_ptr)(keys + i * 256 + 16 * (c ^ (i & 15))),
                                     (lds_ptr)(slot + 1024 * t), 16, 0, kDmaStreaming);
  }
}

// Live bf16 pages [ja, jb) of row b through the wave's one LDS slot: page t+1
// is requested as soon as page t is in registers, and flies while page t is
// multiplied.
__device__ __forceinline__ void row_pages_dma_bf16(const Params& p, int32_t b, int32_t ja, int32_t jb,
                                                   int32_t L, int lane, lds_u8* slot, lds_f32* sbuf) {
  RowQuery rq;
  load_row_query(p, b, lane, rq);
  const int32_t* tab = p.pt + (int64_t)b * p.pt_stride;
  ScoreBuffer out{sbuf, p.out + (int64_t)b * p.width * kPage, ja, 0, kScoreBufPages, p.fill != 0};
  // A page id outside the pool is never dereferenced: its DMA reads the row's
  // own query (16 KiB, always valid memory) and its logits become NaN.
  const uint8_t* safe = p.q + (int64_t)b * (kHeads * kDim * 2);
  const int32_t J = jb - ja;
  const int32_t g0 = load_uniform(tab, ja);
  bool ok = page_ok(g0, p.pages_lim);
  dma_page_bf16(ok ? p.kv + (int64_t)g0 * p.kv_stride : safe, slot, lane);
  // The query was requested before the DMA: wait for it here with the DMA in
  // flight, so that no conservative wait lands in the page loop.
  __builtin_amdgcn_s_waitcnt(wait_vm(kBf16DmaOps));
  const uint32_t sb = (uint32_t)(uintptr_t)slot;
  int32_t g_ahead = (1 < J) ? load_uniform(tab, ja + 1) : -1;
  for (int32_t tt = 0; tt < J; ++tt) {
    // Page tt's DMA is the newest operation (apart from the stores of a
    // buffer flush, which this wait then also covers).
    PageKeys<kBf16> pk;
    read_slot_bf16<0>(sb, lane, pk);
    const bool cur_ok = ok;
    const int32_t g = g_ahead;
    g_ahead = (tt + 2 < J) ? load_uniform(tab, ja + tt + 2) : -1;
    if (tt + 1 < J) {
      ok = page_ok(g, p.pages_lim);
      dma_page_bf16(ok ? p.kv + (int64_t)g * p.kv_stride : safe, slot, lane);
    }
    score_buffer_put(out, cur_ok, cur_ok ? score_page<kBf16>(rq, pk, lane) : 0.f, L, lane);
  }
  score_buffer_flush(out, lane);
}

// Live pages [ja, jb) of row b through the wave's NS LDS slots: NS pages are
// in flight while one is multiplied.
template <int NS>
__device__ __forceinline__ void row_pages_dma(const Params& p, int32_t b, int32_t ja, int32_t jb,
                                              int32_t L, int lane, lds_u8* slots, lds_f32* sbuf) {
  RowQuery rq;
  load_row_query(p, b, lane, rq);
  const int32_t* tab = p.pt + (int64_t)b * p.pt_stride;
  ScoreBuffer out{sbuf, p.out + (int64_t)b * p.width * kPage, ja, 0, kScoreBufPages, p.fill != 0};
  // A page id outside the pool is never dereferenced: its DMA reads the row's
  // own query bytes instead (always valid memory) and its logits become NaN.
  const uint8_t* safe = p.q + (int64_t)b * (kHeads * kDim * 2);
  const int32_t J = jb - ja;
  bool ok[NS];
#pragma unroll
  for (int t = 0; t < NS; ++t) {
    // (a short segment still issues NS groups, the extra ones from the query
    // row, so that the prologue always holds NS groups)
    const int32_t g = t < J ? load_uniform(tab, ja + t) : -1;
    ok[t] = page_ok(g, p.pages_lim);
    const uint8_t* keys = ok[t] ? p.kv + (int64_t)g * p.kv_stride : safe;
    const uint8_t* sc = ok[t] ? p.ks + (int64_t)g * p.ks_stride : safe + 8192;
    dma_page(keys, sc, slots + t * kSlotBytes, lane);
  }
  // The query and weights were requested before the NS DMA groups (9
  // operations each): wait for them here with the groups still in flight, so
  // that no conservative wait for them lands inside the page loop.
  __builtin_amdgcn_s_waitcnt(wait_vm(kDmaOps * NS));
  const uint32_t base = (uint32_t)(uintptr_t)slots;
  const uint32_t off0 = slot_chunk_offset(lane, 0), off1 = slot_chunk_offset(lane, 1);
  // page id of the group issued next; read one iteration ahead so the scalar
  // load never stalls the DMA issue
  int32_t g_ahead = (NS < J) ? load_uniform(tab, ja + NS) : -1;
  for (int32_t t = 0; t < J; t += NS) {
#pragma unroll
    for (int u = 0; u < NS; ++u) {
      const int32_t tt = t + u;
      if (tt < J) {
        lds_u8* slot = slots + u * kSlotBytes;
        const uint32_t a0 = base + u * kSlotBytes + off0;
        const uint32_t a1 = base + u * kSlotBytes + off1;
        const uint32_t a4 = base + u * kSlotBytes + 8192 + 4 * lane;
        // Operations issued after page tt's DMA group: the groups of the
        // pages after it -- prologue groups for tt < NS, plus one group per
        // iteration i in [tt-NS+1, tt-1] with i+NS < J.  (The stores of a
        // buffer flush are not counted: the wait then also covers them.)
        const int32_t lo = max(0, tt - NS + 1), hi = min(tt - 1, J - NS - 1);
        const int32_t groups = (tt < NS ? NS - 1 - tt : 0) + max(0, hi - lo + 1);
        PageKeys<kFp8> pk;
        read_slot_after<NS>(uniform(groups), a0, a1, a4, pk);
        const bool cur_ok = ok[u];
        const int32_t g = g_ahead;
        g_ahead = (tt + NS + 1 < J) ? load_uniform(tab, ja + tt + NS + 1) : -1;
        if (tt + NS < J) {
          ok[u] = page_ok(g, p.pages_lim);
          const uint8_t* keys = ok[u] ? p.kv + (int64_t)g * p.kv_stride : safe;
          const uint8_t* sc = ok[u] ? p.ks + (int64_t)g * p.ks_stride : safe + 8192;
          dma_page(keys, sc, slot, lane);
        }
        score_buffer_put(out, cur_ok, cur_ok ? score_page<kFp8>(rq, pk, lane) : 0.f, L, lane);
      }
    }
  }
  score_buffer_flush(out, lane);
}

// Live pages [s, e) of the row-major sequence of all rows' live pages.
template <int KEY, int NS>
__device__ __forceinline__ void live_share(const Params& p, int64_t s, int64_t e, int lane,
                                           lds_u8* my_slots) {
  const int32_t rows = p.rows, width = p.width;

  // Row holding live page s and the number of live pages before that row.
  int32_t r = 0;
  int64_t excl = 0;
  for (int32_t r0 = 0; r0 < rows; r0 += 64) {
    const int32_t rr = r0 + lane;
    const int32_t lp = rr < rows ? live_pages_of(clamp_len(p.sl[rr], width)) : 0;
    const int32_t incl = wave_inclusive_scan(lp, lane);
    const int32_t csum = __builtin_amdgcn_readlane(incl, 63);
    if (excl + csum > s) {
      const uint64_t m = __ballot(excl + incl > s);
      const int first = uniform((int32_t)__builtin_ctzll(m));
      r = uniform(r0 + first);
      excl = uniform(excl + __builtin_amdgcn_readlane(incl - lp, first));
      break;
    }
    excl = uniform(excl + csum);
  }

  int64_t pos = s;
  while (pos < e) {
    const int32_t L = clamp_len(load_uniform(p.sl, r), width);
    const int32_t lp = live_pages_of(L);
    const int32_t ja = (int32_t)(pos - excl);
    const int32_t jb = (int32_t)min<int64_t>(lp, e - excl);
    if (ja < jb) {
      if constexpr (KEY == kFp8)
        row_pages_dma<NS>(p, r, ja, jb, L, lane, my_slots, (lds_f32*)(my_slots + NS * kSlotBytes));
      else
        row_pages_dma_bf16(p, r, ja, jb, L, lane, my_slots, (lds_f32*)(my_slots + kBf16SlotBytes));
    }
    pos = uniform(excl + jb);
    excl = uniform(excl + lp);
    r = uniform(r + 1);
  }
}

template <int KEY, int WAVES, int NS>
__global__ __launch_bounds__(64 * WAVES) __attribute__((amdgpu_waves_per_eu(2, 2))) void balanced_kernel(Params p) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t nw = (int64_t)gridDim.x * WAVES;
  const int64_t wid = (int64_t)blockIdx.x * WAVES + wave;
  const int32_t rows = p.rows, width = p.width;
  // per wave: the DMA slots, then the logits buffer
  constexpr int kWaveLds = ((KEY == kFp8) ? NS * kSlotBytes : kBf16SlotBytes) + kScoreBufPages * kPage * 4;
  __shared__ __attribute__((aligned(16))) uint8_t lds_raw[WAVES * kWaveLds];
  lds_u8* dma_slots = (lds_u8*)lds_raw;

  // (1) total live pages, then this wave's range [s, e) of them.
  int64_t acc = 0;
  for (int32_t r0 = 0; r0 < rows; r0 += 64) {
    const int32_t r = r0 + lane;
    if (r < rows) acc += live_pages_of(clamp_len(p.sl[r], width));
  }
  const int64_t total = uniform(wave_sum(acc));
  // Waves of the grid's first half write their -inf share before their pages;
  // those of the second half start on the pages at once and write their share
  // at the end.  The first half's live share is weighted up so that both
  // halves finish together: 2:1 when the -inf bytes are at least a quarter of
  // the live key bytes, 4:1 when they are fewer (measured on one box: the
  // 4097-wide decode 37.7 us at 3:2, 36.8 at 2:1, 40.1 at 3:1; its 513-wide
  // control 32.9 at 3:2, 31.7 at 4:1; the 128-wide decode 16.2 at 3:2, 15.8
  // at 4:1).
  const int64_t h = (int64_t)WAVES * ((gridDim.x + 1) / 2);  // first-half waves
  const int64_t dead = (int64_t)rows * width - total;          // page slots written -inf
  constexpr int64_t kLivePageBytes = (KEY == kFp8) ? kSlotBytes : kBf16SlotBytes;
  const bool big_fill = 4 * dead * (kPage * 4) >= total * kLivePageBytes;
  const int64_t wa = p.fill ? (big_fill ? 2 : 4) : 1, wb = 1;  // no -inf share: even split
  const int64_t s = share_bound(wid, nw, h, wa, wb, total), e = share_bound(wid + 1, nw, h, wa, wb, total);
  // (2) the -inf share: an equal share of the page slots.  Workgroups of the
  // grid's second half score first and write -inf after, those of the first
  // half the reverse.  The dispatcher gives every CU one workgroup of each
  // half, so each SIMD keeps one wave on the MFMA/VALU-heavy scoring while the
  // other streams stores, and HBM sees reads and writes together.
  FillCursor fc = fill_cursor(p, wid, nw);
  if (!p.fill) fc.z = fc.a;  // nothing to write past the live pages
  if (2 * blockIdx.x >= gridDim.x) {
    if (s < e) live_share<KEY, NS>(p, s, e, lane, dma_slots + wave * kWaveLds);
    fill_rest(p, fc, lane);
  } else {
    fill_rest(p, fc, lane);
    if (s < e) live_share<KEY, NS>(p, s, e, lane, dma_slots + wave * kWaveLds);
  }
}

// ---------------------------------------------------------------------------
// shared kernel: rows share page tables (one, or one per request through a
// row -> table map).  Unit = (block of 4 rows, chunk of `chunk` page slots);
// wave w scores row 4*rb + w.  Pages go through LDS.
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

// One page of the shared table through LDS by DMA: each of the kSharedRows
// waves copies 64/kSharedRows of the key rows (16 B per lane, the XOR swizzle
// of LdsPage applied on the source side since the DMA destination is
// lane-linear); wave 0 also copies the 256 scale bytes (fp8).  The wave's
// operation count per page is shared_dma_ops(wave).
constexpr int kSharedRowsPerWave = kPage / kSharedRows;
template <int KEY>
constexpr int32_t shared_dma_ops(int wave) {
  return (KEY == kBf16) ? kSharedRowsPerWave / 4 : kSharedRowsPerWave / 8 + (wave == 0 ? 1 : 0);
}
template <int KEY>
__device__ __forceinline__ void shared_dma_page(const uint8_t* page, const uint8_t* scales, lds_u8* slot,
                                                int wave, int lane) {
  // The lane's source offsets are 32-bit and the page address wave-uniform,
  // so each DMA takes the scalar base + vector offset form (no 64-bit
  // address arithmetic per page).
  const int r0 = kSharedRowsPerWave * wave;
  if constexpr (KEY == kBf16) {
    // rows of 256 B, 4 per DMA
#pragma unroll
    for (int t = 0; t < kSharedRowsPerWave / 4; ++t) {
      const int i = r0 + 4 * t + (lane >> 4), c = lane & 15;
      const uint32_t off = (uint32_t)(i * 256 + 16 * (c ^ (i & 15)));
      __builtin_amdgcn_global_load_lds((global_ptr)(page + off), (lds_ptr)(slot + (r0 + 4 * t) * 256), 16, 0, 0);
    }
  } else {
    // rows of 128 B, 8 per DMA
#pragma unroll
    for (int t = 0; t < kSharedRowsPerWave / 8; ++t) {
      const int i = r0 + 8 * t + (lane >> 3), c = lane & 7;
      const uint32_t off = (uint32_t)(i * 128 + 16 * (c ^ (i & 7)));
      __builtin_amdgcn_global_load_lds((global_ptr)(page + off), (lds_ptr)(slot + (r0 + 8 * t) * 128), 16, 0, 0);
    }
    if (wave == 0)
      __builtin_amdgcn_global_load_lds((global_ptr)(scales + 4 * lane), (lds_ptr)(slot + 8192), 4, 0, 0);
  }
}


// Wait until at most n (<= 11) vector-memory operations are outstanding.
__device__ __forceinline__ void wait_vm_n(int32_t n) {
  switch (n) {
    case 0: __builtin_amdgcn_s_waitcnt(wait_vm(0)); break;
    case 1: __builtin_amdgcn_s_waitcnt(wait_vm(1)); break;
    case 2: __builtin_amdgcn_s_waitcnt(wait_vm(2)); break;
    case 3: __builtin_amdgcn_s_waitcnt(wait_vm(3)); break;
    case 4: __builtin_amdgcn_s_waitcnt(wait_vm(4)); break;
    case 5: __builtin_amdgcn_s_waitcnt(wait_vm(5)); break;
    case 6: __builtin_amdgcn_s_waitcnt(wait_vm(6)); break;
    case 7: __builtin_amdgcn_s_waitcnt(wait_vm(7)); break;
    case 8: __builtin_amdgcn_s_waitcnt(wait_vm(8)); break;
    case 9: __builtin_amdgcn_s_waitcnt(wait_vm(9)); break;
    case 10: __builtin_amdgcn_s_waitcnt(wait_vm(10)); break;
    case 11: __builtin_amdgcn_s_waitcnt(wait_vm(11)); break;
    default: __builtin_amdgcn_s_waitcnt(wait_vm(0)); break;
  }
}

// Page of a slot whose DMA is complete, through LDS loads the compiler sees
// (same fragment layout as read_slot / read_slot_bf16).  Used where no DMA is
// in flight when the page is read, so the compiler adds no wait for one; it
// waits for each fragment only where an MFMA first needs it, and the loads
// overlap the next page's DMA issue.
typedef __attribute__((address_space(3))) const u32x4 lds_u32x4c;
typedef __attribute__((address_space(3))) const float lds_f32c;
// The lane's byte offsets in a slot of its fragments of position block 0 (a
// block adds 4096 bytes for bf16, 2048 for fp8) and of its scale: computed once,
// so that a page costs one add per offset and the block steps are immediate
// offsets of the LDS loads.
struct SharedSlotOffsets {
  uint32_t o[4];
};
template <int KEY>
__device__ __forceinline__ SharedSlotOffsets shared_slot_offsets(int lane) {
  SharedSlotOffsets so;
  const int n = lane & 15, g = lane >> 4;
  if constexpr (KEY == kBf16) {
#pragma unroll
    for (int v = 0; v < 4; ++v) so.o[v] = (uint32_t)(n * 256 + 16 * ((8 * (v >> 1) + 2 * g + (v & 1)) ^ n));
  } else {
    so.o[0] = slot_chunk_offset(lane, 0);
    so.o[1] = slot_chunk_offset(lane, 1);
    so.o[2] = (uint32_t)(8192 + 4 * lane);
    so.o[3] = 0u;
  }
  return so;
}

template <int KEY>
__device__ __forceinline__ void read_shared_slot(uint32_t sb, const SharedSlotOffsets& so, PageKeys<KEY>& pk) {
  if constexpr (KEY == kBf16) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      lds_u32x4c* src = (lds_u32x4c*)(size_t)(sb + so.o[v]);
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) pk.v[nb][v] = src[256 * nb];
    }
    pk.s = 1.0f;
  } else {
    lds_u32x4c* s0 = (lds_u32x4c*)(size_t)(sb + so.o[0]);
    lds_u32x4c* s1 = (lds_u32x4c*)(size_t)(sb + so.o[1]);
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      pk.v[nb][0] = s0[128 * nb];
      pk.v[nb][1] = s1[128 * nb];
    }
    pk.s = *(lds_f32c*)(size_t)(sb + so.o[2]);
  }
}

// Rows sharing page tables (page_table_row_stride == 0: the query tokens of
// one prefill request; MULTI: rows mapped to request tables by p.rt).  Unit =
// (block of 4 rows, chunk of `chunk` page slots[, table group]); wave w scores
// row 4*rb + w.  Each page is copied once into LDS by DMA -- kSharedSlots
// slots, pages kSharedSlots-1 ahead in flight -- and the waves whose rows use
// the unit's table multiply it against their own row's query; one barrier per
// page.
constexpr int kSharedSlots = 2;  // (read_shared_slot relies on no DMA in flight at the read)

template <int KEY, bool MULTI>
__global__ __launch_bounds__(64 * kSharedRows) __attribute__((amdgpu_waves_per_eu(2, 2))) void shared_kernel(Params p, int32_t row_blocks,
                                                                  int32_t chunk, int32_t chunks,
                                                                  int32_t rb_per_xcd,
                                                                  int64_t total_slots, int32_t paired) {
  constexpr int NS = kSharedSlots;
  constexpr int kSlot = (KEY == kFp8) ? kSlotBytes : 16384;
  // page slots, then one logits buffer per wave
  __shared__ __attribute__((aligned(16))) uint8_t lds_raw[NS * kSlot + kSharedRows * kSharedScoreBufPages * kPage * 4];
  lds_u8* slots = (lds_u8*)lds_raw;
  const uint32_t base = (uint32_t)(uintptr_t)slots;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int32_t ops = shared_dma_ops<KEY>(wave);  // DMA operations per page
  const SharedSlotOffsets so = shared_slot_offsets<KEY>(lane);
  lds_f32* sbuf = (lds_f32*)(lds_raw + NS * kSlot + wave * kSharedScoreBufPages * kPage * 4);
  const int32_t width = p.width;

  // MULTI: four groups per (row block, chunk) unit, the group index slowest
  // (total_slots is a multiple of 8, so a unit keeps its XCD in every group).
  const int64_t units = MULTI ? 4 * total_slots : total_slots;
  for (int64_t us = blockIdx.x; us < units; us += gridDim.x) {
    const int gi = MULTI ? (int)(us / total_slots) : 0;
    const int64_t slot = MULTI ? us % total_slots : us;
    // Workgroup ids are dealt to the 8 XCDs round-robin; keep all chunks of a
    // row block on one XCD (its query rows stay in that L2) and hand out row
    // blocks longest-first (largest index first).
    int32_t rb, c;
    if (!MULTI && paired) {
      // Whole-table units, grid of resident workgroups: passes of gridDim.x
      // row blocks, longest-first in even passes and shortest-first in odd
      // ones, so that workgroup b takes blocks k = b, 2G-1-b, ... and every
      // workgroup gets about the same number of pages of the causal triangle.
      const int64_t G = gridDim.x, pass = slot / G, b = slot % G;
      const int64_t k = pass * G + ((pass & 1) ? G - 1 - b : b);
      if (k >= row_blocks) continue;
      rb = (int32_t)(row_blocks - 1 - k);
      c = 0;
    } else {
      const int32_t xcd = (int32_t)(slot % 8);
      const int64_t seq = slot / 8;
      const int32_t rb_local = (int32_t)(seq / chunks);
      c = (int32_t)(seq % chunks);
      const int32_t rb_rev = rb_local * 8 + xcd;
      if (rb_local >= rb_per_xcd || rb_rev >= row_blocks) continue;
      rb = row_blocks - 1 - rb_rev;
    }

    const int32_t j0 = c * chunk;
    const int32_t jend = min(j0 + chunk, width);
    const int32_t b = rb * kSharedRows + wave;
    float* orow = p.out + (int64_t)b * width * kPage;

    // Table of each of the block's rows.  Rows of one request share a table;
    // a block that straddles requests is scored once per distinct table (the
    // unit's group gi: the table of the block's row gi, if no earlier row of
    // the block has it), with only that table's rows scoring -- the other
    // waves still copy their part of each page and meet every barrier.
    // Table indices are scalar loads, re-read where needed; p.rt is read only
    // at row indices below p.rows (the last block may hold fewer than 4 rows).
    auto table_of = [&](int32_t br) -> int32_t { return load_uniform(p.rt, br); };
    if (MULTI && rb * kSharedRows + gi >= p.rows) continue;
    const int32_t T = MULTI ? table_of(rb * kSharedRows + gi) : 0;
    if constexpr (MULTI) {
      bool lead = true;
      for (int r = 0; r < gi; ++r) lead = lead && table_of(rb * kSharedRows + r) != T;
      if (!lead) continue;
    }
    {
      // An index outside the tables reads no table: its rows score NaN.
      const bool table_ok = !MULTI || (T >= 0 && T < p.num_tables);
      const int32_t* tab = MULTI ? p.pt + (int64_t)(table_ok ? T : 0) * p.pt_stride : p.pt;
      const bool row_ok = b < p.rows && (!MULTI || table_of(b) == T);

      // Longest live prefix over the group's rows decides which pages to load.
      int32_t Lmax = 0;
#pragma unroll
      for (int r = 0; r < kSharedRows; ++r) {
        const int32_t br = rb * kSharedRows + r;
        if (br < p.rows && (!MULTI || table_of(br) == T)) Lmax = max(Lmax, clamp_len(load_uniform(p.sl, br), width));
      }
      const int32_t L = row_ok ? clamp_len(load_uniform(p.sl, b), width) : 0;
      const int32_t live_w = (L + kPage - 1) / kPage;
      const int32_t jl = max(j0, min(jend, (Lmax + kPage - 1) / kPage));  // pages any row needs

      if (j0 < jl) {
        RowQuery rq;
        if (row_ok && j0 < live_w) load_row_query(p, b, lane, rq);
        // A page id outside the pool -- or a page past jl, issued only to keep
        // the operation count per iteration constant -- is copied from the
        // query buffer instead (always valid memory, at least 16 KiB).
        // Page id whose DMA each slot holds (scalar selects on the slot index,
        // no per-page vector work).
        int32_t slot_id[NS];
#pragma unroll
        for (int v = 0; v < NS; ++v) slot_id[v] = -1;
        // Table entry of page j0 + t (-1 past the pages any row needs).  Read
        // one iteration before its DMA is issued, so that the scalar load's
        // latency is not on the page loop's path.
        auto table_entry = [&](int32_t t) -> int32_t {
          const int32_t j = j0 + t;
          return (j < jl && table_ok) ? load_uniform(tab, j) : -1;
        };
        auto issue = [&](int32_t t, int32_t g) {
          const bool ok = page_ok(g, p.pages_lim);
          const int u = t % NS;
#pragma unroll
          for (int v = 0; v < NS; ++v)
            if (v == u) slot_id[v] = g;
          const uint8_t* page = ok ? p.kv + (int64_t)g * p.kv_stride : p.q;
          const uint8_t* sc = (KEY == kFp8 && ok) ? p.ks + (int64_t)g * p.ks_stride : p.q + 8192;
          shared_dma_page<KEY>(page, sc, slots + u * kSlot, wave, lane);
        };
#pragma unroll
        for (int t = 0; t < NS - 1; ++t) issue(t, table_entry(t));
        int32_t g_next = table_entry(NS - 1);
        // The query was requested before these DMAs: wait for it here with them
        // still in flight, so that no conservative wait lands in the page loop.
        // (Wave 0 of the fp8 kernel has one more operation per page; waiting on
        // the smaller count there costs it a part of page 0, no more.)
        __builtin_amdgcn_s_waitcnt(wait_vm((NS - 1) * shared_dma_ops<KEY>(1)));
        ScoreBuffer logits{sbuf, orow, j0, 0, kSharedScoreBufPages, p.fill != 0};
        for (int32_t t = 0; j0 + t < jl; ++t) {
          const int32_t j = j0 + t;
          const int u = t % NS;
          // Operations issued after page t's DMA: the pages of the (NS-2) later
          // DMAs (the stores of a buffer flush are not counted: the wait then
          // also covers them).
          const int32_t n_after = uniform((NS - 2) * ops);
          // Every wave waits for its own part of page t; the barrier then makes
          // the whole page visible -- and also guarantees that every wave is
          // done with slot (t-1) % NS, which the next DMA overwrites (the
          // release fence waits for this wave's reads of it).  The acquire
          // fence keeps the page's LDS loads after the barrier.  With two
          // slots no DMA is in flight here (n_after is 0).
          wait_vm_n(n_after);
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
          __builtin_amdgcn_s_barrier();
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
          PageKeys<KEY> pk;
          if (row_ok && j < live_w) read_shared_slot<KEY>(base + (uint32_t)(u * kSlot), so, pk);
          issue(t + NS - 1, g_next);
          g_next = table_entry(t + NS);
          if (row_ok) {  // (a page past this row's length is all -inf)
            int32_t gu = slot_id[0];
#pragma unroll
            for (int v = 1; v < NS; ++v)
              if (v == u) gu = slot_id[v];
            const bool valid = page_ok(gu, p.pages_lim);
            score_buffer_put(logits, valid, (j < live_w && valid) ? score_page<KEY>(rq, pk, lane) : 0.f,
                             L, lane);
          }
        }
        if (row_ok) score_buffer_flush(logits, lane);
        __builtin_amdgcn_s_waitcnt(wait_vm(0));
        __builtin_amdgcn_s_barrier();  // LDS is reused by this workgroup's next unit
      }
      if (row_ok && p.fill && jl < jend) fill_neg_inf(orow, jl, jend - jl, lane);
    }
  }
}

// ---------------------------------------------------------------------------
// Paged key store: the write side of the cache block.  Key t (128 values)
// goes to flat slot slots[t] = 64*page + i.  16 lanes per key, 8 values
// (16 bytes of bf16) per lane, 4 keys per wave per step.  fp8: per key
// scale = amax/448 (1 for an all-zero key) and the e4m3fn codes of the
// quotient clamped to +-448, every step in float32; bf16: a copy.
constexpr int kStoreWaves = 4;
constexpr int kStoreUnroll = 4;  // groups of 4 keys per wave and iteration

template <int KEY>
__global__ __launch_bounds__(64 * kStoreWaves) void store_keys_kernel(const uint8_t* keys, const int64_t* slots,
                                                                     int64_t n, uint8_t* kv, uint8_t* ks,
                                                                     int64_t num_pages, int64_t kv_stride,
                                                                     int64_t ks_stride) {
  const int lane = threadIdx.x & 63;
  const int c = lane & 15;  // 16-byte part of the key
  const int64_t wave_id = (int64_t)blockIdx.x * kStoreWaves + (threadIdx.x >> 6);
  const int64_t step = (int64_t)gridDim.x * kStoreWaves * 4 * kStoreUnroll;
  // kStoreUnroll groups of 4 keys per iteration: all their loads are issued
  // before the first group is quantised, so a wave has that many in flight.
  for (int64_t base = wave_id * 4 * kStoreUnroll; base < n; base += step) {
    int64_t slot[kStoreUnroll];
    u32x4 raw[kStoreUnroll];
#pragma unroll
    for (int u = 0; u < kStoreUnroll; ++u) {
      const int64_t t = base + 4 * u + (lane >> 4);
      slot[u] = -1;
      raw[u] = (u32x4){0u, 0u, 0u, 0u};
      if (t < n) {
        slot[u] = slots[t];
        raw[u] = *reinterpret_cast<const u32x4*>(keys + t * (kDim * 2) + 16 * c);
      }
    }
#pragma unroll
    for (int u = 0; u < kStoreUnroll; ++u) {
      const bool ok = slot[u] >= 0 && slot[u] < num_pages * kPage;  // (slot -1 past n)
      const int64_t g = ok ? slot[u] / kPage : 0;
      const int i = ok ? (int)(slot[u] % kPage) : 0;
      if constexpr (KEY == kBf16) {
        if (ok) *reinterpret_cast<u32x4*>(kv + g * kv_stride + (int64_t)i * (kDim * 2) + 16 * c) = raw[u];
      } else {
        float v[8];
        const uint32_t w[4] = {raw[u].x, raw[u].y, raw[u].z, raw[u].w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          v[2 * k] = __builtin_bit_cast(float, w[k] << 16);
          v[2 * k + 1] = __builtin_bit_cast(float, w[k] & 0xffff0000u);
        }
        float m = 0.0f;
#pragma unroll
        for (int k = 0; k < 8; ++k) m = fmaxf(m, fabsf(v[k]));
        // amax over the key's 16 lanes (the xor masks stay inside a 16-lane group)
        m = fmaxf(m, __shfl_xor(m, 8));
        m = fmaxf(m, __shfl_xor(m, 4));
        m = fmaxf(m, __shfl_xor(m, 2));
        m = fmaxf(m, __shfl_xor(m, 1));
        const float scale = m > 0.0f ? m / 448.0f : 1.0f;
        // Quotients v / scale as the float32 division rounds them, with one
        // division per key: y = 1/scale (correctly rounded), q0 = v*y, and one
        // fma residual step q = q0 + (v - scale*q0)*y, which gives the correctly
        // rounded quotient in round-to-nearest away from underflow (Markstein's
        // correction with a correctly rounded reciprocal).  A zero quotient may
        // come out +0 for v = -0, so the code's sign is taken from v below.
        // Quotients under 2^-11 (code 0) may differ in their last bits when the
        // residual underflows; a scale outside [2^-60, 2^100] (tiny or infinite
        // keys) takes the division.  Checked on the host against division for
        // 1.4e9 bf16 values and scales: no code differs.
        float q[8];
        if (__ballot(!(scale >= 0x1p-60f && scale <= 0x1p100f)) == 0) {
          const float y = 1.0f / scale;
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            const float q0 = v[k] * y;
            q[k] = fmaf(fmaf(-scale, q0, v[k]), y, q0);
          }
        } else {
#pragma unroll
          for (int k = 0; k < 8; ++k) q[k] = v[k] / scale;
        }
        uint32_t out[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          float y[4];
#pragma unroll
          for (int k = 0; k < 4; ++k) y[k] = fminf(fmaxf(q[4 * h + k], -448.0f), 448.0f);
          uint32_t code = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
          code = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], (int)code, true);
          // a value that rounds to zero keeps its sign (0x80 for -0); the sign
          // of v is the sign of v / scale
          uint32_t sign = 0u;
#pragma unroll
          for (int k = 0; k < 4; ++k) sign |= (__builtin_bit_cast(uint32_t, v[4 * h + k]) >> 31) << (8 * k + 7);
          out[h] = code | sign;
        }
        if (ok) {
          *reinterpret_cast<uint2*>(kv + g * kv_stride + (int64_t)i * kDim + 8 * c) = make_uint2(out[0], out[1]);
          if (c == 0) *reinterpret_cast<float*>(ks + g * ks_stride + 4 * i) = scale;
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Top-k over logits rows.  Candidates of row b are positions p < L_b; the
// order is larger value first, equal values (+0 and -0 are equal) by lower
// position, NaN after every number; the first min(k, L) candidates are
// written in ascending position order, then -1 (value -inf) up to k.
//
// One workgroup per row.  A radix select over 32-bit order keys (digits of
// 11, 11 and 10 bits, most significant first) finds the key T of the k-th
// candidate and how many candidates with key T are taken (`need`; every key
// above T is taken).  An order-preserving compaction then writes candidate p
// to slot (#keys > T before p) + min(#keys == T before p, need): each wave
// owns a contiguous segment of the row, 4 positions per lane and 256 per
// step, counts its candidates per lane, and emits them after a prefix over
// the waves' counts and one wave scan per step.
// A row of at most CAP candidates is read from memory once, by the first
// pass, which stages each value's order key in LDS; later passes read the
// keys there, and a selected value is its key inverted (read again from the
// row for NaN and zeros only in a row that holds a NaN or a -0).  After the first digit, one
// sweep over the waves' segments counts each segment's keys above that digit
// and lists the positions of the keys in it (at most CAND of them).  The
// later digits scan the list instead of the row, and the segments' counts
// above and at the final key come from those counts and the list, so the
// compaction reads the row only once more.  A longer row is re-read from
// memory by each pass.  A staged row that takes at most a quarter of its
// keys (1024-thread kernel) goes another way after the first digit: each
// thread keeps bit words of its own 32 positions (topk_row_owned).
constexpr int kTopkBins = 2048;

// Per-thread bit words (sparse rows) in the 1024-thread kernel only: the rows
// of the 256-thread kernel are at most 6,144 long and dense at the usual k,
// and the same path there (24 positions per thread) measured 43.5 us against
// 35.1 on the 4096-row prefill top-k.
template <int THREADS>
constexpr bool kTopkBitmap = THREADS >= 1024;

template <int THREADS, int CAP, int CAND>
struct TopkShared {
  static constexpr int kThreads = THREADS;
  uint32_t vals[CAP];    // the staged row's order keys, when it fits
  uint32_t cand[CAND];   // positions of the keys sharing the first digit
  uint32_t hist[kTopkBins];
  uint32_t wave_gt[THREADS / 64], wave_eq[THREADS / 64];
  uint32_t pick[3];      // chosen digit, candidates in the digits above it, in it
  uint32_t ncand;
  uint32_t special;      // the staged row holds a NaN or a -0 (checked when values are returned)
};

// Unsigned order equals the value order; -0 and +0 share a key; NaN gets 0,
// below -inf (0x007fffff).
__device__ __forceinline__ uint32_t order_key(float v) {
  if (v != v) return 0u;
  const uint32_t b = (v == 0.0f) ? 0u : __float_as_uint(v);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Inclusive prefix sum over the wave's 64 lanes with DPP moves (no LDS
// round trips): shifts by 1, 2, 4, 8 within each row of 16 lanes, then the
// row totals carried by row_bcast:15 (row r's last lane into row r+1, rows 1
// and 3) and row_bcast:31 (lane 31 into rows 2 and 3).  Lanes with no source
// add 0.
__device__ __forceinline__ uint32_t wave_inclusive_scan_u32(uint32_t v, int lane) {
  (void)lane;
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, true);  // row_shr:1
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, true);  // row_shr:2
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, true);  // row_shr:4
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, true);  // row_shr:8
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false); // row_bcast:15
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false); // row_bcast:31
  return v;
}

// Set bits of a wave mask below this lane.
__device__ __forceinline__ uint32_t lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

__device__ __forceinline__ int topk_shift(int pass) { return pass == 0 ? 21 : (pass == 1 ? 10 : 0); }
__device__ __forceinline__ uint32_t topk_dmask(int pass) { return pass < 2 ? 0x7FFu : 0x3FFu; }

// Four consecutive values starting at i (a multiple of 4); entries at or past
// L are not read.
__device__ __forceinline__ void load4(const float* x, int32_t i, int32_t L, float (&v)[4]) {
  if (i + 4 <= L) {
    const f32x4 t = *reinterpret_cast<const f32x4*>(x + i);
    v[0] = t[0]; v[1] = t[1]; v[2] = t[2]; v[3] = t[3];
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = (i + e < L) ? x[i + e] : 0.0f;
  }
}

// Four consecutive order keys starting at i (a multiple of 4), 0 at or past
// L.  RES: from the stage, which the first pass has filled; otherwise from the
// values in memory, keyed here.
template <bool RES, typename SH>
__device__ __forceinline__ void keys4(const SH& sh, const float* x, int32_t i, int32_t L, uint32_t (&kk)[4]) {
  if constexpr (RES) {
    if (i + 4 <= L) {
      const u32x4 t = *reinterpret_cast<const u32x4*>(&sh.vals[i]);
      kk[0] = t[0]; kk[1] = t[1]; kk[2] = t[2]; kk[3] = t[3];
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) kk[e] = (i + e < L) ? sh.vals[i + e] : 0u;
    }
  } else {
    float v[4];
    load4(x, i, L, v);
#pragma unroll
    for (int e = 0; e < 4; ++e) kk[e] = order_key(v[e]);
  }
}

// The value of position pos of row x, given its order key: the key inverted,
// or for the two keys that lose bits (0: NaN, any payload; 0x80000000: +0 or
// -0) the value itself, read from the row.  PLAIN: the row holds no NaN and
// no -0, so every key inverts (0x80000000 to +0) and nothing is read.
template <bool PLAIN>
__device__ __forceinline__ float key_value(uint32_t key, const float* x, int32_t pos) {
  if (!PLAIN && (key == 0u || key == 0x80000000u)) return x[pos];
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
}

// Wave 0, once sh.hist holds this digit's counts over the candidates that
// match (prefix, mask): pick the digit holding the need-th largest of them,
// with the counts above it and in it, and clear the histogram.  Two levels:
// lane l sums digits 2047-32l down to 2016-32l and a scan finds the lane
// whose range holds the pick; then lanes 0..31 take that range's digits in
// descending order and a second scan finds the digit.
// ROT: the lane reads its 32 counts one word at a time in an order rotated by
// the lane (bin lo + i lies in bank i, lo being a multiple of 32, so one read
// of the wave covers every bank twice), and the histogram is cleared with
// consecutive words per lane; otherwise 16-byte reads and stores of the
// lane's own range.  Measured on MI355X: ROT is faster in the 256-thread
// kernel (4096-row prefill top-k 38.1 -> 35.3 us) and slower in the
// 1024-thread one (64-row decode top-k 20.6 -> 22.0 us).
template <typename SH>
__device__ __forceinline__ void pick_digit(SH& sh, uint32_t need, int lane) {
  constexpr bool ROT = SH::kThreads <= 256;
  const int lo = kTopkBins - 32 * (lane + 1);  // lowest digit of the lane
  uint32_t sum = 0u;
  if constexpr (ROT) {
#pragma unroll
    for (int i = 0; i < 32; ++i) sum += sh.hist[lo + ((i + lane) & 31)];
  } else {
#pragma unroll
    for (int i = 0; i < 32; i += 4) {
      const u32x4 t = *reinterpret_cast<const u32x4*>(&sh.hist[lo + i]);
      sum += t[0] + t[1] + t[2] + t[3];
    }
  }
  const uint32_t incl = wave_inclusive_scan_u32(sum, lane);
  const uint64_t hit = __ballot(incl - sum < need && need <= incl);  // exactly one lane
  const int l1 = __builtin_amdgcn_readfirstlane(hit ? (int)__builtin_ctzll(hit) : 0);
  const uint32_t above1 = __builtin_amdgcn_readlane(incl - sum, l1);
  const int dg = kTopkBins - 1 - 32 * l1 - lane;  // lanes 0..31: the range, descending
  const uint32_t c = lane < 32 ? sh.hist[dg] : 0u;
  const uint32_t incl2 = above1 + wave_inclusive_scan_u32(c, lane);
  if (lane < 32 && incl2 - c < need && need <= incl2) {  // exactly one lane
    sh.pick[0] = (uint32_t)dg;
    sh.pick[1] = incl2 - c;
    sh.pick[2] = c;
  }
  if constexpr (ROT) {
#pragma unroll
    for (int i = 0; i < kTopkBins; i += 64) sh.hist[i + lane] = 0u;
  } else {
#pragma unroll
    for (int i = 0; i < 32; i += 4) *reinterpret_cast<u32x4*>(&sh.hist[lo + i]) = (u32x4){0u, 0u, 0u, 0u};
  }
}

// After a histogram: pick the digit, fold it into (prefix, mask), take the
// candidates of the larger digits off `need`.  Returns the candidates in the
// picked digit.  Every thread calls it.
template <typename SH>
__device__ __forceinline__ uint32_t radix_step(SH& sh, int pass, uint32_t& prefix, uint32_t& mask,
                                               uint32_t& need, int wave, int lane) {
  __syncthreads();  // the histogram is complete
  if (wave == 0) pick_digit(sh, need, lane);
  __syncthreads();  // (pick is next written after the next histogram's barrier)
  need -= sh.pick[1];
  prefix |= sh.pick[0] << topk_shift(pass);
  mask |= topk_dmask(pass) << topk_shift(pass);
  return sh.pick[2];
}

// Histogram of one digit over the row's keys that match (prefix, mask).  RES:
// the first pass reads the row from memory and stages its keys.
template <bool RES, int THREADS, int STEPS, typename SH>
__device__ __forceinline__ void row_histogram(SH& sh, const float* x, int32_t L, int pass, uint32_t prefix,
                                              uint32_t mask, bool find_special = false) {
  const int shift = topk_shift(pass);
  const uint32_t dmask = topk_dmask(pass);
  auto count4 = [&](int32_t i) {
    uint32_t kk[4];
    keys4<RES>(sh, x, i, L, kk);
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (i + e < L && (kk[e] & mask) == prefix) atomicAdd(&sh.hist[(kk[e] >> shift) & dmask], 1u);
  };
  const int tid = threadIdx.x;
  if constexpr (RES) {
    if (pass == 0) {
      // The row comes from memory: every load is in flight before the first
      // key is written to the stage and counted.
      float v[STEPS][4];
#pragma unroll
      for (int j = 0; j < STEPS; ++j) {
        const int32_t i = 4 * THREADS * j + 4 * tid;
        if (i < L) load4(x, i, L, v[j]);
      }
      bool special = false;  // a NaN or a -0 (whose keys do not invert to them)
#pragma unroll
      for (int j = 0; j < STEPS; ++j) {
        const int32_t i = 4 * THREADS * j + 4 * tid;
        if (i < L) {
          uint32_t kk[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            kk[e] = order_key(v[j][e]);
            if (find_special)
              special |= i + e < L && (v[j][e] != v[j][e] || __float_as_uint(v[j][e]) == 0x80000000u);
          }
          if (i + 4 <= L) {
            *reinterpret_cast<u32x4*>(&sh.vals[i]) = (u32x4){kk[0], kk[1], kk[2], kk[3]};
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (i + e < L) sh.vals[i + e] = kk[e];
          }
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (i + e < L) atomicAdd(&sh.hist[(kk[e] >> shift) & dmask], 1u);  // (pass 0 matches every key)
        }
      }
      if (special) sh.special = 1u;  // (read after the next barrier)
      return;
    }
#pragma unroll
    for (int j = 0; j < STEPS; ++j) {  // STEPS 16-byte groups per thread cover the staged row
      const int32_t i = 4 * THREADS * j + 4 * tid;
      if (i < L) count4(i);
    }
  } else {
    for (int32_t i = 4 * tid; i < L; i += 4 * THREADS) count4(i);
  }
}

// Rows of the 1024-thread kernel that take at most a quarter of their keys,
// from the first digit on.  Thread t owns the 32 positions 32t .. 32t+31 and
// keeps them as two words of bits: `ab`, its keys above the current digit,
// and `eb`, its keys in it.  The later digits count only the positions in eb
// (their keys re-read from the stage), the final key splits eb into keys above
// it and keys at it, and one block scan of the packed counts gives each
// thread its first output slot.  No position list and no shared bitmaps.
template <int THREADS, int CAP, int CAND>
__device__ __forceinline__ void topk_row_owned(TopkShared<THREADS, CAP, CAND>& sh, const float* x, int32_t L,
                                               int32_t* io, float* vo, uint32_t prefix, uint32_t mask,
                                               uint32_t need, uint32_t in_digit, int wave, int lane) {
  static_assert(CAP == 32 * THREADS, "one 32-position word per thread");
  const int32_t p0 = 32 * (int32_t)threadIdx.x;
  uint32_t ab = 0u, eb = 0u;
  if (p0 < L) {
    // After the first digit, mask keeps its 11 bits: a key is in the digit
    // when it is >= prefix and below the next digit's first key.
    const uint32_t next = prefix + (1u << topk_shift(0));  // 0 for the top digit
    uint32_t ge = 0u, gt = 0u;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      // lane l starts at chunk l % 8: the 8 lanes that one 16-byte LDS read
      // serves at a time then cover distinct banks
      const int ch = (c + lane) & 7;
      const u32x4 kk = *reinterpret_cast<const u32x4*>(&sh.vals[p0 + 4 * ch]);
      uint32_t g4 = 0u, t4 = 0u;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        g4 |= (kk[e] >= prefix ? 1u : 0u) << e;
        t4 |= (kk[e] >= next ? 1u : 0u) << e;
      }
      ge |= g4 << (4 * ch);
      gt |= t4 << (4 * ch);
    }
    if (next == 0u) gt = 0u;
    const uint32_t valid = (L - p0 >= 32) ? ~0u : ((1u << (L - p0)) - 1u);
    ab = gt & valid;
    eb = ge & ~gt & valid;
  }
  for (int pass = 1; pass < 3 && need != in_digit; ++pass) {
    const int shift = topk_shift(pass);
    const uint32_t dmask = topk_dmask(pass);
    for (uint32_t bits = eb; bits != 0u; bits &= bits - 1u) {
      const uint32_t key = sh.vals[p0 + __builtin_ctz(bits)];
      if ((key & mask) == prefix) atomicAdd(&sh.hist[(key >> shift) & dmask], 1u);
    }
    in_digit = radix_step(sh, pass, prefix, mask, need, wave, lane);
  }
  uint32_t at = 0u;  // keys at the final key (all of them taken when need == in_digit)
  for (uint32_t bits = eb; bits != 0u; bits &= bits - 1u) {
    const int b = __builtin_ctz(bits);
    const uint32_t key = sh.vals[p0 + b] & mask;
    if (key > prefix) ab |= 1u << b;
    else if (key == prefix) at |= 1u << b;
  }
  const uint32_t c = (uint32_t)__builtin_popcount(ab) | ((uint32_t)__builtin_popcount(at) << 16);
  const uint32_t incl = wave_inclusive_scan_u32(c, lane);  // (each half stays below 2^16)
  if (lane == 63) sh.wave_gt[wave] = incl;
  __syncthreads();
  uint32_t ex = incl - c;
  for (int w = 0; w < wave; ++w) ex += sh.wave_gt[w];
  // a key at the final key is taken while fewer than `need` came before it
  auto emit_bits = [&](auto plain) {
    uint32_t gl = ex & 0xFFFFu, ql = ex >> 16;
    for (uint32_t bits = ab | at; bits != 0u; bits &= bits - 1u) {
      const int b = __builtin_ctz(bits);
      const bool above = (ab >> b) & 1u;
      if (above || ql < need) {
        const uint32_t slot = gl + min(ql, need);
        io[slot] = p0 + b;
        if (vo) vo[slot] = key_value<decltype(plain)::value>(sh.vals[p0 + b], x, p0 + b);
      }
      gl += above ? 1u : 0u;
      ql += above ? 0u : 1u;
    }
  };
  if (sh.special == 0u) emit_bits(std::true_type{});
  else emit_bits(std::false_type{});
  __syncthreads();  // wave_gt / vals are rewritten by the next row
}

// Row of L > k candidates.  RES: the row is in sh.vals (L <= CAP).
template <bool RES, int THREADS, int CAP, int CAND>
__device__ __forceinline__ void topk_row(TopkShared<THREADS, CAP, CAND>& sh, const float* x, int32_t L,
                                         int32_t k, int32_t* io, float* vo) {
  constexpr int kWaves = THREADS / 64;
  constexpr int kSteps = (CAP + 4 * THREADS - 1) / (4 * THREADS);  // staged 16-byte groups per thread
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // The compaction's segments: wave w owns positions [w*seg, (w+1)*seg), seg
  // a multiple of 256 with kWaves * seg >= L.
  const int32_t seg = ((L + kWaves - 1) / kWaves + 255) & ~255;
  const int32_t s0 = min(wave * seg, L), s1 = min(s0 + seg, L);
  // Radix select.  Invariant: 1 <= need <= candidates matching (prefix, mask).
  uint32_t prefix = 0u, mask = 0u, need = (uint32_t)k;
  row_histogram<RES, THREADS, kSteps>(sh, x, L, 0, prefix, mask, vo != nullptr);
  uint32_t in_digit = radix_step(sh, 0, prefix, mask, need, wave, lane);
  if constexpr (kTopkBitmap<THREADS> && RES) {
    if (4 * (int64_t)k <= (int64_t)L) {  // sparse rows: compaction from per-thread bit words
      topk_row_owned(sh, x, L, io, vo, prefix, mask, need, in_digit, wave, lane);
      return;
    }
  }
  bool counted = false;  // sh.wave_gt / wave_eq hold the segments' counts
  if (need != in_digit) {
    // RES rows whose first digit fits the list: one sweep over this wave's
    // segment counts the keys above the digit and lists the positions in it.
    const bool listed = RES && in_digit <= (uint32_t)CAND;
    if (listed) {
      static_assert(4 * kSteps <= 32, "a lane's digit bits fill one word");
      uint32_t lane_g = 0u, eqb = 0u;  // bit 4j+e: position s0 + 256j + 4*lane + e has the digit
      int j = 0;
      for (int32_t c0 = s0; c0 < s1; c0 += 256, ++j) {  // (at most kSteps steps: seg <= 256 * kSteps)
        uint32_t kk[4];
        keys4<true>(sh, x, c0 + 4 * lane, s1, kk);
        uint32_t gb = 0u;  // bit e: position c0 + 4*lane + e is above the digit
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bool ok = c0 + 4 * lane + e < s1;
          const uint32_t key = kk[e] & mask;
          gb |= (ok && key > prefix ? 1u : 0u) << e;
          eqb |= (ok && key == prefix ? 1u : 0u) << (4 * j + e);
        }
        lane_g += __builtin_popcount(gb);
      }
      {
        const uint32_t m = __builtin_popcount(eqb);
        const uint32_t incl = wave_inclusive_scan_u32(m, lane);
        uint32_t base = 0u;
        if (lane == 63) base = atomicAdd(&sh.ncand, incl);
        uint32_t at = __shfl(base, 63) + incl - m;
        while (eqb != 0u) {
          const int bit = __builtin_ctz(eqb);
          sh.cand[at++] = (uint32_t)(s0 + 256 * (bit >> 2) + 4 * lane + (bit & 3));
          eqb &= eqb - 1u;
        }
      }
      const uint32_t wg = __builtin_amdgcn_readlane(wave_inclusive_scan_u32(lane_g, lane), 63);
      if (lane == 0) {
        sh.wave_gt[wave] = wg;
        sh.wave_eq[wave] = 0u;
      }
      __syncthreads();
    }
    for (int pass = 1; pass < 3; ++pass) {
      if (listed) {
        const int shift = topk_shift(pass);
        const uint32_t dmask = topk_dmask(pass);
        for (int32_t i = tid; i < (int32_t)in_digit; i += THREADS) {
          const uint32_t key = sh.vals[sh.cand[i]];  // in_digit == the list's length
          if ((key & mask) == prefix) atomicAdd(&sh.hist[(key >> shift) & dmask], 1u);
        }
      } else {
        row_histogram<RES, THREADS, kSteps>(sh, x, L, pass, prefix, mask);
      }
      const uint32_t in_d = radix_step(sh, pass, prefix, mask, need, wave, lane);
      if (need == in_d) break;  // the whole digit is taken: no finer digit needed
    }
    if (listed) {
      // Keys outside the first digit are above the final key exactly when
      // they are above the digit (counted); the listed ones are counted here
      // into the segment that holds them.
      for (int32_t i = tid; i < (int32_t)in_digit; i += THREADS) {
        const uint32_t pos = sh.cand[i];
        const uint32_t key = sh.vals[pos] & mask;
        const int w = (int)(pos / (uint32_t)seg);
        if (key > prefix) atomicAdd(&sh.wave_gt[w], 1u);
        else if (key == prefix) atomicAdd(&sh.wave_eq[w], 1u);
      }
      __syncthreads();
      counted = true;
    }
  }

  // Compaction over the same segments; lane l holds positions c0+4l ..
  // c0+4l+3 of each 256-position step.  Per lane and step the counts are
  // packed (keys above the threshold in the low 16 bits, keys at it in the
  // high 16; a step holds 256 positions), and one wave scan per step orders
  // them; running totals are 32-bit.
  auto classify = [&](int32_t c0, uint32_t (&kk)[4], uint32_t& bits) -> uint32_t {
    keys4<RES>(sh, x, c0 + 4 * lane, s1, kk);
    uint32_t c = 0u;
    bits = 0u;  // bit e: above, bit 4+e: at the threshold
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool ok = c0 + 4 * lane + e < s1;
      const uint32_t key = kk[e] & mask;
      const uint32_t gt = (ok && key > prefix) ? 1u : 0u, eq = (ok && key == prefix) ? 1u : 0u;
      c += gt | (eq << 16);
      bits |= (gt << e) | (eq << (4 + e));
    }
    return c;
  };
  if (!counted) {
    uint32_t lane_g = 0u, lane_q = 0u;
    for (int32_t c0 = s0; c0 < s1; c0 += 256) {
      uint32_t kk[4], bits;
      const uint32_t c = classify(c0, kk, bits);
      lane_g += c & 0xFFFFu;
      lane_q += c >> 16;
    }
    const uint32_t wg = __builtin_amdgcn_readlane(wave_inclusive_scan_u32(lane_g, lane), 63);
    const uint32_t wq = __builtin_amdgcn_readlane(wave_inclusive_scan_u32(lane_q, lane), 63);
    if (lane == 0) {
      sh.wave_gt[wave] = wg;
      sh.wave_eq[wave] = wq;
    }
    __syncthreads();
  }
  uint32_t g = 0u, q = 0u;  // candidates of the earlier waves' segments
  for (int w = 0; w < wave; ++w) {
    g += sh.wave_gt[w];
    q += sh.wave_eq[w];
  }
  // A row with no NaN and no -0 takes a loop whose values are the inverted
  // keys alone: a load there would make every value store wait for all the
  // stores before it (the memory counter retires in order).
  auto emit = [&](auto plain) {
    for (int32_t c0 = s0; c0 < s1; c0 += 256) {
      uint32_t kk[4], bits;
      const uint32_t c = classify(c0, kk, bits);
      const uint32_t incl = wave_inclusive_scan_u32(c, lane), ex = incl - c;
      uint32_t gl = g + (ex & 0xFFFFu), ql = q + (ex >> 16);  // before this lane's first position
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool gt = (bits >> e) & 1u, eq = (bits >> (4 + e)) & 1u;
        const uint32_t slot = gl + min(ql, need);  // a key at the threshold: gl + ql when taken
        if (gt || (eq && ql < need)) {
          io[slot] = c0 + 4 * lane + e;
          if (vo) vo[slot] = key_value<decltype(plain)::value>(kk[e], x, c0 + 4 * lane + e);
        }
        gl += gt ? 1u : 0u;
        ql += eq ? 1u : 0u;
      }
      const uint32_t tot = __builtin_amdgcn_readlane(incl, 63);
      g += tot & 0xFFFFu;
      q += tot >> 16;
    }
  };
  if (RES && sh.special == 0u) emit(std::true_type{});
  else emit(std::false_type{});
  __syncthreads();  // wave_gt / wave_eq / vals / cand are rewritten by the next row
}

template <int THREADS, int CAP, int CAND, bool LAST_FIRST>
__global__ __launch_bounds__(THREADS) void topk_kernel(const float* logits, int64_t row_stride,
                                                       const int32_t* seqlens, int32_t rows, int32_t ncols,
                                                       int32_t k, int32_t* idx_out, float* val_out) {
  __shared__ __attribute__((aligned(16))) TopkShared<THREADS, CAP, CAND> sh;
  const int tid = threadIdx.x;
  for (int i = tid; i < kTopkBins; i += THREADS) sh.hist[i] = 0u;  // wave 0 re-clears after each pick
  for (int32_t rb = blockIdx.x; rb < rows; rb += gridDim.x) {
    const int32_t b = LAST_FIRST ? rows - 1 - rb : rb;
    const int32_t L = min(max(seqlens[b], 0), ncols);
    const float* x = logits + (int64_t)b * row_stride;
    int32_t* io = idx_out + (int64_t)b * k;
    float* vo = val_out ? val_out + (int64_t)b * k : nullptr;
    for (int32_t t = min(L, k) + tid; t < k; t += THREADS) {
      io[t] = -1;
      if (vo) vo[t] = -INFINITY;
    }
    if (tid == 0) {
      sh.ncand = 0u;
      sh.special = 0u;
    }
    if (L <= k) {  // every candidate is selected
      for (int32_t t = tid; t < L; t += THREADS) {
        io[t] = t;
        if (vo) vo[t] = x[t];
      }
    } else if (L <= CAP) {
      __syncthreads();  // (the histogram is clear; the first pass stages the row's keys)
      topk_row<true>(sh, x, L, k, io, vo);
    } else {
      __syncthreads();
      topk_row<false>(sh, x, L, k, io, vo);
    }
  }
}

// ---------------------------------------------------------------------------
// Host side.

constexpr int kRowwisePPW = 2;
constexpr int kRowwiseWaves = 4;
constexpr int kSharedTargetWgPerCu = 4;  // units per CU wanted before splitting rows into chunks
constexpr int kSharedPairWgPerCu = 2;    // resident shared-kernel workgroups per CU (LDS, 2 waves/SIMD)
constexpr int64_t kMaxGrid = (int64_t)1 << 20;  // larger grids loop (grid-stride)
constexpr int32_t kMaxWidth = 1 << 24;

constexpr int kBalancedWaves = 4;
constexpr int kBalancedWgPerCu = 2;
constexpr int kBalancedSlots = 2;  // fp8 pages in flight per wave (LDS slots)

// Compute units of the current device (queried once per device).
int device_cu_count() {
  static std::atomic<int> cache[64];  // per device; concurrent callers store the same value
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

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
           hipStream_t stream, bool fill = true, const int32_t* row_table = nullptr,
           int32_t num_tables = 1) {
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
  p.pages_lim = (uint32_t)(num_pages < ((int64_t)1 << 31) ? num_pages : ((int64_t)1 << 31));
  p.kv_stride = kv_page_stride;
  p.ks_stride = (KEY == kFp8) ? kscale_page_stride : 0;
  p.pt_stride = page_table_row_stride;
  p.rows = rows;
  p.width = table_width;
  p.fill = fill ? 1 : 0;
  p.rt = row_table;
  p.num_tables = num_tables;

  (void)hipGetLastError();  // start from a clean error state
  if (row_table == nullptr && (page_table_row_stride != 0 || rows == 1)) {
    if (rows <= kBalancedMaxRows) {
      const int64_t slots = (int64_t)rows * table_width;
      const int64_t want = (slots + 7) / 8;
      const int64_t cap = (int64_t)kBalancedWgPerCu * device_cu_count();
      const int64_t grid = want < 1 ? 1 : (want < cap ? want : cap);
      balanced_kernel<KEY, kBalancedWaves, kBalancedSlots>
          <<<dim3((uint32_t)grid), dim3(64 * kBalancedWaves), 0, stream>>>(p);
      return hipGetLastError() == hipSuccess ? IDX_OK : IDX_ERR_LAUNCH;
    }
  }
  if (row_table != nullptr || (page_table_row_stride == 0 && rows > 1)) {
    const int32_t row_blocks = (rows + kSharedRows - 1) / kSharedRows;
    // Whole rows per unit (the query is read once) unless that leaves too few
    // units to fill the chip; then split the table into chunks.
    const int64_t want = (int64_t)kSharedTargetWgPerCu * device_cu_count();
    int32_t chunks = (int32_t)((want + row_blocks - 1) / row_blocks);
    chunks = chunks < 1 ? 1 : (chunks > table_width ? table_width : chunks);
    const int32_t chunk = (table_width + chunks - 1) / chunks;
    chunks = (table_width + chunk - 1) / chunk;
    const int32_t rb_per_xcd = (row_blocks + 7) / 8;
    const int64_t total = (int64_t)8 * rb_per_xcd * chunks;
    const int64_t units = (row_table != nullptr) ? 4 * total : total;
    const int64_t grid = units < kMaxGrid ? units : kMaxGrid;
    // bf16 keys, whole-table units and more row blocks than resident
    // workgroups (two per CU): pair long and short row blocks on one
    // workgroup (measured on the 4096-row prefill: 189.4 -> 181.2 us; with fp8
    // keys the same pairing measured 183.5 -> 189.1 us, so they keep the
    // longest-first order).
    const int64_t resident = (int64_t)kSharedPairWgPerCu * device_cu_count();
    if (row_table != nullptr)
      shared_kernel<KEY, true><<<dim3((uint32_t)grid), dim3(64 * kSharedRows), 0, stream>>>(
          p, row_blocks, chunk, chunks, rb_per_xcd, total, 0);
    else if (KEY == kBf16 && chunks == 1 && row_blocks > resident)
      shared_kernel<KEY, false><<<dim3((uint32_t)resident), dim3(64 * kSharedRows), 0, stream>>>(
          p, row_blocks, chunk, chunks, rb_per_xcd, (row_blocks + resident - 1) / resident * resident, 1);
    else
      shared_kernel<KEY, false><<<dim3((uint32_t)grid), dim3(64 * kSharedRows), 0, stream>>>(
          p, row_blocks, chunk, chunks, rb_per_xcd, total, 0);
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

int validate_topk(const float* logits, int64_t row_stride, const int32_t* seqlens, int32_t rows,
                  int32_t ncols, int32_t k, const int32_t* topk_idx, const float* topk_val) {
  if (rows < 0 || ncols < 0 || k < 0 || row_stride < ncols) return IDX_ERR_SHAPE;
  if (rows == 0 || k == 0) return IDX_OK;
  if ((ncols > 0 && !logits) || !seqlens || !topk_idx) return IDX_ERR_NULL;
  if (!aligned(logits, 16) || (row_stride % 4) != 0 || !aligned(seqlens, 4) || !aligned(topk_idx, 4) ||
      (topk_val && !aligned(topk_val, 4)))
    return IDX_ERR_ALIGN;
  return IDX_OK;
}

// Rows of at most 6144 candidates (ncols bounds every L) take 256-thread
// workgroups staging up to 6144 keys (four fit one CU's LDS); longer ones
// 1024 threads staging up to 32768 (one per CU).  When there are more rows
// than resident workgroups, rows wait for a free workgroup and are taken last
// first: under a causal limit the later rows are the longer ones, and
// starting them first leaves the short rows to fill the end of the launch.
void launch_topk(const float* logits, int64_t row_stride, const int32_t* seqlens, int32_t rows,
                 int32_t ncols, int32_t k, int32_t* topk_idx, float* topk_val, hipStream_t stream) {
  const int64_t cus = device_cu_count();
  if (ncols <= 6144) {
    const int64_t cap = 64 * cus;
    const dim3 grid((uint32_t)(rows < cap ? rows : cap));
    if (rows > 4 * cus)
      topk_kernel<256, 6144, 1024, true><<<grid, dim3(256), 0, stream>>>(logits, row_stride, seqlens, rows,
                                                                          ncols, k, topk_idx, topk_val);
    else
      topk_kernel<256, 6144, 1024, false><<<grid, dim3(256), 0, stream>>>(logits, row_stride, seqlens, rows,
                                                                           ncols, k, topk_idx, topk_val);
  } else {
    const int64_t cap = 16 * cus;
    const dim3 grid((uint32_t)(rows < cap ? rows : cap));
    if (rows > cus)
      topk_kernel<1024, 32768, 4096, true><<<grid, dim3(1024), 0, stream>>>(logits, row_stride, seqlens, rows,
                                                                             ncols, k, topk_idx, topk_val);
    else
      topk_kernel<1024, 32768, 4096, false><<<grid, dim3(1024), 0, stream>>>(logits, row_stride, seqlens, rows,
                                                                              ncols, k, topk_idx, topk_val);
  }
}

template <int KEY>
int launch_logits_topk(const void* q, const void* kv_pages, const float* kscale, const int32_t* page_table,
                       const int32_t* seqlens, const float* weights, float* logits, int32_t rows,
                       int32_t num_heads, int32_t head_dim, int32_t table_width, int64_t num_pages,
                       int64_t kv_page_stride, int64_t kscale_page_stride,
                       int64_t page_table_row_stride, int32_t k, int32_t* topk_idx, float* topk_val,
                       hipStream_t stream) {
  const int st = validate(KEY, q, kv_pages, kscale, page_table, seqlens, weights, logits, rows, num_heads,
                          head_dim, table_width, num_pages, kv_page_stride, kscale_page_stride,
                          page_table_row_stride);
  if (st != IDX_OK) return st;
  const int64_t ncols = (int64_t)table_width * kPage;
  const int st2 = validate_topk(logits, ncols, seqlens, rows, (int32_t)ncols, k, topk_idx, topk_val);
  if (st2 != IDX_OK) return st2;
  if (rows == 0) return IDX_OK;
  if (table_width == 0) {  // no candidates: the top-k rows are all padding
    if (k == 0) return IDX_OK;
    (void)hipGetLastError();
    launch_topk(logits, 0, seqlens, rows, 0, k, topk_idx, topk_val, stream);
    return hipGetLastError() == hipSuccess ? IDX_OK : IDX_ERR_LAUNCH;
  }
  const int st3 = launch<KEY>(q, kv_pages, kscale, page_table, seqlens, weights, logits, rows, num_heads,
                              head_dim, table_width, num_pages, kv_page_stride, kscale_page_stride,
                              page_table_row_stride, stream, /*fill=*/false);
  if (st3 != IDX_OK || k == 0) return st3;
  launch_topk(logits, ncols, seqlens, rows, (int32_t)ncols, k, topk_idx, topk_val, stream);
  return hipGetLastError() == hipSuccess ? IDX_OK : IDX_ERR_LAUNCH;
}

template <int KEY>
int launch_varlen(const void* q, const void* kv_pages, const float* kscale, const int32_t* page_table,
                  const int32_t* row_table, int32_t num_tables, const int32_t* seqlens,
                  const float* weights, float* out, int32_t rows, int32_t num_heads, int32_t head_dim,
                  int32_t table_width, int64_t num_pages, int64_t kv_page_stride,
                  int64_t kscale_page_stride, int64_t page_table_row_stride, hipStream_t stream) {
  const int st = validate(KEY, q, kv_pages, kscale, page_table, seqlens, weights, out, rows, num_heads,
                          head_dim, table_width, num_pages, kv_page_stride, kscale_page_stride,
                          page_table_row_stride);
  if (st != IDX_OK) return st;
  if (num_tables < 0) return IDX_ERR_SHAPE;
  if (rows == 0 || table_width == 0) return IDX_OK;
  if (!row_table) return IDX_ERR_NULL;
  if (!aligned(row_table, 4)) return IDX_ERR_ALIGN;
  return launch<KEY>(q, kv_pages, kscale, page_table, seqlens, weights, out, rows, num_heads, head_dim,
                     table_width, num_pages, kv_page_stride, kscale_page_stride, page_table_row_stride,
                     stream, /*fill=*/true, row_table, num_tables);
}

template <int KEY>
int store_keys(const void* keys, const int64_t* slots, int64_t n, void* kv_pages, float* kscale,
               int64_t num_pages, int64_t kv_page_stride, int64_t kscale_page_stride,
               hipStream_t stream) {
  if (n < 0 || num_pages < 0) return IDX_ERR_SHAPE;
  const int64_t min_kv = (KEY == kFp8) ? (int64_t)kPage * kDim : (int64_t)kPage * kDim * 2;
  if (kv_page_stride < min_kv || kv_page_stride > ((int64_t)1 << 32)) return IDX_ERR_SHAPE;
  if (KEY == kFp8 && (kscale_page_stride < kPage * 4 || kscale_page_stride > ((int64_t)1 << 32)))
    return IDX_ERR_SHAPE;
  if (n == 0) return IDX_OK;
  if (!keys || !slots || !kv_pages) return IDX_ERR_NULL;
  if (KEY == kFp8 ? (kscale == nullptr) : (kscale != nullptr)) return IDX_ERR_NULL;
  if (!aligned(keys, 16) || !aligned(slots, 8) || !aligned(kv_pages, 16) || (kv_page_stride % 16) != 0)
    return IDX_ERR_ALIGN;
  if (KEY == kFp8 && (!aligned(kscale, 4) || (kscale_page_stride % 4) != 0)) return IDX_ERR_ALIGN;
  (void)hipGetLastError();
  const int64_t want = (n + 4 * kStoreWaves * kStoreUnroll - 1) / (4 * kStoreWaves * kStoreUnroll);
  const int64_t cap = (int64_t)8 * device_cu_count();
  const int64_t grid = want < cap ? want : cap;
  store_keys_kernel<KEY><<<dim3((uint32_t)grid), dim3(64 * kStoreWaves), 0, stream>>>(
      static_cast<const uint8_t*>(keys), slots, n, static_cast<uint8_t*>(kv_pages),
      reinterpret_cast<uint8_t*>(kscale), num_pages, kv_page_stride,
      (KEY == kFp8) ? kscale_page_stride : 0);
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

int idx_paged_mqa_logits_varlen_fp8(const void* q, const void* kv_pages, const float* kscale,
                                    const int32_t* page_table, const int32_t* row_table,
                                    int32_t num_tables, const int32_t* seqlens, const float* weights,
                                    float* out, int32_t rows, int32_t num_heads, int32_t head_dim,
                                    int32_t table_width, int64_t num_pages, int64_t kv_page_stride,
                                    int64_t kscale_page_stride, int64_t page_table_row_stride,
                                    hipStream_t stream) {
  return launch_varlen<kFp8>(q, kv_pages, kscale, page_table, row_table, num_tables, seqlens, weights, out,
                             rows, num_heads, head_dim, table_width, num_pages, kv_page_stride,
                             kscale_page_stride, page_table_row_stride, stream);
}

int idx_paged_mqa_logits_varlen_bf16(const void* q, const void* kv_pages, const float* kscale,
                                     const int32_t* page_table, const int32_t* row_table,
                                     int32_t num_tables, const int32_t* seqlens, const float* weights,
                                     float* out, int32_t rows, int32_t num_heads, int32_t head_dim,
                                     int32_t table_width, int64_t num_pages, int64_t kv_page_stride,
                                     int64_t kscale_page_stride, int64_t page_table_row_stride,
                                     hipStream_t stream) {
  return launch_varlen<kBf16>(q, kv_pages, kscale, page_table, row_table, num_tables, seqlens, weights,
                              out, rows, num_heads, head_dim, table_width, num_pages, kv_page_stride,
                              kscale_page_stride, page_table_row_stride, stream);
}

int idx_topk_logits(const float* logits, int64_t row_stride, const int32_t* seqlens, int32_t rows,
                    int32_t ncols, int32_t k, int32_t* topk_idx, float* topk_val, hipStream_t stream) {
  const int st = validate_topk(logits, row_stride, seqlens, rows, ncols, k, topk_idx, topk_val);
  if (st != IDX_OK || rows == 0 || k == 0) return st;
  (void)hipGetLastError();
  launch_topk(logits, row_stride, seqlens, rows, ncols, k, topk_idx, topk_val, stream);
  return hipGetLastError() == hipSuccess ? IDX_OK : IDX_ERR_LAUNCH;
}

int idx_paged_mqa_topk_fp8(const void* q, const void* kv_pages, const float* kscale,
                           const int32_t* page_table, const int32_t* seqlens, const float* weights,
                           float* logits, int32_t rows, int32_t num_heads, int32_t head_dim,
                           int32_t table_width, int64_t num_pages, int64_t kv_page_stride,
                           int64_t kscale_page_stride, int64_t page_table_row_stride, int32_t k,
                           int32_t* topk_idx, float* topk_val, hipStream_t stream) {
  return launch_logits_topk<kFp8>(q, kv_pages, kscale, page_table, seqlens, weights, logits, rows,
                                  num_heads, head_dim, table_width, num_pages, kv_page_stride,
                                  kscale_page_stride, page_table_row_stride, k, topk_idx, topk_val,
                                  stream);
}

int idx_paged_mqa_topk_bf16(const void* q, const void* kv_pages, const float* kscale,
                            const int32_t* page_table, const int32_t* seqlens, const float* weights,
                            float* logits, int32_t rows, int32_t num_heads, int32_t head_dim,
                            int32_t table_width, int64_t num_pages, int64_t kv_page_stride,
                            int64_t kscale_page_stride, int64_t page_table_row_stride, int32_t k,
                            int32_t* topk_idx, float* topk_val, hipStream_t stream) {
  return launch_logits_topk<kBf16>(q, kv_pages, kscale, page_table, seqlens, weights, logits, rows,
                                   num_heads, head_dim, table_width, num_pages, kv_page_stride,
                                   kscale_page_stride, page_table_row_stride, k, topk_idx, topk_val,
                                   stream);
}

int idx_store_keys_fp8(const void* keys, const int64_t* slots, int64_t n, void* kv_pages, float* kscale,
                       int64_t num_pages, int64_t kv_page_stride, int64_t kscale_page_stride,
                       hipStream_t stream) {
  return store_keys<kFp8>(keys, slots, n, kv_pages, kscale, num_pages, kv_page_stride,
                          kscale_page_stride, stream);
}

int idx_store_keys_bf16(const void* keys, const int64_t* slots, int64_t n, void* kv_pages,
                        int64_t num_pages, int64_t kv_page_stride, hipStream_t stream) {
  return store_keys<kBf16>(keys, slots, n, kv_pages, nullptr, num_pages, kv_page_stride, 0, stream);
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
