// prefill_bf16.hip -- prefill attention with a learned relative-position bias
// over a paged KV pool, bf16 in / fp32 accumulate, for gfx950 (CDNA4).
//
// Computes, for every query token t of a sequence and query head h,
//   out[t,h] = softmax_s( sm_scale * q[t,h].k[s,g] + bias[t,h,min(t-s,R-1)] ) v[s,g]
// over the visible keys s (s <= t, and t - s < window on local layers),
// g = h / (Hq/Hkv).  The bias is added before the softmax and indexed by
// (query token, head, relative distance) as the TensorRT-LLM PR #17062 page
// ("Support Inkling-NVFP4 model", Description, Architecture list) states;
// its [T, heads, rel_extent] shape is the one in that page's review comment
// on _build_rel_logits.
//
// Work decomposition: a work-group of NW waves (4 or 8) covers hpw query
// heads of one KV head times NW/hpw blocks of 32 consecutive queries; each
// wave owns 32 queries of one head and every K/V tile it loads serves all
// 32*NW (head, query) rows:
//  * 64-key K and V tiles go HBM -> LDS directly (buffer_load_dwordx4 with
//    the LDS bit through a buffer resource where a page holds whole tiles,
//    else global_load_lds_dwordx4; no register staging) into two buffers,
//    row-major with XOR-swizzled
//    16-byte chunks: tile i+1 streams in while tile i computes, one barrier
//    per tile.  Tile rows outside the work-group's key range (below the
//    first key any of its queries sees, or past the end of the sequence)
//    are filled from the nearest end of that range, so every K/V row loaded
//    is a key some query of the call sees (finite data whose probabilities
//    are exactly zero where it is masked);
//  * S^T = K Q^T and O^T += V^T P^T run on v_mfma_f32_32x32x16_bf16, so each
//    lane owns one query column: the softmax row statistics stay in a lane
//    pair (lane, lane^32);
//  * the K operand reads key rows in an order with bits 2 and 3 of the row
//    index swapped, which hands each lane runs of 8 consecutive keys;
//  * the V^T operand comes straight from the row-major V tile through the
//    transposing LDS read ds_read_b64_tr_b16;
//  * for each tile a query row needs the 64 distances t-s0-63 .. t-s0 of its
//    bias row.  Each wave streams them for its 32 rows straight into a 4 KiB
//    LDS stage of its own (buffer loads with the LDS bit, eight lanes per
//    row, so a load instruction touches 8 rows instead of 32), one tile ahead, and
//    every lane then picks its four runs of 8 consecutive distances out of
//    it with aligned 16-byte reads; every bias element crosses HBM once.
//    Tiles whose distances all lie at or beyond R-1 use the single clamped
//    value bias[t,h,R-1] and load nothing;
//  * three score paths chosen per wave and tile: clamp-only unmasked (scale,
//    bias and max folded into one FMA before exp2), band unmasked, and a
//    general path for window/causal/sequence-end edges and the clamp border;
//  * masking selects (never multiplies), and no K/V row outside the keys the
//    work-group's queries see is ever loaded, so pool slots no query may see
//    (unwritten ring slots, pages past a sequence, keys older than the
//    window) cannot reach the output whatever they hold;
//  * the running max is rescaled lazily (only when a row's max grows by more
//    than 2^8), which is exact because numerator and denominator share it.
//
// The fused variant (DR = d_rel > 0) takes no bias tensor: it forms
// bias[t,h,d] = r[t,h,:] . W[:,d] on the fly, the product that page's review
// comment on _build_rel_logits materialises as [T, heads, rel_extent] (there
// in fp32).  Per tile the work-group loads, with K and V, the rows of W^T
// ([R][d_rel], distance-major) for the distances its queries meet, clamped to
// [0, R-1]; each wave with a band tile multiplies them by its 32 r rows on the
// matrix cores (3 x d_rel/16 MFMAs give the 96 distances of its 32 queries),
// rounds the products to bf16 and writes them skewed into its stage, eight
// consecutive distances per 16-byte store; each lane then reads its four runs
// back as 4-byte words, shifted by one element on odd rows.  Tiles
// at or beyond R-1 use r . W[:,R-1], formed once per row in fp32 and rounded
// to bf16 like the stage entries: every bias value is the product rounded
// once to bf16, the tensor a materialised bf16 bias would hold.
#include "rba_internal.h"

#include <climits>
#include <type_traits>

namespace rba {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

constexpr int BN = 64;         // keys per tile
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;
constexpr float NEG_INIT = -1.0e30f;  // finite start of the running max (log2 units)
constexpr float TAU = 8.0f;           // lazy-rescale threshold (log2 units)

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Element e (compile-time) of eight packed bf16 values, as fp32.
__device__ __forceinline__ float bf16x8_elem(const u32x4_t &p, int e) {
  const uint32_t w = p[e >> 1];
  return __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two floats -> two bf16 (round to nearest even) in one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2_t v = __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t);
  return __builtin_bit_cast(uint32_t, v);
}

// XOR swizzles of the 16-byte chunks of a row.  K: chunk ^ (row mod CHUNKS)
// keeps the 32 rows an MFMA operand read touches on distinct banks.  V: a
// transposing read touches 4 rows of equal (row mod 4) pattern x 2..4
// consecutive chunks, which the per-row pattern below spreads over distinct
// banks.
template <int D>
__device__ __forceinline__ int v_swizzle(int row) {
  if constexpr (D == 128) {
    constexpr int tab = (0) | (6 << 4) | (12 << 8) | (10 << 12);
    return (tab >> ((row & 3) * 4)) & 15;
  } else {
    return 2 * (row & 3);
  }
}

// Key row of S^T row m within a 32-key block: bits 2 and 3 swapped.  Lane
// (col, half) then holds keys 8*half + 0..7 and 16 + 8*half + 0..7.
__device__ __forceinline__ int key_of_row(int m) {
  return (m & 0x13) | ((m & 4) << 1) | ((m & 8) >> 1);
}

typedef __attribute__((address_space(3))) void lds_void_t;

// One 16-byte-per-lane direct load: lane l's 16 bytes at src land at
// lds + 16*l.  (Kept in a device function of its own: the host compilation
// pass drops kernels that name this builtin directly.)
__device__ __forceinline__ void dma16(const void *src, lds_void_t *lds) {
  __builtin_amdgcn_global_load_lds(src, lds, 16, 0, 0);
}

// The same through a buffer resource (base and byte count uniform, lane l's
// 16 bytes at base + voff, zeros past the count).  While a load of the global
// form is in flight the compiler waits for every LDS read to complete before
// using any of them; with the buffer form it keeps partial waits.
constexpr int BUF_WORD3 = 0x00020000;   // resource word 3: 32-bit data format
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void *base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, bytes, BUF_WORD3);
}
__device__ __forceinline__ void buf16(__amdgpu_buffer_rsrc_t r, uint32_t voff, lds_void_t *lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds, 16, voff, 0, 0, 0);
}

// s_waitcnt immediate (vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt
// 11:8) that waits for LDS and scalar memory traffic only.
constexpr unsigned waitcnt_lgkm0 = 0xFu | (7u << 4) | (0u << 8) | (3u << 14);
// ... and the one that also waits for all vector memory traffic
constexpr unsigned waitcnt_vm0_lgkm0 = 7u << 4;

// Fused stage layout: two parts of 16 query rows.  Row r of part hi starts at
// element h1*hi + 32 + 105*r and holds distance index e (0..63 in use) at +e
// (h1: 16 when the parts are separate slices, below; else 0 with part 1 =
// part 0 + 16 rows).  The product for distance index idx = e + q of query
// q = 16*hi + r is written at 32 + 104*r + (h1 - 16)*hi + idx, so a lane's
// writes sit at fixed offsets from one per-lane base, and its runs of eight
// consecutive indices (idx = 8k .. 8k+7) are 16-byte aligned: one 16-byte
// store each.  The indices a lane also computes outside 0..63 (-31..95) land in the
// unused elements 64..104 of its own or the previous row, or in the part's
// head (writes and reads stay in elements 32..1700 of a separate slice).  A row starts on
// an odd element when r is odd, so the lanes read their 8-element runs as
// five 4-byte words and shift out one element.
// The two parts are either one stage of 32 rows or, in 4-wave work-groups
// over head_dim 128, the wave's own 4 KiB slices of the next K and V buffers,
// which are free until the wave issues its loads of the next tile.
constexpr int FUSED_ROW = 105;
constexpr int FUSED_PART1 = 16;

// Which matrices of a K/V tile a load issues, and which of the wave's writes
// (J < 0: all of them).
template <bool K, bool V, int J>
struct KVSel {
  static constexpr bool k = K, v = V;
  static constexpr int j = J;
};
// chunk swizzle of W^T row r in the fused variant's LDS buffers: rows are
// 2*DR bytes, 128/DR of them fill the 64 banks, so the swizzle steps once
// per that many rows
template <int DR>
__device__ __forceinline__ int wsl_swizzle(int r) {
  return (r / (128 / DR)) % (DR / 8);
}
constexpr int FUSED_STAGE = 32 + 32 * FUSED_ROW;

template <int D, int NW, bool BIG_PAGE, bool VEC_BIAS, int DR>
__global__ __launch_bounds__(64 * NW, 8 / NW) void prefill_bf16_kernel(PrefillArgs a) {
  constexpr bool FUSED = DR > 0;                // bias formed from r and W^T
  static_assert(!FUSED || ((NW == 8 || NW == 4) && (DR == 16 || DR == 32)),
                "fused variant: 4 or 8 waves, d_rel 16 or 32");
  // fused, 4 waves, head_dim 128: the bias stage lives in the next K/V buffer
  // (two work-groups then fit a CU's LDS)
  constexpr bool ALIAS = FUSED && NW == 4 && D == 128;
  constexpr int CHUNKS = D / 8;                 // 16-byte chunks per key row
  constexpr int KB = D / 16;                    // MFMA k-steps over head_dim
  constexpr int DSUB = D / 32;                  // 32-row slabs of O^T
  constexpr int ROWS_PER_DMA = 512 / D;         // key rows per 1 KiB LDS write
  constexpr int DMA_PER_WAVE = BN * D / 512 / NW;  // 1 KiB writes per wave per matrix
  // a fused stage part (writes up to element h1 - 16 + 32 + 15*104 + 95,
  // reads up to h1 + 32 + 15*105 + 56 + 9) fits the wave's slice of a K or V buffer
  static_assert(!ALIAS || (DMA_PER_WAVE * 512 > FUSED_PART1 + 32 + 15 * (FUSED_ROW - 1) + 99 &&
                           DMA_PER_WAVE * 512 > FUSED_PART1 + 32 + 15 * FUSED_ROW + 65),
                "stage part too large");
  static_assert(FUSED_ROW % 8 == 1 && FUSED_ROW > 96 && FUSED_PART1 % 8 == 0,
                "fused stage: 16-byte aligned runs of eight, rows apart by more than 96");
  // two K/V buffers as separate objects, so the compiler can tell that the
  // direct loads into one do not alias reads of the other
  __shared__ __align__(16) uint16_t k_lds0[BN * D], v_lds0[BN * D];
  __shared__ __align__(16) uint16_t k_lds1[BN * D], v_lds1[BN * D];
  // bias stage: per wave, 32 rows x 64 distances, 16-byte chunks of row r
  // XOR-swizzled by (r/2) mod 8 so the lanes' aligned reads avoid bank
  // conflicts (fused variant: the skewed layout above, unswizzled; none when
  // it lives in the K/V buffers)
  constexpr int STAGE_W = FUSED ? FUSED_STAGE : 32 * BN;
  uint16_t *stage_base = nullptr;
  if constexpr (!ALIAS) {
    __shared__ __align__(16) uint16_t bias_stage[NW * STAGE_W];
    stage_base = bias_stage;
  }
  // fused variant: two buffers of W^T rows (distances P0-s0-63 .. P0+QM-1-s0
  // of tile s0, P0 the work-group's first query position), QM+64 rows of DR
  // elements: at most 32*NW+64, and 128 in 4-wave work-groups, which the
  // host gives at least two heads (QM <= 64); the 16-byte chunks of row r are
  // XOR-swizzled by wsl_swizzle(r) so that 16 consecutive rows read on
  // distinct banks
  constexpr int WSL_ROWS = NW == 4 ? 128 : 32 * NW + 64;
  uint16_t *wsl0 = nullptr, *wsl1 = nullptr;
  if constexpr (FUSED) {
    __shared__ __align__(16) uint16_t w_sl0[WSL_ROWS * DR], w_sl1[WSL_ROWS * DR];
    wsl0 = w_sl0;
    wsl1 = w_sl1;
  }

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform per wave

  // Work-group -> (sequence, KV head, head group, query tile).  Blocks are
  // dealt to the 8 XCDs round-robin; remap so each XCD walks a contiguous
  // range, in which the head groups of one KV head and its query tiles
  // (heaviest first) are adjacent and share that XCD's L2.
  const int nb = a.num_blocks;
  const int bid = blockIdx.x;
  const int xcd = bid & 7, xidx = bid >> 3;
  const int base = nb >> 3, rem = nb & 7;
  const int r = (xcd < rem) ? xcd * (base + 1) + xidx
                            : rem * (base + 1) + (xcd - rem) * base + xidx;
  const int nqt = a.num_qtiles;
  const int hpw = a.hpw;                     // query heads per work-group
  const int ngroups = a.G / hpw;             // head groups per KV head
  const int per_seq = a.Hkv * ngroups * nqt;
  const int b = r / per_seq;
  int rr = r - b * per_seq;
  const int per_kvh = ngroups * nqt;
  const int kvh = rr / per_kvh;
  rr -= kvh * per_kvh;
  const int qt = nqt - 1 - rr / ngroups;
  const int hg = rr % ngroups;
  const int QM = 32 * (NW / hpw);            // queries per head per work-group
  if constexpr (FUSED && WSL_ROWS < 32 * NW + 64) {
    if (QM + 64 > WSL_ROWS) return;          // W^T rows would not fit (the host never asks)
  }
  // this wave: head slot wave % hpw, query block wave / hpw
  const int h = kvh * a.G + hg * hpw + wave % hpw;
  const int qb = wave / hpw;

  const int tok0 = a.cu_seqlens[b];
  const int L = a.cu_seqlens[b + 1] - tok0;  // this call's query tokens of the sequence
  const int t0 = qt * QM;
  if (t0 >= L) return;
  // The sequence holds n_k keys, this call's included, and the call's L
  // tokens are its last L positions: token index i sits at position
  // hist + i (no key count given: no history).
  const int n_k = a.seq_lens != nullptr ? max(a.seq_lens[b], L) : L;
  const int hist = n_k - L;
  const int tq0 = t0 + 32 * qb;              // this wave's first query (token index)
  const int pq0 = hist + tq0;                // and its position

  const int Hq = a.Hq;
  const int R = a.R;
  const int W = a.window;
  const int p_last = hist + min(t0 + QM, L) - 1;   // position of the work-group's last query
  // first key any query of the work-group sees (its first query's window start)
  const int s_first = (W > 0) ? max(0, hist + t0 - W + 1) : 0;
  const int s_begin = s_first & ~(BN - 1);

  // Key tile s0 (a multiple of BN) against this wave's queries at positions
  // pq0..pq0+31, each test one compare with a per-wave bound (d = p - s
  // ranges over [pq0 - s0 - 63, pq0 + 31 - s0]):
  //   active     s_lo < s0 <= s_hi  some key is visible
  //   band       s0 > s_band        some distance is below R-1, or at most
  //                                 R-1 on narrow layers (bias staged)
  //   masked     s0 > s_diag, s0 <= s_wedge or s0 > s_tail
  //              (causal diagonal, window edge, sequence end inside the tile)
  //   beyond     s0 <= s_strad      some distance exceeds R-1
  const int s_hi = pq0 + 31;
  const int s_lo = (W > 0) ? pq0 - (BN - 1) - W : INT_MIN;
  // A layer whose window stays within the R buckets (narrow) never sees a
  // distance beyond R-1 inside its window.  With the streamed bias, its band
  // also takes the tiles whose smallest distance is exactly R-1: the stage
  // then holds every visible distance, bucket R-1 included, and the clamped
  // bucket is never read on its own.
  const bool wide_layer = W <= 0 || W > R;
  const int s_band = pq0 - (BN - 2) - R - ((FUSED || wide_layer) ? 0 : 1);
  const int s_diag = pq0 - (BN - 1);
  const int s_wedge = (W > 0) ? pq0 + 31 - W : INT_MIN;
  const int s_tail = n_k - BN;
  const int s_strad = pq0 + 31 - R;
  // The same tests as single unsigned range compares, s0 - lo - 1 < span
  // (tiles are never below 0, so lower bounds under -1 are clamped to -1):
  //   active     lo = max(s_lo, -1),        up to s_hi
  //   band       lo = max(s_lo, s_band, -1), up to s_hi (active and band)
  //   path 0     lo = max(s_wedge, -1), up to min(s_diag, s_tail, s_band):
  //              active, unmasked and clamp-only
  const int act_lo = max(s_lo, -1);
  const uint32_t act_span = (uint32_t)(s_hi - act_lo);
  const int band_lo = max(max(s_lo, s_band), -1);
  const uint32_t band_span = (uint32_t)max(s_hi - band_lo, 0);
  const int p0_lo = max(s_wedge, -1);
  const uint32_t p0_span = (uint32_t)max(min(min(s_diag, s_tail), s_band) - p0_lo, 0);
  auto in_range = [](int s0, int lo, uint32_t span) { return (uint32_t)(s0 - lo - 1) < span; };

  const uint16_t *qp = static_cast<const uint16_t *>(a.q);
  const uint16_t *kp = static_cast<const uint16_t *>(a.k_pool);
  const uint16_t *vp = static_cast<const uint16_t *>(a.v_pool);
  const int32_t *trow = a.block_table + (size_t)b * a.max_pages;
  const int P = a.page_size;
  const int lp = a.log2_page;
  const size_t head_stride = (size_t)P * D;           // elements per (page, head)
  const size_t page_stride = (size_t)a.Hkv * head_stride;

  // ---- this lane's query row --------------------------------------------
  const int col = lane & 31;
  const int half = lane >> 5;
  const int t = tq0 + col;                   // token index
  const int p = hist + t;                    // position
  const bool row_ok = t < L;
  const size_t row = ((size_t)tok0 + (row_ok ? t : 0)) * Hq + h;

  u32x4_t qf[KB];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    const u32x4_t v = *reinterpret_cast<const u32x4_t *>(qp + row * D + kb * 16 + half * 8);
    qf[kb] = row_ok ? v : u32x4_t{0, 0, 0, 0};
  }

  // Bias row of this lane's query.  A tile a wave reads bias for has every
  // distance of the wave inside [-94, R + 94), so the staged 64-distance rows
  // stay inside the bias tensor except for rows within 1024 elements of
  // either end of it: waves holding such a row read element by element with
  // distances clamped to [0, R) instead.  Values read outside [0, R) are
  // masked or replaced by the clamped bucket, which only wide layers use
  // (narrow ones never read it).
  //
  // Fused variant: this lane's B operand of the bias product, r[row] in
  // k-steps of 16 (lane half `half` holds elements 8*half .. 8*half+7 of
  // each), and the clamped bucket r[row] . W[:,R-1] formed in fp32 and
  // rounded to bf16.
  const uint16_t *brow = nullptr;
  float b_last;
  bool edge_wave;
  u32x4_t rf[FUSED ? DR / 16 : 1];
  if constexpr (FUSED) {
    const uint16_t *rp = static_cast<const uint16_t *>(a.rel_r);
    const uint16_t *wlast = static_cast<const uint16_t *>(a.w_rel_t) + (size_t)(R - 1) * DR;
    float part = 0.f;
#pragma unroll
    for (int kk = 0; kk < DR / 16; ++kk) {
      const u32x4_t v = *reinterpret_cast<const u32x4_t *>(rp + row * DR + kk * 16 + half * 8);
      rf[kk] = row_ok ? v : u32x4_t{0, 0, 0, 0};
      const u32x4_t w = *reinterpret_cast<const u32x4_t *>(wlast + kk * 16 + half * 8);
#pragma unroll
      for (int x = 0; x < 8; ++x) part = fmaf(bf16x8_elem(rf[kk], x), bf16x8_elem(w, x), part);
    }
    // rounded to bf16 like every other bias entry this variant forms
    const float bl = part + __shfl_xor(part, 32);
    b_last = bf16_to_f32(pack_bf16x2(bl, bl) & 0xffffu);
    edge_wave = false;
  } else {
    brow = static_cast<const uint16_t *>(a.bias) + row * R;
    b_last = wide_layer ? bf16_to_f32(brow[R - 1]) : 0.f;
    const long long row_off = (long long)row * R;
    const long long bias_elems = (long long)a.total_tokens * Hq * R;
    edge_wave = __ballot(row_off < 1024 || bias_elems - row_off < R + 1024) != 0;
  }

  // ---- K/V tile loads, global -> LDS -------------------------------------
  // Write j of this wave fills LDS rows (DMA_PER_WAVE*wave + j)*ROWS_PER_DMA
  // + lane/CHUNKS, physical chunk lane%CHUNKS, which holds logical chunk
  // (lane%CHUNKS) ^ swizzle(row) of the key row.
  const u32x4_t zero4 = {0, 0, 0, 0};
  int dma_row[DMA_PER_WAVE];            // tile row this lane fills, per write
  uint32_t k_off[DMA_PER_WAVE], v_off[DMA_PER_WAVE];   // byte offset inside the row
#pragma unroll
  for (int j = 0; j < DMA_PER_WAVE; ++j) {
    const int rw = (DMA_PER_WAVE * wave + j) * ROWS_PER_DMA + lane / CHUNKS;
    const int pc = lane % CHUNKS;
    dma_row[j] = rw;
    k_off[j] = (uint32_t)((pc ^ (rw & (CHUNKS - 1))) * 16);
    v_off[j] = (uint32_t)((pc ^ v_swizzle<D>(rw)) * 16);
  }

  // `page` is the pool page of the tile when pages hold whole tiles; it is
  // read from the block table one tile ahead of its use, so the table read
  // never sits in front of the tile's loads.
  const char *k_head = reinterpret_cast<const char *>(kp + (size_t)kvh * head_stride);
  const long long v_minus_k = reinterpret_cast<const char *>(vp) - reinterpret_cast<const char *>(kp);
  const uint32_t page_bytes = (uint32_t)(page_stride * 2);   // checked on the host to fit
  // (sel_tag: which matrices and writes, a KVSel, known at compile time.)
  auto load_kv_sel = [&](auto sel_tag, int s0, int page_v, uint16_t *kl, uint16_t *vl) {
    using SEL = decltype(sel_tag);
    // Rows below `first` repeat the work-group's first visible key, rows
    // above `last` the sequence's last key: only keys some query of the
    // work-group sees are ever read (a 0 probability times a finite value is
    // an exact 0 in the PV product; a non-finite one would not be).
    const int first = s_first - s0;
    const int last = n_k - 1 - s0;
    if constexpr (BIG_PAGE) {
      // the 64-key tile lies inside one page
      const uint32_t page = (uint32_t)__builtin_amdgcn_readfirstlane(page_v);
      const char *kt = k_head + ((uint64_t)page * page_bytes + (uint32_t)((s0 & (P - 1)) * D * 2));
      const char *vt = kt + v_minus_k;
      // resources over the tile's BN rows
      const __amdgpu_buffer_rsrc_t rk = buf_rsrc(kt, BN * D * 2), rv = buf_rsrc(vt, BN * D * 2);
#pragma unroll
      for (int j = 0; j < DMA_PER_WAVE; ++j) {
        if (SEL::j >= 0 && j != SEL::j) continue;
        const uint32_t ro = (uint32_t)min(max(dma_row[j], first), last) * (D * 2);
        if constexpr (SEL::k) buf16(rk, ro + k_off[j], (lds_void_t *)(kl + (DMA_PER_WAVE * wave + j) * 512));
        if constexpr (SEL::v) buf16(rv, ro + v_off[j], (lds_void_t *)(vl + (DMA_PER_WAVE * wave + j) * 512));
      }
    } else {
#pragma unroll
      for (int j = 0; j < DMA_PER_WAVE; ++j) {
        if (SEL::j >= 0 && j != SEL::j) continue;
        const int sk = s0 + min(max(dma_row[j], first), last);
        const size_t ko = ((size_t)trow[sk >> lp] * page_stride + (size_t)kvh * head_stride +
                           (size_t)(sk & (P - 1)) * D) * 2;
        if constexpr (SEL::k)
          dma16(reinterpret_cast<const char *>(kp) + ko + k_off[j], (lds_void_t *)(kl + (DMA_PER_WAVE * wave + j) * 512));
        if constexpr (SEL::v)
          dma16(reinterpret_cast<const char *>(vp) + ko + v_off[j], (lds_void_t *)(vl + (DMA_PER_WAVE * wave + j) * 512));
      }
    }
  };

  auto load_kv = [&](int s0, int page_v, uint16_t *kl, uint16_t *vl) {
    load_kv_sel(KVSel<true, true, -1>{}, s0, page_v, kl, vl);
  };

  // ---- bias runs ---------------------------------------------------------
  // For key tile s0, run p (p = 2*sub + G) holds the distances
  // t - s0 - 8*half - 16*p - 7 .. t - s0 - 8*half - 16*p in ascending order,
  // i.e. the keys s0 + 32*sub + 16*G + 8*half + 7 down to + 0: chunk
  // 7 - half - 2p of the row's 64 staged distances t - s0 - 63 .. t - s0.
  const bool use_stage = FUSED || (VEC_BIAS && !edge_wave);
  uint16_t *stage_w = ALIAS ? nullptr : stage_base + wave * STAGE_W;
  // Fused stage part of this lane's query row, given the step's next K/V
  // buffers, and this lane's offsets in it: write base (element 4*half of
  // distance index 0) and row start.
  // (One stage: parts 0 and 1 are contiguous, so rows count from part 0.)
  auto fused_part = [&](uint16_t *kn, uint16_t *vn) {
    if constexpr (ALIAS) return (col < 16 ? kn : vn) + DMA_PER_WAVE * wave * 512;
    else return stage_w;
  };
  const int frow = ALIAS ? (col & 15) : col;
  const int fw_off = 32 + (FUSED_ROW - 1) * frow + (ALIAS ? (FUSED_PART1 - 16) * (col >> 4) : 0) + 8 * half;
  const int fr_off = 32 + FUSED_ROW * frow + (ALIAS ? FUSED_PART1 * (col >> 4) : 0);
  // the row start's element parity: a run is read as five words from the
  // word holding its first element, shifted right by fr_shift bytes
  const uint32_t fr_shift = 2u * (uint32_t)(fr_off & 1);
  const int fr_word = fr_off >> 1;
  // Stage write k of this lane: row 8k + lane/8 of the wave, physical chunk
  // lane%8 = logical chunk c ^ swizzle.  The loads go through a resource
  // over the wave's 32 bias rows, from 128 elements before its first row (a
  // wave wholly past the sequence takes the sequence's last row instead, so
  // the resource never starts past the tensor); sofs is the byte offset of
  // tile 0, tile s0 is s0 elements lower.  A staged distance is at least -94,
  // so every offset stays above 68 bytes, and at most R + 100 elements past
  // its row start.  Rows of queries past the sequence get an offset of at
  // least 2^31 for every tile (positions stay below 2^29), beyond the record
  // count: the hardware returns zeros for them without a memory access, and
  // their outputs are never stored.
  const int tq_base = min(tq0, L - 1);
  const size_t srow0 = ((size_t)tok0 + tq_base) * Hq + h;
  const __amdgpu_buffer_rsrc_t rstage = buf_rsrc(
      static_cast<const uint16_t *>(a.bias) + ((long long)srow0 * R - 128),
      (int)min(((long long)31 * Hq * R + R + 256) * 2, (long long)INT_MAX));
  uint32_t sofs[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int rq = 8 * k + (lane >> 3);
    const int tq = tq0 + rq;
    const int c = (lane & 7) ^ ((rq >> 1) & 7);
    sofs[k] = (tq < L) ? (uint32_t)((((long long)(tq - tq_base) * Hq) * R + 128 + hist + tq - (BN - 1) + 8 * c) * 2)
                       : 0xC0000000u;
  }
  auto stage_bias = [&](int s0) {       // direct loads, tile s0 -> this wave's stage
#pragma unroll
    for (int k = 0; k < 4; ++k) buf16(rstage, sofs[k] - 2 * (uint32_t)s0, (lds_void_t *)(stage_w + k * 512));
  };
  auto load_bias = [&](int s0, u32x4_t (&bp)[4], const uint16_t *part) {
    if constexpr (FUSED) {
#pragma unroll
      for (int p = 0; p < 4; ++p)
      {
        const uint32_t *wp = reinterpret_cast<const uint32_t *>(part) + fr_word + (7 - half - 2 * p) * 4;
        uint32_t w[5];
#pragma unroll
        for (int k = 0; k < 5; ++k) w[k] = wp[k];
#pragma unroll
        for (int k = 0; k < 4; ++k) bp[p][k] = __builtin_amdgcn_alignbyte(w[k + 1], w[k], fr_shift);
      }
    } else if (use_stage) {
      const int sw = (col >> 1) & 7;
#pragma unroll
      for (int p = 0; p < 4; ++p)
        bp[p] = *reinterpret_cast<const u32x4_t *>(stage_w + col * BN + (((7 - half - 2 * p) ^ sw) * 8));
    } else {
      const int ds0 = p - s0 - 8 * half - 7;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        u32x4_t v = zero4;
#pragma unroll
        for (int x = 0; x < 8; ++x) {
          const int d = min(max(ds0 - 16 * p + x, 0), R - 1);
          v[x >> 1] |= (uint32_t)brow[d] << ((x & 1) * 16);
        }
        bp[p] = v;
      }
    }
  };

  // ---- fused variant: W^T rows and the bias product ---------------------------
  // The W^T buffer of tile s0 holds rows d0 .. d0 + QM + 63 of W^T, clamped to
  // [0, R-1], with d0 = P0 - s0 - 63 the smallest distance of the work-group's
  // first query P0 (finite values for distances below 0, which are masked).
  // Wave (query block qb) reads rows 32*qb .. 32*qb + 95: distance index idx
  // of its query q is distance pq0 + q - s0 - 63 + (idx - q).
  const int P0 = hist + t0;
  // some wave of the work-group reads bias for tile s0: the first query
  // block (qb = 0, queries from P0) meets the smallest distances
  auto wg_band = [&](int s0) { return s0 > P0 - (BN - 2) - R; };
  auto load_wslice = [&](int s0, uint16_t *dst) {
    if constexpr (FUSED) {
      constexpr int LPR = DR / 8;        // lanes per W^T row (16 bytes each)
      constexpr int RPI = 64 / LPR;      // rows per 1 KiB direct load
      const __amdgpu_buffer_rsrc_t rw = buf_rsrc(a.w_rel_t, R * DR * 2);
      const int n_ld = (QM + 64) / RPI;
      const int d0 = P0 - s0 - (BN - 1);
      for (int i = wave; i < n_ld; i += NW) {
        const int rr = i * RPI + lane / LPR;                 // buffer row this lane fills
        const int dd = min(max(d0 + rr, 0), R - 1);
        const int c = (lane % LPR) ^ wsl_swizzle<DR>(rr);    // logical chunk it fetches
        buf16(rw, (uint32_t)((dd * DR + c * 8) * 2), (lds_void_t *)(dst + i * 512));
      }
    }
  };
  // Bias of tile s0 for this wave's 32 queries into its stage: C^T = W^T r^T
  // over 96 distance indices in three 32-row MFMA blocks (A = W^T rows from
  // the buffer, B = r), rounded to bf16.  Output row m of a block is A row m,
  // which lane m loads from W^T row sigma(m) of the block: sigma swaps bits 2
  // and 3 of m, so register 4i+j holds index idx = 32b + 16(i/2) + 8*half +
  // 4(i%2) + j of query col, and registers 8k .. 8k+7 hold the eight
  // consecutive indices 32b + 16k + 8*half + 0..7, written at
  // fw_off - 8*half + idx of the lane's stage part.
  auto fuse_bias = [&](const uint16_t *wsl, uint16_t *part) {
    if constexpr (FUSED) {
      // row 32*qb + 32*b + sigma(col), logical chunk 2*kk + half (the
      // swizzle of a row depends on the row mod 32 only); the 16 rows a
      // 16-lane group reads are the same set as without sigma
      const int arow = (col & ~12) | ((col & 4) << 1) | ((col & 8) >> 1);
      const int wsw = wsl_swizzle<DR>(arow);
      const uint16_t *wa = wsl + (32 * qb + arow) * DR;
      // 16-byte stores of eight consecutive indices (16-byte aligned)
      typedef __attribute__((address_space(3))) u32x4_t lds_u32x4_t;
      lds_u32x4_t *sb = (lds_u32x4_t *)(part + fw_off);
#pragma unroll
      for (int b = 0; b < 3; ++b) {
        f32x16_t acc;
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[j] = 0.f;
#pragma unroll
        for (int kk = 0; kk < DR / 16; ++kk) {
          const u32x4_t w = *reinterpret_cast<const u32x4_t *>(wa + 32 * b * DR + ((2 * kk + half) ^ wsw) * 8);
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, w),
                                                        __builtin_bit_cast(bf16x8_t, rf[kk]), acc, 0, 0, 0);
        }
#pragma unroll
        for (int k = 0; k < 2; ++k)   // indices 32b + 16k + 8*half .. +7: element offset 32b + 16k
          sb[(32 * b + 16 * k) / 8] = u32x4_t{pack_bf16x2(acc[8 * k], acc[8 * k + 1]),
                                              pack_bf16x2(acc[8 * k + 2], acc[8 * k + 3]),
                                              pack_bf16x2(acc[8 * k + 4], acc[8 * k + 5]),
                                              pack_bf16x2(acc[8 * k + 6], acc[8 * k + 7])};
      }
    }
  };

  // ---- accumulators ------------------------------------------------------
  f32x16_t oacc[DSUB];
#pragma unroll
  for (int i = 0; i < DSUB; ++i)
#pragma unroll
    for (int j = 0; j < 16; ++j) oacc[i][j] = 0.f;
  float m2 = NEG_INIT;   // running max, log2 units, shared by the lane pair
  float lsum = 0.f;      // this lane's share of the softmax denominator
  const float scale = a.sm_scale;
  const float scale2 = scale * LOG2E;

  // ---- LDS read addressing ---------------------------------------------------
  // K operand: lane supplies S^T row col = key key_of_row(col) (+32 for the
  // second key block), chunk (2kb + half) ^ (key mod CHUNKS) = (2kb) ^ kx.
  const int krow = key_of_row(col);
  const int kx = half ^ (krow & (CHUNKS - 1));
  const int kbase = krow * D;
  // V operand via the transposing read: this lane supplies the address of
  // key ks*16 + 8*(g/2) + kk (+4 for k-slots 4..7), head-dim elements
  // ds*32 + 16*(g%2) + 4*i .. +3, where g = lane/16, kk = (lane/4)%4, i = lane%4.
  // The read hands lane 16g+4i+j element j of lanes 16g+i+4kk, kk = 0..3, which
  // is row d = ds*32 + lane%32 of V^T at keys ks*16 + 8*half + 0..3 (+4).
  const int vg = lane >> 4, vkk = (lane >> 2) & 3, vi = lane & 3;
  const int vrow = 8 * (vg >> 1) + vkk;
  const int vchunk_lo = 2 * (vg & 1) + (vi >> 1);        // chunk within a 32-wide slab
  const int vsw = v_swizzle<D>(vrow);                   // rows ks*16+vrow(+4) share it
  const int vbase = vrow * D + (vi & 1) * 4;

  // S^T block of keys 32*sub .. 32*sub+31 of the K tile at kl (8 MFMAs over
  // head_dim).
  auto s_block = [&](const uint16_t *kl, int sub) {
    f32x16_t acc;
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[j] = 0.f;
    const uint16_t *kb0 = kl + kbase + sub * 32 * D;
    u32x4_t kf[2];
    kf[0] = *reinterpret_cast<const u32x4_t *>(kb0 + (kx * 8));
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      if (kb + 1 < KB)
        kf[(kb + 1) & 1] = *reinterpret_cast<const u32x4_t *>(kb0 + (((2 * (kb + 1)) ^ kx) * 8));
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, kf[kb & 1]),
                                                    __builtin_bit_cast(bf16x8_t, qf[kb]), acc, 0, 0, 0);
    }
    return acc;
  };
  auto max16 = [&](const f32x16_t &acc) {
    // a chain of two-input maxes, which the compiler fuses into v_max3
    float m = fmaxf(acc[0], acc[1]);
#pragma unroll
    for (int j = 2; j < 16; j += 2) m = fmaxf(fmaxf(m, acc[j]), acc[j + 1]);
    return m;
  };
  // P = exp2(score - max) in bf16, as the PV MFMA consumes it; the row sum
  // adds exactly these rounded values, two per v_dot2 against (1, 1).
  // (sa: the exp2 argument's multiplier, c2 its offset)
  auto probs = [&](f32x16_t &acc, float sa, float c2, u32x4_t (&pw)[2]) {
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[j] = __builtin_amdgcn_exp2f(fmaf(acc[j], sa, c2));
#pragma unroll
    for (int j = 0; j < 8; ++j) pw[j >> 2][j & 3] = pack_bf16x2(acc[2 * j], acc[2 * j + 1]);
    const bf16x2_t one2 = {(__bf16)1.0f, (__bf16)1.0f};
    float r0 = 0.f, r1 = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      // (bit_cast of a vector element lvalue reads element 0: copy it out first)
      const uint32_t w0 = pw[0][j], w1 = pw[1][j];
      r0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w0), one2, r0, false);
      r1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w1), one2, r1, false);
    }
    lsum += r0 + r1;
  };
  // O^T += V^T P^T over keys 32*sub .. 32*sub+31 of the V tile at vl, 16 keys
  // per MFMA.  k-slots of lane half `half` in step ks are keys ks*16 + 8*half
  // + 0..7: exactly S^T registers 8*(ks&1) + 0..7, and exactly the keys the
  // two transposing reads deliver.
  auto pv_block = [&](const uint16_t *vl, const u32x4_t (&pw)[2], int sub) {
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      const int ks = 2 * sub + kh;
      const bf16x8_t pb = __builtin_bit_cast(bf16x8_t, pw[kh]);
#pragma unroll
      for (int ds = 0; ds < DSUB; ++ds) {
        const uint16_t *v0 = vl + vbase + ks * 16 * D + (((ds * 4) | vchunk_lo) ^ vsw) * 8;
        const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)(v0));
        const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)(v0 + 4 * D));
        const u32x2_t lw = __builtin_bit_cast(u32x2_t, lo);
        const u32x2_t hw = __builtin_bit_cast(u32x2_t, hi);
        const bf16x8_t vb = __builtin_bit_cast(bf16x8_t, u32x4_t{lw[0], lw[1], hw[0], hw[1]});
        oacc[ds] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vb, pb, oacc[ds], 0, 0, 0);
      }
    }
  };

  // Lazy rescale, decided per lane on its own 32 scores: while neither lane
  // of a pair sees a score above m2 + TAU the shared m2 stands, with no
  // exchange; otherwise the pair's maximum is formed and both lanes move
  // m2 to it (mt2: this lane's tile maximum in log2 units).
  auto rescale = [&](float mt2) {
    if (__ballot(mt2 > m2 + TAU)) {
      const float mtp = fmaxf(mt2, __shfl_xor(mt2, 32));
      const bool exceed = mtp > m2 + TAU;
      const float mnew = exceed ? mtp : m2;
      const float alpha = __builtin_amdgcn_exp2f(m2 - mnew);
      lsum *= alpha;
#pragma unroll
      for (int i = 0; i < DSUB; ++i)
#pragma unroll
        for (int j = 0; j < 16; ++j) oacc[i][j] *= alpha;
      m2 = mnew;
    }
  };

  // fixed_tag: std::integral_constant<bool, true> on tiles known (for the
  // whole work-group) to be clamp-only and unmasked, which then compile to
  // score path 0 with no classification, bias or mask code at all.
  auto compute_tile = [&](auto fixed_tag, int s0, const uint16_t *kl, const uint16_t *vl,
                          const u32x4_t (&bp)[4]) {
    constexpr bool FIXED = decltype(fixed_tag)::value;
    const bool fixed0 = FIXED || in_range(s0, p0_lo, p0_span);   // clamp-only, unmasked
    if (!fixed0 && !in_range(s0, act_lo, act_span)) return;   // no key of the tile is visible
    const bool need_mask = s0 > s_diag || s0 <= s_wedge || s0 > s_tail;
    const bool band = s0 > s_band;
    const bool beyond = s0 <= s_strad;         // some distance exceeds R-1
    // score path: 0 clamp-only unmasked, 1 band unmasked, 2 general (a band
    // tile with a visible distance beyond R-1 is one of the edges)
    const int path = fixed0 ? 0 : ((!need_mask && !(beyond && wide_layer)) ? 1 : 2);
    const bool clamp_free = band && (!wide_layer || !beyond);
    // exp2 argument = fma(v, sa, sb - m2): v is the raw q.k on path 0 (scale
    // and the clamped bias folded into sa, sb), the finished score otherwise
    const float sa = (path == 0) ? scale2 : LOG2E;
    const float sb = (path == 0) ? b_last * LOG2E : 0.f;

    // Element j of 32-key half `sub` is key s0 + 8*half + koff,
    // koff = 32*sub + 16*(j>>3) + (j&7), at distance dq - koff.
    const int dq = p - s0 - 8 * half;

    // Finished scores of a block on paths 1 and 2 (path 0 keeps the raw q.k).
    auto finish = [&](f32x16_t &acc, int sub) {
      if (path == 1) {
#pragma unroll
        for (int j = 0; j < 16; ++j)
          acc[j] = fmaf(acc[j], scale, bf16x8_elem(bp[2 * sub + (j >> 3)], 7 - (j & 7)));
      } else if (path == 2) {
        // visible iff kv_lo < koff <= kv_hi, i.e. (unsigned)(koff - kv_lo - 1) < span
        const int kv_hi = min(dq, n_k - 1 - s0 - 8 * half);
        const int kv_lo1 = (W > 0) ? dq - W + 1 : -(1 << 30);
        const uint32_t span = (uint32_t)max(kv_hi - kv_lo1 + 1, 0);
        if (clamp_free) {
          // every visible distance is at most R-1: all of them are staged
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const int koff = 32 * sub + 16 * (j >> 3) + (j & 7);
            const float x = fmaf(acc[j], scale, bf16x8_elem(bp[2 * sub + (j >> 3)], 7 - (j & 7)));
            acc[j] = ((uint32_t)(koff - kv_lo1) < span) ? x : -INFINITY;
          }
        } else {
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const int koff = 32 * sub + 16 * (j >> 3) + (j & 7);
            const float bv = (band && dq - koff < R - 1)
                                 ? bf16x8_elem(bp[2 * sub + (j >> 3)], 7 - (j & 7)) : b_last;
            const float x = fmaf(acc[j], scale, bv);
            acc[j] = ((uint32_t)(koff - kv_lo1) < span) ? x : -INFINITY;
          }
        }
      }
    };

    // Both S^T blocks, then both blocks' scores, exponentials and P V.  (A
    // wave's own MFMAs and vector instructions do not run side by side; the
    // two waves of a SIMD overlap each other's.)  The running max is updated
    // once per tile.
    f32x16_t sa0 = s_block(kl, 0);
    f32x16_t sa1 = s_block(kl, 1);
    finish(sa0, 0);
    const float mx0 = max16(sa0);
    finish(sa1, 1);
    rescale(fmaf(fmaxf(mx0, max16(sa1)), sa, sb));
    const float c2 = sb - m2;
    u32x4_t pw0[2], pw1[2];
    probs(sa0, sa, c2, pw0);
    pv_block(vl, pw0, 0);
    probs(sa1, sa, c2, pw1);
    pv_block(vl, pw1, 1);
  };

  // ---- main loop -------------------------------------------------------------
  // Tile i computes from K/V buffer i%2 while tile i+1's K/V stream into the
  // other buffer and its bias rows into the wave's stage (after the lanes
  // have copied tile i's runs out of it); the barrier closing tile i waits
  // for both.  Unrolled by two so each buffer is fixed at compile time.
  auto wave_band = [&](int s0) {      // this wave computes tile s0 and reads its bias
    return in_range(s0, band_lo, band_span);
  };

  // bias runs of the current tile (in 8-wave work-groups set before the
  // first general step, so that they are not live across the two-group
  // phase below)
  u32x4_t bias_r[4];
  auto clear_bias_r = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i) bias_r[i] = zero4;
  };
  if constexpr (NW != 8) clear_bias_r();
  // Page of tile s (0 past the last tile, where it is not used).  The index
  // carries an opaque zero so the value stays in a vector register until
  // load_kv reads it, instead of being moved to a scalar register (and
  // waited for) right after the load.
  const int opaque_zero = (int)__builtin_amdgcn_mbcnt_lo(0u, 0u);   // 0 in every lane
  auto tile_page = [&](int s) {       // s is always a tile of this work-group
    return BIG_PAGE ? trow[(s >> lp) + opaque_zero] : 0;
  };
  // One tile: bias runs of tile s0 into registers, then the loads of tile
  // sn = s0 + BN, then the compute of tile s0.
  // Key tiles T_first .. T_last of this work-group are visited in rotated
  // order, tile index = step (mod n_t): on a windowed layer the interior
  // work-groups of one head span the same number of tiles, so every
  // work-group that needs a K/V tile loads it in the same step and the
  // co-resident ones share it in L2.  (The online softmax does not depend on
  // the order; on global layers T_first = 0 and the order is the natural one,
  // which already aligns the work-groups.)
  const int T_first = s_begin / BN;
  const int n_t = p_last / BN - T_first + 1;
  const int rot = (n_t - T_first % n_t) % n_t;
  const int s_tfirst = T_first * BN, s_tlast = (T_first + n_t - 1) * BN;
  auto tile_after = [&](int s) { return s == s_tlast ? s_tfirst : s + BN; };
  // s_cur, s_nxt, s_nxt2: tiles of this step and the next two (the sequence
  // wraps, so all three are always tiles of this work-group); page_nxt is
  // the pool page of s_nxt, read one step ahead.
  int s_cur = (T_first + rot) * BN;
  int s_nxt = tile_after(s_cur);
  int s_nxt2 = tile_after(s_nxt);
  int steps_left = n_t;
  // One step: bias runs of tile s_cur into registers, then the loads of
  // s_nxt (unless s_cur is the last), then the compute of s_cur.
  // (Fused variant: the bias product of tile s_cur goes into the stage first,
  // from the W^T buffer loaded with the tile; the W^T rows of s_nxt load with
  // its K/V into the other buffer.)
  auto step = [&](auto fixed_tag, uint16_t *kc, uint16_t *vc, uint16_t *kn, uint16_t *vn,
                  const uint16_t *wc, uint16_t *wn, int &page_nxt) {
    constexpr bool FIXED = decltype(fixed_tag)::value;
    const int s0 = s_cur;
    const bool more = --steps_left > 0;
    if (!FIXED && wave_band(s0)) {
      uint16_t *part = fused_part(kn, vn);
      fuse_bias(wc, part);
      load_bias(s0, bias_r, part);
    }
    if (more) {
      // a stage in the next K/V buffers: this lane's reads of it must be
      // done before the loads below overwrite it
      if constexpr (ALIAS) __builtin_amdgcn_s_waitcnt(waitcnt_lgkm0);
      load_kv(s_nxt, page_nxt, kn, vn);
      page_nxt = tile_page(s_nxt2);
      if constexpr (FUSED) {
        if (wg_band(s_nxt)) load_wslice(s_nxt, wn);
      } else if (use_stage && wave_band(s_nxt)) {
        // the stage is rewritten: this lane's reads of it must be done
        __builtin_amdgcn_s_waitcnt(waitcnt_lgkm0);
        stage_bias(s_nxt);
      }
    }
    compute_tile(fixed_tag, s0, kc, vc, bias_r);
    __syncthreads();
    s_cur = s_nxt;
    s_nxt = s_nxt2;
    s_nxt2 = tile_after(s_nxt2);
    return more;
  };

  load_kv(s_cur, tile_page(s_cur), k_lds0, v_lds0);
  if constexpr (FUSED) {
    if (wg_band(s_cur)) load_wslice(s_cur, wsl0);
  } else if (use_stage && wave_band(s_cur)) {
    stage_bias(s_cur);
  }
  int page_nxt = tile_page(s_nxt);
  __syncthreads();

  // Global layers visit their tiles in natural order from 0, and the leading
  // ones, up to the last tile at distance >= R-1 from the work-group's first
  // query (and before the sequence's last tile), are clamp-only and
  // unmasked for every wave: they run a loop of their own with the score
  // path fixed at compile time.  The diagonal tile is never among them, so
  // the general loop always follows.
  typedef std::integral_constant<bool, true> FixedTile;
  typedef std::integral_constant<bool, false> AnyTile;
  int n_fixed = 0;
  if (W <= 0) {
    const int lim = min(P0 - (BN - 2) - R, n_k - BN);
    n_fixed = lim < 0 ? 0 : min(lim / BN + 1, n_t - 1);
  }
  bool go = true;
  if constexpr (NW == 8) {
    if (n_fixed > 0) {
      // Two wave groups in opposite phases.  A SIMD runs one wave's matrix
      // instructions beside another wave's vector instructions, but not
      // beside its own, and waves w and w+4 share a SIMD.  Every wave runs
      // M(j) (P V of tile j-1, then S^T of tile j: matrix work), a barrier,
      // V(j) (the probabilities of tile j: vector work), a barrier, for
      // j = 0, 1, ...; the lead group (waves 0-3) starts one barrier ahead,
      // so its M(j) runs in phase 2j beside the other group's V(j-1), and
      // its V(j) in phase 2j+1 beside the other group's M(j).  A wave's
      // arithmetic is that of the one-phase step, in the same order.
      // K(j) is read in phases 2j and 2j+1, V(j) in 2j+2 and 2j+3.  In phase
      // 2j every wave issues its slices of K(j+1) and V(j), into the buffers
      // that K(j-1) and V(j-2) last used in phase 2j-1; they are waited for
      // at the end of phase 2j+1.  A wave's direct loads stall its issue
      // while the memory pipeline is busy, so each wave spreads its loads
      // through its phase: the lead group between its MFMAs, the other
      // between the steps of its vector work.
      const int n = n_fixed;
      const bool lead = wave < 4;
      const float sb0 = b_last * LOG2E;
      f32x16_t ps0, ps1;                // S^T of a tile, from its M to its V
      u32x4_t pp0[2], pp1[2];           // its P, from its V to the next M
      // Loads of phase 2t: K(t+1) while t < n with the page in pk, V(t) from
      // t = 1 (V(0) came with K(0)) with the page in pv.
      auto pp_dma = [&](int t, uint16_t *kn, uint16_t *vc, int pv, int pk) {
        if (t < n) load_kv_sel(KVSel<true, false, -1>{}, (t + 1) * BN, pk, kn, kn);
        if (t > 0) load_kv_sel(KVSel<false, true, -1>{}, t * BN, pv, vc, vc);
      };
      // The rest of phase 2t's loads: at t = n each wave's bias stage or W^T
      // rows of tile t; then pv takes the page of tile t+2, so the two page
      // registers swap roles from one tile to the next.
      // (last_tag: t = n is known to hold, false, or to be tested, a
      // std::integral_constant<int, 1, 0 or -1>)
      auto pp_load_end = [&](auto last_tag, int t, uint16_t *wn, int &pv) {
        constexpr int LAST = decltype(last_tag)::value;
        if (LAST == 1 || (LAST < 0 && t == n)) {
          if constexpr (FUSED) {
            if (wg_band(t * BN)) load_wslice(t * BN, wn);
          } else if (use_stage && wave_band(t * BN)) {
            stage_bias(t * BN);
          }
        }
        pv = tile_page(min(t + 2, n_t - 1) * BN);
      };
      auto pp_load = [&](auto last_tag, int t, uint16_t *kn, uint16_t *vc, uint16_t *wn, int &pv, int &pk) {
        pp_dma(t, kn, vc, pv, pk);
        pp_load_end(last_tag, t, wn, pv);
      };
      const std::integral_constant<int, 1> is_last{};
      const std::integral_constant<int, 0> not_last{};
      const std::integral_constant<int, -1> maybe_last{};
      // End of a phase: this wave's LDS reads, and at the end of odd phases
      // its direct loads, are done.  No fence: a release fence would also
      // wait for the loads left in flight across even phases; the empty asm
      // keeps the compiler from moving memory accesses across the barrier,
      // and the scheduling barriers keep each phase's arithmetic in it (the
      // scheduler would otherwise sink the exponentials into the next phase,
      // beside the same wave's MFMAs).
      auto pp_barrier = [&](auto loads_tag) {
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("" ::: "memory");
        if constexpr (decltype(loads_tag)::value) __builtin_amdgcn_s_waitcnt(waitcnt_vm0_lgkm0);
        else __builtin_amdgcn_s_waitcnt(waitcnt_lgkm0);
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
      };
      const std::true_type waits{};       // end of an odd phase: loads done too
      const std::false_type no_wait{};
      // M: MFMAs i0 .. i1-1 of the stream P V of the tile in vp (0 .. NPV-1:
      // block sub, k-step kh, slab ds), then S^T of the tile in kc (NPV ..
      // NM-1: k-step kb, block sub, the two blocks' chains interleaved), each
      // LDS operand read three MFMAs ahead.  The order of the MFMAs into each
      // accumulator is that of pv_block and s_block.
      constexpr int NPV = 2 * 2 * DSUB, NM = NPV + 2 * KB;
      auto pp_m = [&](const uint16_t *vp, const uint16_t *kc, int i0, int i1, auto hook) {
        auto rd = [&](int i) {
          if (i < NPV) {
            const int ks = 2 * (i / (2 * DSUB)) + (i / DSUB) % 2, ds = i % DSUB;
            const uint16_t *v0 = vp + vbase + ks * 16 * D + (((ds * 4) | vchunk_lo) ^ vsw) * 8;
            const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)(v0));
            const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)(v0 + 4 * D));
            const u32x2_t lw = __builtin_bit_cast(u32x2_t, lo);
            const u32x2_t hw = __builtin_bit_cast(u32x2_t, hi);
            return u32x4_t{lw[0], lw[1], hw[0], hw[1]};
          }
          const int sub = (i - NPV) & 1, kb = (i - NPV) >> 1;
          return *reinterpret_cast<const u32x4_t *>(kc + kbase + sub * 32 * D + (((2 * kb) ^ kx) * 8));
        };
        auto mf = [&](int i, const u32x4_t &op) {
          const bf16x8_t a = __builtin_bit_cast(bf16x8_t, op);
          if (i < NPV) {
            const int kh = (i / DSUB) % 2, ds = i % DSUB;
            const bf16x8_t pb = __builtin_bit_cast(bf16x8_t, (i / (2 * DSUB)) ? pp1[kh] : pp0[kh]);
            oacc[ds] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb, oacc[ds], 0, 0, 0);
          } else {
            const int kb = (i - NPV) >> 1;
            f32x16_t &acc = ((i - NPV) & 1) ? ps1 : ps0;
            if (kb == 0) {
#pragma unroll
              for (int e = 0; e < 16; ++e) acc[e] = 0.f;
            }
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(bf16x8_t, qf[kb]), acc, 0, 0, 0);
          }
        };
        constexpr int AHEAD = 3;
        u32x4_t ob[AHEAD + 1];
#pragma unroll
        for (int i = 0; i < AHEAD; ++i)
          if (i0 + i < i1) ob[(i0 + i) % (AHEAD + 1)] = rd(i0 + i);
#pragma unroll
        for (int i = 0; i < NM; ++i) {
          if (i >= i0 && i < i1) {
            if (i + AHEAD < i1) ob[(i + AHEAD) % (AHEAD + 1)] = rd(i + AHEAD);
            mf(i, ob[i % (AHEAD + 1)]);
            hook(i);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      };
      // V: the probabilities of the tile, hook(q) between its steps (the
      // scheduling barriers keep loads issued there spread through it)
      auto pp_v = [&](auto hook) {
        hook(0);
        __builtin_amdgcn_sched_barrier(0);
        rescale(fmaf(fmaxf(max16(ps0), max16(ps1)), scale2, sb0));
        float c2 = sb0 - m2;
        asm volatile("" : "+v"(c2));
        hook(1);
        __builtin_amdgcn_sched_barrier(0);
        probs(ps0, scale2, c2, pp0);
        {
          u32x4_t q0 = pp0[0], q1 = pp0[1];
          asm volatile("" : "+v"(q0), "+v"(q1));
          pp0[0] = q0, pp0[1] = q1;
        }
        hook(2);
        __builtin_amdgcn_sched_barrier(0);
        probs(ps1, scale2, c2, pp1);
        hook(3);
        // formed here, not after the wait that ends the phase (through
        // locals: the asm may not name the kernel's variables here)
        u32x4_t q0 = pp0[0], q1 = pp0[1], q2 = pp1[0], q3 = pp1[1];
        float ls = lsum;
        asm volatile("" : "+v"(q0), "+v"(q1), "+v"(q2), "+v"(q3), "+v"(ls));
        pp0[0] = q0, pp0[1] = q1, pp1[0] = q2, pp1[1] = q3, lsum = ls;
      };
      // Each group runs its own copy of the phase sequence, so that every wait
      // in it is known at compile time.
      auto pp_run = [&](auto lead_tag, int &pa, int &pb) {
        constexpr bool LEAD = decltype(lead_tag)::value;
        auto no_hook = [](int) {};
        // Tile j (0 < j < n): K(j) in kc, V(j-1) in vp; the loads of phase 2j
        // (lead: after the LDS reads of M(j)) and 2j+2 (others: before V(j))
        // go to kn/vc and kc/vp.  pa holds the page of tile j, pb that of
        // tile j+1.
        // (last_tag: whether j + 1 = n, for the other group's loads)
        auto pp_tile = [&](auto last_tag, int j, uint16_t *kc, uint16_t *kn, uint16_t *vc, uint16_t *vp,
                           int &pa, int &pb) {
          pp_m(vp, kc, 0, NM, no_hook);
          if constexpr (LEAD) {
            pp_load(not_last, j, kn, vc, nullptr, pa, pb);
            pp_barrier(no_wait);
            pp_v(no_hook);
            pp_barrier(waits);
          } else {
            pp_barrier(waits);
            pp_load(last_tag, j + 1, kc, vp, (j & 1) ? wsl0 : wsl1, pb, pa);
            pp_v(no_hook);
            pp_barrier(no_wait);
          }
        };
        // tile 0: no P V before its S^T; the other group starts one barrier later
        if constexpr (!LEAD) {
          pp_load(not_last, 0, k_lds1, v_lds0, nullptr, pa, pb);
          pp_barrier(no_wait);
        }
        pp_m(nullptr, k_lds0, NPV, NM, no_hook);
        if constexpr (LEAD) {
          pp_load(not_last, 0, k_lds1, v_lds0, nullptr, pa, pb);
          pp_barrier(no_wait);
        } else {
          pp_barrier(waits);
          pp_load(maybe_last, 1, k_lds0, v_lds1, wsl1, pb, pa);
        }
        pp_v(no_hook);
        if constexpr (LEAD) pp_barrier(waits);
        else pp_barrier(no_wait);
        int j = 1;
        for (; j + 2 <= n; j += 2) {
          pp_tile(maybe_last, j, k_lds1, k_lds0, v_lds1, v_lds0, pb, pa);
          pp_tile(maybe_last, j + 1, k_lds0, k_lds1, v_lds0, v_lds1, pa, pb);
        }
        if (j < n) pp_tile(maybe_last, j, k_lds1, k_lds0, v_lds1, v_lds0, pb, pa);
        // j = n: P V of tile n-1, with the lead's loads of phase 2n (the other
        // group skips its last barrier: its phases end one barrier later)
        pp_m((n & 1) ? v_lds0 : v_lds1, nullptr, 0, NPV, no_hook);
        if constexpr (LEAD) {
          pp_load(is_last, n, (n & 1) ? k_lds0 : k_lds1, (n & 1) ? v_lds1 : v_lds0, (n & 1) ? wsl1 : wsl0,
                  (n & 1) ? pb : pa, (n & 1) ? pa : pb);
          pp_barrier(no_wait);
        }
        pp_barrier(waits);
      };
      int pa = 0, pb = page_nxt;
      if (lead) pp_run(std::true_type{}, pa, pb);
      else pp_run(std::false_type{}, pa, pb);
      // page of tile n+1 for the general loop
      int &pg_n1 = (n & 1) ? pa : pb;
      page_nxt = pg_n1;
      // the general loop goes on from tile n_fixed, in buffer n_fixed % 2
      clear_bias_r();
      s_cur = n_fixed * BN;
      s_nxt = tile_after(s_cur);
      s_nxt2 = tile_after(s_nxt);
      steps_left = n_t - n_fixed;
      if (n_fixed & 1) go = step(AnyTile{}, k_lds1, v_lds1, k_lds0, v_lds0, wsl1, wsl0, page_nxt);
    } else {
      clear_bias_r();
    }
  } else {
    int i_fixed = 0;
    for (; i_fixed + 2 <= n_fixed; i_fixed += 2) {
      step(FixedTile{}, k_lds0, v_lds0, k_lds1, v_lds1, wsl0, wsl1, page_nxt);
      step(FixedTile{}, k_lds1, v_lds1, k_lds0, v_lds0, wsl1, wsl0, page_nxt);
    }
    if (i_fixed < n_fixed) {   // an odd count: the general loop starts on buffer 1
      step(FixedTile{}, k_lds0, v_lds0, k_lds1, v_lds1, wsl0, wsl1, page_nxt);
      go = step(AnyTile{}, k_lds1, v_lds1, k_lds0, v_lds0, wsl1, wsl0, page_nxt);
    }
  }
  while (go) {
    if (!step(AnyTile{}, k_lds0, v_lds0, k_lds1, v_lds1, wsl0, wsl1, page_nxt)) break;
    if (!step(AnyTile{}, k_lds1, v_lds1, k_lds0, v_lds0, wsl1, wsl0, page_nxt)) break;
  }

  // ---- epilogue ------------------------------------------------------------
  const float ltot = lsum + __shfl_xor(lsum, 32);
  if (row_ok) {
    const float inv = 1.0f / ltot;
    uint16_t *op = static_cast<uint16_t *>(a.out) + row * D;
#pragma unroll
    for (int ds = 0; ds < DSUB; ++ds)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = ds * 32 + 8 * g + 4 * half;
        u32x2_t w;
        w[0] = pack_bf16x2(oacc[ds][4 * g + 0] * inv, oacc[ds][4 * g + 1] * inv);
        w[1] = pack_bf16x2(oacc[ds][4 * g + 2] * inv, oacc[ds][4 * g + 3] * inv);
        *reinterpret_cast<u32x2_t *>(op + d0) = w;
      }
    if (a.lse != nullptr && half == 0) a.lse[row] = (m2 + __log2f(ltot)) * LN2;
  }
}

}  // namespace

template <int D, int NW>
static void launch_d(const PrefillArgs &a, hipStream_t s) {
  dim3 grid(a.num_blocks), block(64 * NW);
  const bool big = a.page_size >= BN;
  const bool vec = a.R >= 8;
  if (big && vec) hipLaunchKernelGGL((prefill_bf16_kernel<D, NW, true, true, 0>), grid, block, 0, s, a);
  else if (big) hipLaunchKernelGGL((prefill_bf16_kernel<D, NW, true, false, 0>), grid, block, 0, s, a);
  else if (vec) hipLaunchKernelGGL((prefill_bf16_kernel<D, NW, false, true, 0>), grid, block, 0, s, a);
  else hipLaunchKernelGGL((prefill_bf16_kernel<D, NW, false, false, 0>), grid, block, 0, s, a);
}

template <int D, int NW, int DR>
static void launch_fused_d(const PrefillArgs &a, hipStream_t s) {
  dim3 grid(a.num_blocks), block(64 * NW);
  if (a.page_size >= BN) hipLaunchKernelGGL((prefill_bf16_kernel<D, NW, true, true, DR>), grid, block, 0, s, a);
  else hipLaunchKernelGGL((prefill_bf16_kernel<D, NW, false, true, DR>), grid, block, 0, s, a);
}

template <int NW>
static hipError_t launch_fused_nw(const PrefillArgs &a, int head_dim, hipStream_t s) {
  if (head_dim == 128) {
    if (a.d_rel == 32) launch_fused_d<128, NW, 32>(a, s);
    else launch_fused_d<128, NW, 16>(a, s);
  } else if (head_dim == 64) {
    if (a.d_rel == 32) launch_fused_d<64, NW, 32>(a, s);
    else launch_fused_d<64, NW, 16>(a, s);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_prefill_bf16(const PrefillArgs &a, int head_dim, hipStream_t s) {
  if (a.waves != 4 && a.waves != 8) return hipErrorInvalidValue;
  if (head_dim == 128) {
    if (a.waves == 8) launch_d<128, 8>(a, s);
    else launch_d<128, 4>(a, s);
  } else if (head_dim == 64) {
    if (a.waves == 8) launch_d<64, 8>(a, s);
    else launch_d<64, 4>(a, s);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_prefill_fused(const PrefillArgs &a, int head_dim, hipStream_t s) {
  if (a.d_rel != 16 && a.d_rel != 32) return hipErrorInvalidValue;
  // 4-wave work-groups hold W^T rows for at most 64 queries: two heads or more
  if (a.waves == 4 && a.hpw >= 2) return launch_fused_nw<4>(a, head_dim, s);
  if (a.waves == 8) return launch_fused_nw<8>(a, head_dim, s);
  return hipErrorInvalidValue;
}

}  // namespace rba
