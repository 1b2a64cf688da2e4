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
// Work decomposition (one work-group = 4 waves = 128 queries of one head):
//  * 64-key K and V tiles are staged HBM -> registers (one tile ahead) ->
//    LDS, both row-major with XOR-swizzled 16-byte chunks;
//  * S^T = K Q^T and O^T += V^T P^T run on v_mfma_f32_32x32x16_bf16, so each
//    lane owns one query column: the softmax row statistics stay in a lane
//    pair (lane, lane^32);
//  * the V^T operand comes straight from the row-major V tile through the
//    transposing LDS read ds_read_b64_tr_b16;
//  * the bias of query row t at distance d sits in a per-row ring of two
//    64-wide distance chunks in LDS, with the odd chunk mirrored in front of
//    the even one so any four consecutive distances are contiguous; each key
//    tile brings in one new chunk per row, loaded with aligned 16-byte reads,
//    so every bias element crosses HBM once.  Tiles whose distances all lie
//    at or beyond R-1 use the single clamped value bias[t,h,R-1];
//  * three score paths chosen per wave and tile: clamp-only unmasked (scale,
//    bias and max folded into one FMA before exp2), band unmasked, and a
//    general path for window/causal/sequence-end edges and the clamp border;
//  * masking selects (never multiplies), so NaN in keys past the end of a
//    sequence or in masked positions cannot leak into the output;
//  * the running max is rescaled lazily (only when a row's max grows by more
//    than 2^8), which is exact because numerator and denominator share it.
#include "rba_internal.h"

#include <type_traits>

namespace rba {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

constexpr int BM = 128;        // queries per work-group
constexpr int BN = 64;         // keys per tile (= one bias chunk)
constexpr int NTHREADS = 256;
constexpr int RROW = 3 * BN;   // bias ring row: [odd-slot mirror | even slot | odd slot]
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;
constexpr float NEG_INIT = -1.0e30f;  // finite start of the running max (log2 units)
constexpr float TAU = 8.0f;           // lazy-rescale threshold (log2 units)

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
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
// transposing read touches 4 consecutive rows x 2..4 consecutive chunks, which
// the per-row pattern below spreads over distinct banks.
template <int D>
__device__ __forceinline__ int v_swizzle(int row) {
  if constexpr (D == 128) {
    constexpr int tab = (0) | (6 << 4) | (12 << 8) | (10 << 12);
    return (tab >> ((row & 3) * 4)) & 15;
  } else {
    return 2 * (row & 3);
  }
}

template <int D>
struct __align__(16) PrefillSmem {
  uint16_t k[BN * D];           // K tile [key][D]
  uint16_t v[BN * D];           // V tile [key][D]
  uint16_t ring[BM * RROW];     // bias ring, one row per query
};

template <int D, bool BIG_PAGE, bool VEC_BIAS>
__global__ __launch_bounds__(NTHREADS, 2) void prefill_bf16_kernel(PrefillArgs a) {
  constexpr int CHUNKS = D / 8;                 // 16-byte chunks per key row
  constexpr int KPT = BN * CHUNKS / NTHREADS;   // key rows per thread per tile
  constexpr int KB = D / 16;                    // MFMA k-steps over head_dim
  constexpr int DSUB = D / 32;                  // 32-row slabs of O^T
  __shared__ PrefillSmem<D> sm;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform per wave

  // Work-group -> (sequence, head, query tile).  Blocks are dealt to the 8
  // XCDs round-robin; remap so each XCD walks a contiguous range, in which
  // the query heads of one KV head and its query tiles (heaviest first)
  // are adjacent and share that XCD's L2.
  const int nb = a.num_blocks;
  const int bid = blockIdx.x;
  const int xcd = bid & 7, xidx = bid >> 3;
  const int base = nb >> 3, rem = nb & 7;
  const int r = (xcd < rem) ? xcd * (base + 1) + xidx
                            : rem * (base + 1) + (xcd - rem) * base + xidx;
  const int nqt = a.num_qtiles;
  const int per_seq = a.Hq * nqt;
  const int b = r / per_seq;
  int rr = r - b * per_seq;
  const int per_kvh = a.G * nqt;
  const int kvh = rr / per_kvh;
  rr -= kvh * per_kvh;
  const int qt = nqt - 1 - rr / a.G;
  const int h = kvh * a.G + rr % a.G;

  const int tok0 = a.cu_seqlens[b];
  const int L = a.cu_seqlens[b + 1] - tok0;
  const int t0 = qt * BM;
  if (t0 >= L) return;

  const int Hq = a.Hq;
  const int R = a.R;
  const int W = a.window;
  const int t_last = min(t0 + BM, L) - 1;
  int s_begin = (W > 0) ? max(0, t0 - W + 1) : 0;
  s_begin &= ~(BN - 1);

  const uint16_t *qp = static_cast<const uint16_t *>(a.q);
  const uint16_t *kp = static_cast<const uint16_t *>(a.k_pool);
  const uint16_t *vp = static_cast<const uint16_t *>(a.v_pool);
  const int32_t *trow = a.block_table + (size_t)b * a.max_pages;
  const int P = a.page_size;
  const int lp = a.log2_page;
  const size_t head_stride = (size_t)P * D;           // elements per (page, head)
  const size_t page_stride = (size_t)a.Hkv * head_stride;
  // bias rows of this work-group start here; row q adds q * Hq * R
  const uint16_t *bwg = static_cast<const uint16_t *>(a.bias) +
                        ((size_t)(tok0 + t0) * Hq + h) * R;
  const uint32_t brow_stride = (uint32_t)Hq * (uint32_t)R;

  // ---- this lane's query row --------------------------------------------
  const int col = lane & 31;
  const int half = lane >> 5;
  const int q_local = wave * 32 + col;
  const int t = t0 + q_local;
  const bool row_ok = t < L;
  const size_t row = ((size_t)tok0 + (row_ok ? t : 0)) * Hq + h;

  u32x4_t qf[KB];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    const u32x4_t v = *reinterpret_cast<const u32x4_t *>(qp + row * D + kb * 16 + half * 8);
    qf[kb] = row_ok ? v : u32x4_t{0, 0, 0, 0};
  }
  const float b_last = bf16_to_f32(bwg[(row_ok ? (uint32_t)q_local : 0u) * brow_stride + (R - 1)]);

  // ---- K/V tile loaders (every load unconditional; rows past the end of
  // the sequence are read from inside the same page, then zeroed) ----------
  const int kc = tid % CHUNKS;          // 16-byte chunk this thread moves
  const int krow0 = tid / CHUNKS;       // K and V rows krow0 + j*(NTHREADS/CHUNKS)

  u32x4_t kreg[KPT], vreg[KPT];
  const u32x4_t zero4 = {0, 0, 0, 0};

  auto load_kv = [&](int s0) {
    if constexpr (BIG_PAGE) {
      const int page = trow[s0 >> lp];
      const uint16_t *kt = kp + (size_t)page * page_stride + (size_t)kvh * head_stride +
                           (size_t)(s0 & (P - 1)) * D;
      const uint16_t *vt = vp + (kt - kp);
#pragma unroll
      for (int j = 0; j < KPT; ++j) {
        const int kr = krow0 + j * (NTHREADS / CHUNKS);
        kreg[j] = *reinterpret_cast<const u32x4_t *>(kt + (uint32_t)(kr * D + kc * 8));
        vreg[j] = *reinterpret_cast<const u32x4_t *>(vt + (uint32_t)(kr * D + kc * 8));
      }
    } else {
#pragma unroll
      for (int j = 0; j < KPT; ++j) {
        const int kr = krow0 + j * (NTHREADS / CHUNKS);
        const int sk = min(s0 + kr, L - 1);
        const size_t ko = (size_t)trow[sk >> lp] * page_stride + (size_t)kvh * head_stride +
                          (size_t)(sk & (P - 1)) * D + kc * 8;
        kreg[j] = *reinterpret_cast<const u32x4_t *>(kp + ko);
        vreg[j] = *reinterpret_cast<const u32x4_t *>(vp + ko);
      }
    }
  };

  // Rows at or past the end of the sequence are zeroed here, at the LDS
  // write, so the loads themselves stay unconditional and in flight.
  auto commit_kv = [&](int s0) {
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const int kr = krow0 + j * (NTHREADS / CHUNKS);
      const bool ok = s0 + kr < L;
      *reinterpret_cast<u32x4_t *>(&sm.k[kr * D + ((kc ^ (kr & (CHUNKS - 1))) * 8)]) = ok ? kreg[j] : zero4;
      *reinterpret_cast<u32x4_t *>(&sm.v[kr * D + ((kc ^ v_swizzle<D>(kr)) * 8)]) = ok ? vreg[j] : zero4;
    }
  };

  // ---- bias ring loader: one 64-wide distance chunk per query row ----------
  // For key tile s0, row q needs distances t0+q-s0-63 .. t0+q-s0, i.e. the
  // chunks lo(q) = floor((t0-s0-63+q)/64) and lo(q)+1.  Moving to the next
  // tile (s0 += 64) needs chunk lo-1 and drops lo+1: same ring slot.  The
  // ring row is [odd slot mirror | even slot | odd slot]: distance d lives at
  // 64 + (d mod 128), and also at d mod 128 - 64 when its chunk is odd.
  // Thread tid moves 16-byte piece (tid & 7) of rows tid/8 + 32*j.
  u32x4_t breg[4];
  const int bq0 = tid >> 3;
  const int bv8 = (tid & 7) * 8;

  auto chunk_elem = [&](int s0, int q, int which) {
    return (((t0 - s0 - (BN - 1) + q) >> 6) + which) * BN + bv8;
  };

  auto load_chunk = [&](int s0, int which) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int q = bq0 + 32 * j;
      const int e = chunk_elem(s0, q, which);
      const bool ok = (t0 + q < L) && e >= 0 && e < R;
      if constexpr (VEC_BIAS) {
        const uint32_t off = ok ? (uint32_t)q * brow_stride + (uint32_t)e : 0u;
        breg[j] = *reinterpret_cast<const u32x4_t *>(bwg + off);
      } else {
        u32x4_t v = zero4;
#pragma unroll
        for (int x = 0; x < 8; ++x) {
          const bool okx = ok && (e + x < R);
          const uint32_t off = okx ? (uint32_t)q * brow_stride + (uint32_t)(e + x) : 0u;
          const uint32_t el = bwg[off];
          v[x >> 1] |= (okx ? el : 0u) << ((x & 1) * 16);
        }
        breg[j] = v;
      }
    }
  };

  auto commit_chunk = [&](int s0, int which) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int q = bq0 + 32 * j;
      const int e = chunk_elem(s0, q, which);
      const bool ok = (t0 + q < L) && e >= 0 && e < R;
      const u32x4_t v = ok ? breg[j] : zero4;
      const int pos = BN + (e & (2 * BN - 1));
      *reinterpret_cast<u32x4_t *>(&sm.ring[q * RROW + pos]) = v;
      if (e & BN) *reinterpret_cast<u32x4_t *>(&sm.ring[q * RROW + pos - 2 * BN]) = v;
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
  // K operand: lane reads key row col (+32 for the second key block), chunk
  // (2kb + half) ^ (col mod CHUNKS) = (2kb) ^ kx.
  const int kx = half ^ (col & (CHUNKS - 1));
  const uint16_t *kbase = &sm.k[col * D];
  // V operand via the transposing read: this lane supplies the address of
  // key ks*16 + 4*(g/2) + kk (+8 for k-slots 4..7), head-dim elements
  // ds*32 + 16*(g%2) + 4*i .. +3, where g = lane/16, kk = (lane/4)%4, i = lane%4.
  // The read hands lane 16g+4i+j element j of lanes 16g+i+4kk, kk = 0..3, which
  // is row d = ds*32 + lane%32 of V^T at keys ks*16 + 4*half + 0..3 (+8).
  const int vg = lane >> 4, vkk = (lane >> 2) & 3, vi = lane & 3;
  const int vrow = 4 * (vg >> 1) + vkk;
  const int vchunk_lo = 2 * (vg & 1) + (vi >> 1);        // chunk within a 32-wide slab
  const int vsw = v_swizzle<D>(vrow);                   // rows ks*16+vrow(+8) share it
  const uint16_t *vbase = &sm.v[vrow * D + (vi & 1) * 4];
  const uint16_t *ringrow = &sm.ring[q_local * RROW + BN];   // distance d at [d mod 128]

  auto compute_tile = [&](int s0) {
    const int tq0 = t0 + wave * 32;
    const int dmax_w = tq0 + 31 - s0;
    const int dmin_w = tq0 - (s0 + BN - 1);
    if (dmax_w < 0) return;                    // every key lies in this wave's future
    if (W > 0 && dmin_w >= W) return;          // every key lies before the window
    const bool need_mask = (dmin_w < 0) || (W > 0 && dmax_w >= W) || (s0 + BN > L);
    const bool band = dmin_w < R - 1;
    // some visible distance beyond R-1 inside a band tile (global layers only)
    const bool straddle = band && dmax_w > R - 1 && (W <= 0 || W > R);
    // score path: 0 clamp-only unmasked, 1 band unmasked, 2 general
    const int path = (!need_mask && !band) ? 0 : ((!need_mask && !straddle) ? 1 : 2);
    // exp2 argument = fma(v, sa, sb - m2): v is the raw q.k on path 0 (scale
    // and the clamped bias folded into sa, sb), the finished score otherwise
    const float sa = (path == 0) ? scale2 : LOG2E;
    const float sb = (path == 0) ? b_last * LOG2E : 0.f;

    // The tile is processed as two 32-key halves (sub = 0, 1): S^T = K Q^T on
    // one 32x32 block, its softmax update, then O^T += V^T P^T for its keys.
    const int dq = t - s0 - 4 * half;          // distance of key s0 + 4*half
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      f32x16_t sacc;
#pragma unroll
      for (int j = 0; j < 16; ++j) sacc[j] = 0.f;
      const uint16_t *kb0 = kbase + sub * 32 * D;
      u32x4_t kf[2];
      kf[0] = *reinterpret_cast<const u32x4_t *>(kb0 + (kx * 8));
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        if (kb + 1 < KB)
          kf[(kb + 1) & 1] = *reinterpret_cast<const u32x4_t *>(kb0 + (((2 * (kb + 1)) ^ kx) * 8));
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, kf[kb & 1]),
                                                       __builtin_bit_cast(bf16x8_t, qf[kb]), sacc, 0, 0, 0);
      }

      // Element j is key s0 + 4*half + koff, koff = 32*sub + 8*(j>>2) + (j&3),
      // at distance dq - koff.  Four consecutive j share one ring base.
      auto ring_group = [&](int g) {           // address of distance (dq - koff0 - 3)
        const int d0 = dq - (32 * sub + 8 * g);
        return ringrow + ((d0 & (2 * BN - 1)) - 3);
      };
      if (path == 1) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const uint16_t *rg = ring_group(g);
#pragma unroll
          for (int i = 0; i < 4; ++i)
            sacc[4 * g + i] = fmaf(sacc[4 * g + i], scale, bf16_to_f32(rg[3 - i]));
        }
      } else if (path == 2) {
        const int kv_hi = min(dq, L - 1 - s0 - 4 * half);   // visible iff kv_lo < koff <= kv_hi
        const int kv_lo = (W > 0) ? dq - W : -1000000;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const uint16_t *rg = ring_group(g);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int koff = 32 * sub + 8 * g + i;
            const float bv = (band && dq - koff < R - 1) ? bf16_to_f32(rg[3 - i]) : b_last;
            const float x = fmaf(sacc[4 * g + i], scale, bv);
            sacc[4 * g + i] = (koff > kv_lo && koff <= kv_hi) ? x : -INFINITY;
          }
        }
      }
      {
        float m4[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          m4[i] = fmaxf(fmaxf(sacc[4 * i + 0], sacc[4 * i + 1]), fmaxf(sacc[4 * i + 2], sacc[4 * i + 3]));
        float mx = fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3]));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mt2 = fmaf(mx, sa, sb);
        const bool exceed = mt2 > m2 + TAU;
        if (__ballot(exceed)) {
          const float mnew = exceed ? mt2 : m2;
          const float alpha = __builtin_amdgcn_exp2f(m2 - mnew);
          lsum *= alpha;
#pragma unroll
          for (int i = 0; i < DSUB; ++i)
#pragma unroll
            for (int j = 0; j < 16; ++j) oacc[i][j] *= alpha;
          m2 = mnew;
        }
        const float c2 = sb - m2;
        float ps[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const float p = __builtin_amdgcn_exp2f(fmaf(sacc[j], sa, c2));
          ps[j & 3] += p;
          sacc[j] = p;
        }
        lsum += (ps[0] + ps[1]) + (ps[2] + ps[3]);
      }

      // O^T += V^T P^T, 16 keys per MFMA.  k-slots of lane half `half` are keys
      // ks*16 + 4*half + {0,1,2,3,8,9,10,11}: exactly S^T registers 8*(ks&1)+0..7,
      // and exactly the keys the two transposing reads deliver.
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {
        const int ks = 2 * sub + kh, rb = kh * 8;
        u32x4_t pw;
#pragma unroll
        for (int j = 0; j < 4; ++j) pw[j] = pack_bf16x2(sacc[rb + 2 * j], sacc[rb + 2 * j + 1]);
        const bf16x8_t pb = __builtin_bit_cast(bf16x8_t, pw);
#pragma unroll
        for (int ds = 0; ds < DSUB; ++ds) {
          const uint16_t *v0 = vbase + ks * 16 * D + (((ds * 4) | vchunk_lo) ^ vsw) * 8;
          const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)(v0));
          const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)(v0 + 8 * D));
          const u32x2_t lw = __builtin_bit_cast(u32x2_t, lo);
          const u32x2_t hw = __builtin_bit_cast(u32x2_t, hi);
          const bf16x8_t vb = __builtin_bit_cast(bf16x8_t, u32x4_t{lw[0], lw[1], hw[0], hw[1]});
          oacc[ds] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vb, pb, oacc[ds], 0, 0, 0);
        }
      }
    }
  };

  // ---- main loop: prefetch tile i+1 while computing tile i -----------------
  auto wg_band = [&](int s0) { return t0 - (s0 + BN - 1) < R - 1; };

  load_kv(s_begin);
  bool ring_ready = false;
  const bool band0 = wg_band(s_begin);
  if (band0) load_chunk(s_begin, 0);
  commit_kv(s_begin);
  if (band0) {
    commit_chunk(s_begin, 0);
    load_chunk(s_begin, 1);
    commit_chunk(s_begin, 1);
    ring_ready = true;
  }
  __syncthreads();

  for (int s0 = s_begin; s0 <= t_last; s0 += BN) {
    const int sn = s0 + BN;
    const bool has_next = sn <= t_last;
    const bool band_next = has_next && wg_band(sn);
    if (has_next) {
      load_kv(sn);
      if (band_next) load_chunk(sn, 0);
    }
    compute_tile(s0);
    __syncthreads();
    if (has_next) {
      commit_kv(sn);
      if (band_next) {
        commit_chunk(sn, 0);
        if (!ring_ready) {
          load_chunk(sn, 1);
          commit_chunk(sn, 1);
          ring_ready = true;
        }
      }
    }
    __syncthreads();
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

template <int D>
static void launch_d(const PrefillArgs &a, hipStream_t s) {
  dim3 grid(a.num_blocks), block(NTHREADS);
  const bool big = a.page_size >= BN;
  const bool vec = (a.R & 7) == 0;
  if (big && vec) hipLaunchKernelGGL((prefill_bf16_kernel<D, true, true>), grid, block, 0, s, a);
  else if (big) hipLaunchKernelGGL((prefill_bf16_kernel<D, true, false>), grid, block, 0, s, a);
  else if (vec) hipLaunchKernelGGL((prefill_bf16_kernel<D, false, true>), grid, block, 0, s, a);
  else hipLaunchKernelGGL((prefill_bf16_kernel<D, false, false>), grid, block, 0, s, a);
}

hipError_t launch_prefill_bf16(const PrefillArgs &a, int head_dim, hipStream_t s) {
  if (head_dim == 128) {
    launch_d<128>(a, s);
  } else if (head_dim == 64) {
    launch_d<64>(a, s);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace rba
