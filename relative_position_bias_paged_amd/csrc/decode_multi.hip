// decode_multi.hip -- decode of a few new tokens per sequence (q_len 2..16)
// over a long paged cache, bf16 in / fp32 accumulate, for gfx950 (CDNA4).
//
// Sequence b holds n_b keys, the keys of its q_len new tokens included; new
// token i sits at position p_i = n_b - q_len + i and attends keys
// s <= p_i (and p_i - s < window on local layers) with score
// sm_scale * q.k + bias[b*q_len + i, h, min(p_i - s, R-1)], as a prefill of
// those tokens over the cached history would (TensorRT-LLM PR #17062
// "Support Inkling-NVFP4 model", Description, Architecture list: the bias is
// per query token, head and distance).  This is the pass that verifies the
// drafts of a multi-token-prediction step together (the vLLM PR #48768 "Add
// Inkling multi-depth MTP support [5/N]" page: the target model checks the
// drafted tokens of every depth in one forward pass): a handful of queries
// per sequence against its whole cache, so the work is a decode's, bound by
// the K/V bytes, not a prefill's.
//
// One wave owns (sequence, KV head, group of hpw query heads, one
// page-aligned partition of the keys any of the sequence's queries sees),
// and its 16 matrix rows are the (head, token) pairs of its heads:
//  * keys come in 16-key tiles, the next tile's K, V and bias in flight in
//    registers while one is computed (the loads of decode_bf16_kernel), at
//    three waves per SIMD;
//  * S^T = K Q^T on v_mfma_f32_16x16x32_bf16: K straight from the loaded
//    registers is the A operand (row = key), so each lane ends up with four
//    keys' scores of one (head, token) row, and the softmax row statistics
//    live in the four lanes c16, c16+16, c16+32, c16+48;
//  * the probabilities, rounded to bf16, are in the B-operand layout of
//    O^T += V^T P^T on v_mfma_f32_16x16x16_bf16 as they stand; V^T comes
//    from a per-wave LDS copy of the V tile through the transposing read
//    ds_read_b64_tr_b16;
//  * a 16-key tile lies inside one page, so its loads stay in the page the
//    table names; V rows of keys outside the partition are zeroed in the
//    registers before the PV product and masking selects, so slots no query
//    sees (past the sequence end, before the window) cannot reach the
//    output whatever they hold.
// Partitions write normalised fp32 partials and their LSE; merge_kernel
// (decode_bf16.hip) combines them, and plan_kernel hands the partitions out
// largest first, as for single-token decode.
#include "rba_internal.h"

namespace rba {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;
constexpr float NEG_INIT = -1.0e30f;   // finite start of the running max (log2 units)
constexpr float TAU = 8.0f;            // lazy-rescale threshold (log2 units)
// Tiles in flight per wave, and the waves per SIMD the register budget is
// set for: 2 tiles at 3 waves (168 VGPRs, no spills).  4 tiles at 2 waves
// (246 VGPRs) and 3 at 2 measured the same or up to 1% slower.
#ifndef RBA_MQ_NBUF
#define RBA_MQ_NBUF 2
#endif
#ifndef RBA_MQ_WAVES
#define RBA_MQ_WAVES 3
#endif
constexpr int NBUF = RBA_MQ_NBUF;

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2_t v = __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t);
  return __builtin_bit_cast(uint32_t, v);
}

// Physical 8-byte unit of unit u (four head-dim elements) in LDS row r of
// the V tile.  A transposing read serves 32 lanes at once: 8 rows (keys 4g+k)
// times 4 consecutive units of one 16-element slab.  XOR-ing the unit with
// 4 x (the row's place among the rows that share the 64 banks) puts those
// 32 units on distinct banks.
template <int D>
__device__ __forceinline__ int v_unit(int u, int r) {
  if constexpr (D == 128) return u ^ (4 * (r & 7));      // 256-byte rows
  else return u ^ (4 * ((r >> 1) & 3));                    // 128-byte rows, two per 256 bytes
}

template <int D>
struct MqTile {
  u32x4_t k[D / 32];       // K[key c16][32*kk + 8*g4 .. +8]
  u32x4_t v[D / 32 == 4 ? 4 : 2];   // D=128: V[4*g4 + i][8*c16 ..+8]; D=64: two rows per register
  uint32_t bias[4];        // raw bf16 bias of (row c16, key 4*g4 + r)
};

template <int D>
__global__ __launch_bounds__(64, RBA_MQ_WAVES) void decode_multi_kernel(DecodeArgs a) {
  constexpr int KK = D / 32;        // MFMAs of S^T over head_dim
  constexpr int DB = D / 16;        // 16-wide head-dim blocks of O^T
  const int lane = threadIdx.x;
  const int c16 = lane & 15;
  const int g4 = lane >> 4;
  __shared__ __align__(16) uint16_t v_lds[2][16 * D];

  // Block -> (partition, sequence, KV head, head group) as in decode_bf16_kernel.
  const int S = a.num_splits;
  const int HG = a.head_groups;
  int item = blockIdx.x;
  const int hg = item % HG;
  item /= HG;
  const int kvh = item % a.Hkv;
  item /= a.Hkv;
  int b, split, n;
  if (a.plan != nullptr) {
    const int2 rec = a.plan[item];
    if (rec.x < 0) return;               // a partition with no key
    b = rec.x / S;
    split = rec.x - b * S;
    n = rec.y;                           // max(seq_lens[b], q_len)
  } else {
    b = item % a.num_seqs;
    split = item / a.num_seqs;
    n = max(a.seq_lens[b], a.q_len);
  }

  const int L = a.q_len;
  const int G = a.G;
  const int hpw = a.hpw;
  const int h_base = kvh * G + hg * hpw;
  const int nh = min(hpw, G - hg * hpw);
  const int Hq = a.Hq, R = a.R, W = a.window, P = a.page_size, lp = a.log2_page;

  // keys any query of the sequence sees, and this partition's share
  const int lo_u = (W > 0) ? max(0, n - L - W + 1) : 0;
  const int p_first = lo_u >> lp;
  const int p_end = (n + P - 1) >> lp;
  const int pg_lo = p_first + split * a.chunk_pages;
  const int pg_hi = min(p_first + (split + 1) * a.chunk_pages, p_end);
  if (pg_lo >= pg_hi) return;            // the merge reads only partitions with keys
  const int part_lo = max(pg_lo << lp, lo_u);       // first key (inclusive)
  const int part_hi = min(pg_hi << lp, n);          // last key + 1
  const int k_lo = part_lo & ~15;
  const int ntiles = (part_hi - k_lo + 15) >> 4;

  // this lane's row: head slot hh, token i (rows past nh * L repeat a valid
  // row and write nothing)
  const int rv = c16 < nh * L;
  const int hh = min(c16 / L, nh - 1);
  const int ti = c16 % L;
  const int h = h_base + hh;
  const int pos = n - L + ti;            // query position
  const size_t qrow = ((size_t)b * L + ti) * Hq + h;
  const int row_lo = max(part_lo, (W > 0) ? pos - W + 1 : 0);   // visible keys of the row
  const int row_hi = min(part_hi - 1, pos);                     // in this partition
  // tile-level bounds over all rows: interior tiles need no mask
  const int all_lo = max(part_lo, (W > 0) ? n - W : 0);         // the largest row_lo
  const int all_hi = min(part_hi - 1, n - L);                   // the smallest row_hi

  const uint16_t *qp = static_cast<const uint16_t *>(a.q);
  const uint16_t *kp = static_cast<const uint16_t *>(a.k_pool);
  const long long v_minus_k = static_cast<const char *>(a.v_pool) - static_cast<const char *>(a.k_pool);
  const uint16_t *brow = static_cast<const uint16_t *>(a.bias) + qrow * R;
  const int32_t *trow = a.block_table + (size_t)b * a.max_pages;
  const size_t head_stride = (size_t)P * D;
  const size_t page_stride = (size_t)a.Hkv * head_stride;

  // Q^T as the B operand of S^T: lane (c16, g4) holds row c16's head-dim
  // elements 32*kk + 8*g4 .. +8
  u32x4_t qb[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk)
    qb[kk] = *reinterpret_cast<const u32x4_t *>(qp + qrow * D + 32 * kk + 8 * g4);
  const float b_last = bf16_to_f32(brow[R - 1]);

  MqTile<D> buf[NBUF];
  // Tile ti (clamped to the last one) of this partition.  A 16-key tile
  // never straddles a page (P >= 16), so all its rows are slots of the page
  // the table names for it.  V goes out with the streaming cache policy
  // (read once), K with the default one, as in decode_bf16_kernel.
  auto issue = [&](int t, MqTile<D> &tb) {
    const int ts = k_lo + min(t, ntiles - 1) * 16;
    const int page = trow[ts >> lp];
    const uint16_t *tile = kp + (size_t)page * page_stride + (size_t)kvh * head_stride +
                           (size_t)(ts & (P - 1)) * D;
    const uint16_t *kt = tile + c16 * D + 8 * g4;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) tb.k[kk] = *reinterpret_cast<const u32x4_t *>(kt + 32 * kk);
    const uint16_t *vt = reinterpret_cast<const uint16_t *>(
        reinterpret_cast<const char *>(tile) + v_minus_k) + 4 * g4 * D;
    if constexpr (D == 128) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        tb.v[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(vt + i * D + 8 * c16));
    } else {
      // 128-byte rows: lane c16 reads 8 bytes of rows 4*g4 + i
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const u32x2_t w = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t *>(vt + i * D + 4 * c16));
        tb.v[i >> 1][2 * (i & 1)] = w[0];
        tb.v[i >> 1][2 * (i & 1) + 1] = w[1];
      }
    }
    // bias of this lane's row at its four keys (clamped in-row indices;
    // tiles wholly at distance >= R-1 read bucket R-1 and use b_last)
    const bool band = (n - L) - (ts + 15) < R - 1;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int d = band ? min(max(pos - (ts + 4 * g4 + r), 0), R - 1) : R - 1;
      tb.bias[r] = brow[d];
    }
  };

  f32x4_t acc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) acc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m2 = NEG_INIT;                   // running max of the row, log2 units
  float lsum = 0.f;                      // this lane's share of the row's denominator
  const float scale = a.sm_scale;

  // transposing-read address of this lane: row 4*g + k, unit 4*db + i, with
  // g = lane/16, k = (lane/4)%4, i = lane%4; it hands lane 16g + 4i' + j the
  // element V[4g + k][16*db + 4i' + j] in component k
  const int tr_row = 4 * g4 + ((lane >> 2) & 3);
  const int tr_i = lane & 3;

  auto process = [&](int t, const MqTile<D> &tb, uint16_t *vl) {
    const int ts = k_lo + t * 16;
    // V tile into LDS, row-major with the unit swizzle; on the partition's
    // edge tiles the rows of keys outside it are written as zeros (their
    // probabilities are 0 for every row, and the slots may hold anything)
    const bool edge = ts < part_lo || ts + 15 >= part_hi;
    if constexpr (D == 128) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * g4 + i;
        u32x4_t w = tb.v[i];
        if (edge && (ts + r < part_lo || ts + r >= part_hi)) w = u32x4_t{0, 0, 0, 0};
        *reinterpret_cast<u32x4_t *>(vl + r * D + v_unit<D>(2 * c16, r) * 4) = w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * g4 + i;
        u32x2_t w = {tb.v[i >> 1][2 * (i & 1)], tb.v[i >> 1][2 * (i & 1) + 1]};
        if (edge && (ts + r < part_lo || ts + r >= part_hi)) w = u32x2_t{0, 0};
        *reinterpret_cast<u32x2_t *>(vl + r * D + v_unit<D>(c16, r) * 4) = w;
      }
    }
    // S^T: lane holds keys ts + 4*g4 + r (r = 0..3) of row c16
    f32x4_t sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, tb.k[kk]),
                                                     __builtin_bit_cast(bf16x8_t, qb[kk]), sacc, 0, 0, 0);
    const bool band = (n - L) - (ts + 15) < R - 1;
    const bool need_mask = ts < all_lo || ts + 15 > all_hi;
    float x[4];
    float mloc = -INFINITY;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int s = ts + 4 * g4 + r;
      const float bv = (band && pos - s < R - 1) ? bf16_to_f32(tb.bias[r]) : b_last;
      float v = fmaf(sacc[r], scale, bv);
      if (need_mask) v = (s >= row_lo && s <= row_hi) ? v : -INFINITY;
      x[r] = v;
      mloc = fmaxf(mloc, v);
    }
    // lazy rescale: while no lane of the row sees a score above m2 + TAU the
    // row's m2 stands; otherwise the four lanes form the row maximum
    const float mt2 = mloc * LOG2E;
    if (__ballot(mt2 > m2 + TAU)) {
      float mr = fmaxf(mt2, __shfl_xor(mt2, 16));
      mr = fmaxf(mr, __shfl_xor(mr, 32));
      const float mnew = (mr > m2 + TAU) ? mr : m2;
      const float alpha = __builtin_amdgcn_exp2f(m2 - mnew);
      lsum *= alpha;
#pragma unroll
      for (int i = 0; i < DB; ++i) acc[i] *= alpha;
      m2 = mnew;
    }
    float p[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) p[r] = __builtin_amdgcn_exp2f(fmaf(x[r], LOG2E, -m2));
    const u32x2_t pw = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])};
    // the denominator adds exactly the rounded values the PV product uses
    lsum += (bf16_to_f32(pw[0] & 0xffffu) + __uint_as_float(pw[0] & 0xffff0000u)) +
            (bf16_to_f32(pw[1] & 0xffffu) + __uint_as_float(pw[1] & 0xffff0000u));
    const i16x4_t pb = __builtin_bit_cast(i16x4_t, pw);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const i16x4_t va = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_i16x4_t *)(vl + tr_row * D + v_unit<D>(4 * db + tr_i, tr_row) * 4));
      acc[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pb, acc[db], 0, 0, 0);
    }
  };

  // software pipeline: NBUF tiles in flight; two LDS copies of the V tile
#pragma unroll
  for (int j = 0; j < NBUF; ++j) issue(j, buf[j]);
  for (int i0 = 0; i0 < ntiles; i0 += NBUF) {
#pragma unroll
    for (int j = 0; j < NBUF; ++j) {
      const int t = i0 + j;
      if (t < ntiles) process(t, buf[j], v_lds[j & 1]);
      issue(t + NBUF, buf[j]);
    }
  }

  // row totals: the four lanes of row c16
  float lt = lsum + __shfl_xor(lsum, 16);
  lt += __shfl_xor(lt, 32);
  if (!rv) return;
  const bool empty = !(lt > 0.f);
  const float inv = empty ? 0.f : 1.0f / lt;
  const float lse_nat = empty ? -INFINITY : (m2 + __log2f(lt)) * LN2;
  // lane (c16, g4) holds O^T[16*db + 4*g4 + k][row c16], k = 0..3
  if (a.num_splits == 1) {
    uint16_t *op = static_cast<uint16_t *>(a.out) + qrow * D + 4 * g4;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const u32x2_t w = {pack_bf16x2(acc[db][0] * inv, acc[db][1] * inv),
                         pack_bf16x2(acc[db][2] * inv, acc[db][3] * inv)};
      *reinterpret_cast<u32x2_t *>(op + 16 * db) = w;
    }
    if (a.lse != nullptr && g4 == 0) a.lse[qrow] = lse_nat;
  } else {
    float *po = a.part_o + (qrow * S + split) * D + 4 * g4;
#pragma unroll
    for (int db = 0; db < DB; ++db)
      *reinterpret_cast<f32x4_t *>(po + 16 * db) = acc[db] * inv;
    if (g4 == 0) a.part_lse[qrow * S + split] = lse_nat;
  }
}

}  // namespace

hipError_t launch_decode_multi(const DecodeArgs &a, int head_dim, hipStream_t s) {
  if (a.q_len < 2 || a.q_len > 16 || a.hpw * a.q_len > 16 || a.hpw < 1) return hipErrorInvalidValue;
  const long long items = (long long)a.num_seqs * a.Hkv * a.num_splits * a.head_groups;
  dim3 grid((unsigned)items), block(64);
  if (head_dim == 128) {
    hipLaunchKernelGGL(decode_multi_kernel<128>, grid, block, 0, s, a);
  } else if (head_dim == 64) {
    hipLaunchKernelGGL(decode_multi_kernel<64>, grid, block, 0, s, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace rba
