// decode_bf16.hip -- single-token decode with a learned relative-position bias
// over a paged KV pool, bf16 in / fp32 accumulate, for gfx950 (CDNA4).
//
// The query of sequence b sits at position t = n_b - 1 and attends keys
// s in [lo, n_b), lo = max(0, n_b - window) on local layers, 0 on global
// ones, with score sm_scale * q.k + bias[b,h,min(t-s, R-1)] (TensorRT-LLM
// PR #17062 "Support Inkling-NVFP4 model", Description, Architecture list:
// the bias is per (query token, head, relative distance) and added before
// softmax; the decode kernel reads keys through the page table, page =
// table[k_pos / page_size], bounded by k_pos < seq_len, as the TensorRT-LLM
// PR #17860 "Inkling attn backend cleanup fake registry" commit that borrows
// the framework page table describes).
//
// One wave owns (sequence, KV head, up to 4 of its query heads, one
// page-aligned partition of the visible keys).  Decode is HBM-bound: every K
// and V byte is read once, and the work per byte is small, so the layout
// favours many bytes in flight:
//  * keys are processed in 16-key tiles; four tiles of K, V and bias are in
//    flight while one is computed;
//  * S = Q K^T runs on v_mfma_f32_16x16x32_bf16 with the (up to 4) query
//    heads replicated over the 16 A rows, so every lane ends up holding the
//    scores of its key column for all heads;
//  * P V runs on the VALU: lane (dg, kg) accumulates head-dim slice dg over
//    keys 4kg..4kg+3 of each tile, fetching the probabilities of those keys
//    with ds_bpermute; partial sums of the four lane groups are folded once
//    at the end.
// Partitions write a normalised fp32 partial output and its natural-log LSE
// to the workspace; merge_kernel combines them with weights exp(lse_j - max).
//
// With partitions, plan_kernel first orders the (sequence, partition) items
// largest first (a counting sort on the device, so the host never reads the
// sequence lengths).  The hardware hands out work-groups in grid order, and
// one wave streams at most a few GB/s however idle the memory system is, so
// a long partition dispatched late would run on alone at the end; largest
// first leaves the short ones for the tail.  The order changes no result:
// every partition writes its own slot and the merge reads them in a fixed
// order.
#include "rba_internal.h"

namespace rba {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;
constexpr float NEG_INIT = -1.0e30f;
constexpr float TAU = 8.0f;
constexpr int NBUF = 4;     // tiles in flight

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Max / sum over the 16 lanes of a DPP row; every lane gets the result.
__device__ __forceinline__ float row16_max(float x) {
  x = fmaxf(x, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false)));
  x = fmaxf(x, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, false)));
  x = fmaxf(x, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x141, 0xF, 0xF, false)));
  x = fmaxf(x, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x140, 0xF, 0xF, false)));
  return x;
}
__device__ __forceinline__ float row16_sum(float x) {
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x141, 0xF, 0xF, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x140, 0xF, 0xF, false));
  return x;
}

__device__ __forceinline__ float lane_read(float x, int src_lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src_lane << 2, __builtin_bit_cast(int, x)));
}

template <int D>
struct TileBuf {
  u32x4_t k[D / 32];                     // K[key = c16][32*kk + 8*g4 ..+8]
  uint32_t v[4][D / 32];                 // V[4*kg+i][(D/16)*dg ..+D/16], D/32 dwords each
  uint32_t bias[4];                      // raw bf16 bias of (head r, key c16)
};

template <int D>
__global__ __launch_bounds__(64) void decode_bf16_kernel(DecodeArgs a) {
  constexpr int KK = D / 32;      // MFMAs over head_dim; also dwords per V slice
  constexpr int DV = D / 16;      // head-dim elements per lane in P V
  const int lane = threadIdx.x;
  const int c16 = lane & 15;
  const int g4 = lane >> 4;

  // Block -> (partition, sequence, KV head, head group), partition slowest.
  // Blocks are dealt to the 8 XCDs round-robin, so every XCD gets a mix of
  // sequences at every partition index; with the partition fastest, a
  // partition count that is a multiple of 8 would send partition j to XCD
  // j mod 8 every time, and the late partitions (which exist only for long
  // sequences) would leave some XCDs idle while others still work.
  const int S = a.num_splits;
  const int HG = a.head_groups;
  int item = blockIdx.x;
  const int hg = item % HG;
  item /= HG;
  const int kvh = item % a.Hkv;
  item /= a.Hkv;
  int b, split, n;
  if (a.plan != nullptr) {
    // item-th largest (sequence, partition); the record carries the length
    const int2 rec = a.plan[item];
    if (rec.x < 0) return;               // a partition with no key: nothing to merge
    b = rec.x / S;
    split = rec.x - b * S;
    n = rec.y;
  } else {
    b = item % a.num_seqs;
    split = item / a.num_seqs;
    n = a.seq_lens[b];
  }

  const int G = a.G;
  const int h_base = kvh * G + hg * 4;
  const int nh = min(4, G - hg * 4);
  const int Hq = a.Hq;
  const int R = a.R;
  const int W = a.window;
  const int P = a.page_size;
  const int lp = a.log2_page;

  const int t = n - 1;
  const int lo = (W > 0) ? max(0, n - W) : 0;
  const int p_first = lo >> lp;
  const int p_end = (n + P - 1) >> lp;
  const int pg_lo = p_first + split * a.chunk_pages;
  const int pg_hi = min(p_first + (split + 1) * a.chunk_pages, p_end);
  const int k_lo = max(pg_lo << lp, lo) & ~15;         // first 16-key tile
  const int k_hi = min(pg_hi << lp, n);                // exclusive
  const int ntiles = (n > 0 && pg_lo < pg_hi) ? (k_hi - k_lo + 15) >> 4 : 0;
  // the merge reads only partitions that hold keys
  if (S > 1 && ntiles == 0) return;

  const uint16_t *qp = static_cast<const uint16_t *>(a.q);
  const uint16_t *kp = static_cast<const uint16_t *>(a.k_pool);
  const uint16_t *vp = static_cast<const uint16_t *>(a.v_pool);
  const uint16_t *bp = static_cast<const uint16_t *>(a.bias);
  const int32_t *trow = a.block_table + (size_t)b * a.max_pages;
  const size_t head_stride = (size_t)P * D;
  const size_t page_stride = (size_t)a.Hkv * head_stride;

  // Q as the A operand: row i = c16 carries head (i & 3) of this group.
  // k-slot group g4 of MFMA kk holds head-dim elements 32*kk + 8*g4 .. +8.
  const int qr = c16 & 3;
  u32x4_t qa[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    const u32x4_t v = *reinterpret_cast<const u32x4_t *>(
        qp + ((size_t)b * Hq + h_base + min(qr, nh - 1)) * D + 32 * kk + 8 * g4);
    qa[kk] = (qr < nh) ? v : u32x4_t{0, 0, 0, 0};
  }
  // bias rows of the (up to 4) heads; heads past nh reuse the last one
  const uint16_t *brow[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) brow[r] = bp + ((size_t)b * Hq + h_base + min(r, nh - 1)) * R;
  float b_last[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) b_last[r] = bf16_to_f32(brow[r][R - 1]);

  TileBuf<D> buf[NBUF];

  // Every load is unconditional: a tile index past the end re-reads the last
  // tile (already in cache), heads past nh read a valid row, and clamp-only
  // tiles read bucket R-1, so no load sits behind a branch and the waits
  // before each tile's use only cover that tile.  V is read once, by this
  // wave only, each load instruction covering whole 128-byte lines, so it is
  // loaded with the streaming (non-temporal) cache policy, which sustains a
  // higher HBM read rate.  K keeps the default policy: its two load
  // instructions per 32 head-dim elements each read half of the same lines,
  // and under the streaming policy the second half was often fetched again.
  auto issue = [&](int ti, TileBuf<D> &tb) {
    const int ts = k_lo + min(ti, ntiles - 1) * 16;     // first key of the tile
    const int page = trow[ts >> lp];
    const size_t base = (size_t)page * page_stride + (size_t)kvh * head_stride +
                        (size_t)(ts & (P - 1)) * D;
    const uint16_t *kt = kp + base + (size_t)c16 * D + 8 * g4;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      tb.k[kk] = *reinterpret_cast<const u32x4_t *>(kt + 32 * kk);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint16_t *vt = vp + base + (size_t)(4 * g4 + i) * D + DV * c16;
      if constexpr (KK == 4) {
        const u32x4_t w = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(vt));
        tb.v[i][0] = w[0]; tb.v[i][1] = w[1]; tb.v[i][2] = w[2]; tb.v[i][3] = w[3];
      } else {
        const u32x2_t w = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t *>(vt));
        tb.v[i][0] = w[0]; tb.v[i][1] = w[1];
      }
    }
    // bias of this lane's key for each head; tiles entirely at distance
    // >= R-1 use b_last and skip the load
    const bool band = (t - (ts + 15)) < R - 1;
    const int idx = band ? min(max(t - (ts + c16), 0), R - 1) : R - 1;
#pragma unroll
    for (int r = 0; r < 4; ++r) tb.bias[r] = brow[r][idx];
  };

  float acc[4][DV];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int e = 0; e < DV; ++e) acc[r][e] = 0.f;
  float m2[4], lsum[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) { m2[r] = NEG_INIT; lsum[r] = 0.f; }
  const float scale = a.sm_scale;

  auto process = [&](int ti, const TileBuf<D> &tb) {
    const int ts = k_lo + ti * 16;
    f32x4_t sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, qa[kk]),
                                                     __builtin_bit_cast(bf16x8_t, tb.k[kk]), sacc, 0, 0, 0);
    // lane holds score(head r, key ts + c16) in sacc[r]
    const int s = ts + c16;
    const int d = t - s;
    const bool band = (t - (ts + 15)) < R - 1;
    const bool need_mask = (ts < lo) || (ts + 16 > n);
    const bool vis = (s >= lo) && (s < n);
    float p[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float bv = (band && d < R - 1) ? bf16_to_f32(tb.bias[r]) : b_last[r];
      float x = fmaf(sacc[r], scale, bv);
      if (need_mask) x = vis ? x : -INFINITY;
      const float mt2 = row16_max(x) * LOG2E;
      const bool exceed = mt2 > m2[r] + TAU;
      if (exceed) {   // uniform: all lanes hold the same row maximum
        const float alpha = __builtin_amdgcn_exp2f(m2[r] - mt2);
        lsum[r] *= alpha;
#pragma unroll
        for (int e = 0; e < DV; ++e) acc[r][e] *= alpha;
        m2[r] = mt2;
      }
      p[r] = __builtin_amdgcn_exp2f(fmaf(x, LOG2E, -m2[r]));
      lsum[r] += p[r];
    }
    // P V on the VALU: keys 4*g4 + i, head-dim slice c16
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int src = 4 * g4 + i;
      float vf[DV];
#pragma unroll
      for (int w = 0; w < KK; ++w) {
        vf[2 * w] = __uint_as_float(tb.v[i][w] << 16);
        vf[2 * w + 1] = __uint_as_float(tb.v[i][w] & 0xffff0000u);
      }
      if (need_mask) {
        const int sk = ts + src;
        const bool vk = (sk >= lo) && (sk < n);
#pragma unroll
        for (int e = 0; e < DV; ++e) vf[e] = vk ? vf[e] : 0.f;
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (r < nh) {
          const float pr = lane_read(p[r], src);
#pragma unroll
          for (int e = 0; e < DV; ++e) acc[r][e] = fmaf(pr, vf[e], acc[r][e]);
        }
      }
    }
  };

  // software pipeline: NBUF tiles in flight
  if (ntiles > 0) {
#pragma unroll
    for (int j = 0; j < NBUF; ++j) issue(j, buf[j]);
    for (int i0 = 0; i0 < ntiles; i0 += NBUF) {
#pragma unroll
      for (int j = 0; j < NBUF; ++j) {
        const int ti = i0 + j;
        if (ti < ntiles) process(ti, buf[j]);
        issue(ti + NBUF, buf[j]);
      }
    }
  }

  // fold the four key groups (lanes c16, c16+16, c16+32, c16+48)
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int e = 0; e < DV; ++e) {
      float x = acc[r][e];
      x += __shfl_xor(x, 16);
      x += __shfl_xor(x, 32);
      acc[r][e] = x;
    }
  float ltot[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) ltot[r] = row16_sum(lsum[r]);

  // lane (c16, g4) writes head r = g4, head-dim slice c16
  const int r = g4;
  if (r >= nh) return;
  float o[DV];
  float lt = ltot[0], mm = m2[0];
#pragma unroll
  for (int e = 0; e < DV; ++e) o[e] = acc[0][e];
#pragma unroll
  for (int rr = 1; rr < 4; ++rr)
    if (r == rr) {
      lt = ltot[rr];
      mm = m2[rr];
#pragma unroll
      for (int e = 0; e < DV; ++e) o[e] = acc[rr][e];
    }
  const int h = h_base + r;
  const size_t orow = (size_t)b * Hq + h;
  const bool empty = !(lt > 0.f);
  const float inv = empty ? 0.f : 1.0f / lt;
  const float lse_nat = empty ? -INFINITY : (mm + __log2f(lt)) * LN2;
  if (S == 1) {
    uint16_t *op = static_cast<uint16_t *>(a.out) + orow * D + DV * c16;
#pragma unroll
    for (int w = 0; w < KK; ++w) {
      const __bf16 x0 = static_cast<__bf16>(o[2 * w] * inv);
      const __bf16 x1 = static_cast<__bf16>(o[2 * w + 1] * inv);
      reinterpret_cast<uint32_t *>(op)[w] =
          (uint32_t)__builtin_bit_cast(uint16_t, x0) | ((uint32_t)__builtin_bit_cast(uint16_t, x1) << 16);
    }
    if (a.lse != nullptr && c16 == 0) a.lse[orow] = lse_nat;
  } else {
    float *po = a.part_o + (orow * S + split) * D + DV * c16;
#pragma unroll
    for (int e = 0; e < DV; ++e) po[e] = o[e] * inv;
    if (c16 == 0) a.part_lse[orow * S + split] = lse_nat;
  }
}

// One wave per (sequence, query head): out = sum_j w_j o_j / sum_j w_j with
// w_j = exp(lse_j - max_j lse_j) over the partitions that hold keys (the
// first ceil((p_end - p_first) / chunk) of them; the others wrote nothing).
// With q_len > 1 the row's sequence is orow / (Hq * q_len) and the
// partitions cover the keys any of its q_len queries sees.
template <int D>
__global__ __launch_bounds__(64) void merge_kernel(DecodeArgs a, int bf16_out) {
  constexpr int E = D / 64;      // elements per lane
  const int lane = threadIdx.x;
  const size_t orow = blockIdx.x;
  const int S = a.num_splits;
  const int ql = a.q_len;
  const int n_raw = a.seq_lens[orow / ((size_t)a.Hq * ql)];
  const int n = ql > 1 ? max(n_raw, ql) : n_raw;
  const int lo = (a.window > 0) ? max(0, n - ql - a.window + 1) : 0;
  const int span = ((n + a.page_size - 1) >> a.log2_page) - (lo >> a.log2_page);
  const int S_b = n > 0 ? min(S, (span + a.chunk_pages - 1) / a.chunk_pages) : 0;
  const float *pl = a.part_lse + orow * S;
  float M = -INFINITY;
  for (int j = 0; j < S_b; ++j) M = fmaxf(M, pl[j]);
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  float wsum = 0.f;
  if (M > -INFINITY) {
    for (int j = 0; j < S_b; ++j) {
      const float lj = pl[j];
      if (lj > -INFINITY) {
        const float w = __expf(lj - M);
        wsum += w;
        const float *po = a.part_o + (orow * S + j) * D + lane * E;
#pragma unroll
        for (int e = 0; e < E; ++e) acc[e] = fmaf(w, po[e], acc[e]);
      }
    }
  }
  const float inv = wsum > 0.f ? 1.0f / wsum : 0.f;
  if (bf16_out) {
    uint16_t *op = static_cast<uint16_t *>(a.out) + orow * D + lane * E;
#pragma unroll
    for (int e = 0; e < E; ++e) op[e] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(acc[e] * inv));
  } else {
    float *op = static_cast<float *>(a.out) + orow * D + lane * E;
#pragma unroll
    for (int e = 0; e < E; ++e) op[e] = acc[e] * inv;
  }
  if (a.lse != nullptr && lane == 0) a.lse[orow] = (wsum > 0.f) ? M + __logf(wsum) : -INFINITY;
}

// Largest-first order of the (sequence, partition) items for the decode grid:
// a counting sort on (chunk_pages - pages) >> plan_shift, with the empty
// partitions last as {-1, 0}.  (Shared with decode_multi_kernel: the record
// carries the key count n_b it planned with.)  One work-group; positions within a bucket
// follow LDS atomics, which changes dispatch order only, never a result.
constexpr int kPlanBuckets = 257;        // 256 size classes + the empty ones
__global__ __launch_bounds__(1024) void plan_kernel(DecodeArgs a) {
  __shared__ int hist[kPlanBuckets];
  const int S = a.num_splits;
  const int C = a.chunk_pages;
  const int items = a.num_seqs * S;
  const int lp = a.log2_page;
  const int ql = a.q_len;
  auto bucket_of = [&](int it, int &n) {
    const int b = it / S;
    const int j = it - b * S;
    n = ql > 1 ? max(a.seq_lens[b], ql) : a.seq_lens[b];
    const int lo = (a.window > 0) ? max(0, n - ql - a.window + 1) : 0;
    const int p_first = lo >> lp;
    const int p_end = (n + a.page_size - 1) >> lp;
    const int pages = (n > 0) ? max(0, min(p_first + (j + 1) * C, p_end) - (p_first + j * C)) : 0;
    return pages > 0 ? (C - pages) >> a.plan_shift : kPlanBuckets - 1;
  };
  for (int i = threadIdx.x; i < kPlanBuckets; i += blockDim.x) hist[i] = 0;
  __syncthreads();
  for (int it = threadIdx.x; it < items; it += blockDim.x) {
    int n;
    atomicAdd(&hist[bucket_of(it, n)], 1);
  }
  __syncthreads();
  if (threadIdx.x == 0) {                // exclusive prefix over the buckets
    int run = 0;
    for (int k = 0; k < kPlanBuckets; ++k) {
      const int c = hist[k];
      hist[k] = run;
      run += c;
    }
  }
  __syncthreads();
  for (int it = threadIdx.x; it < items; it += blockDim.x) {
    int n;
    const int k = bucket_of(it, n);
    const int pos = atomicAdd(&hist[k], 1);
    a.plan[pos] = (k == kPlanBuckets - 1) ? int2{-1, 0} : int2{it, n};
  }
}

}  // namespace

hipError_t launch_decode_plan(const DecodeArgs &a, hipStream_t s) {
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(1024), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_decode_bf16(const DecodeArgs &a, int head_dim, hipStream_t s) {
  if (a.q_len != 1 || a.hpw != 4) return hipErrorInvalidValue;
  const long long items = (long long)a.num_seqs * a.Hkv * a.num_splits * a.head_groups;
  dim3 grid((unsigned)items), block(64);
  if (head_dim == 128) {
    hipLaunchKernelGGL(decode_bf16_kernel<128>, grid, block, 0, s, a);
  } else if (head_dim == 64) {
    hipLaunchKernelGGL(decode_bf16_kernel<64>, grid, block, 0, s, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_merge(const DecodeArgs &a, int head_dim, bool bf16_out, hipStream_t s) {
  dim3 grid((unsigned)((long long)a.num_seqs * a.q_len * a.Hq)), block(64);
  if (head_dim == 128) {
    hipLaunchKernelGGL(merge_kernel<128>, grid, block, 0, s, a, bf16_out ? 1 : 0);
  } else if (head_dim == 64) {
    hipLaunchKernelGGL(merge_kernel<64>, grid, block, 0, s, a, bf16_out ? 1 : 0);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace rba
