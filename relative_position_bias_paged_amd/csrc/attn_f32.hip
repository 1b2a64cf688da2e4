// attn_f32.hip -- fp32 prefill and decode with a learned relative-position
// bias over a paged KV pool.  Same semantics as the bf16 kernels:
// score = sm_scale * q.k + bias[t,h,min(t-s,R-1)] over s <= t (and t - s <
// window on local layers), keys read through page = table[s / page_size],
// never past seq_len (TensorRT-LLM PR #17062 "Support Inkling-NVFP4 model",
// Description, Architecture list; TensorRT-LLM PR #17860 "Inkling attn
// backend cleanup fake registry", the commit that borrows the framework page
// table).
//
// One wave per query row (prefill token or decode sequence, and head).  The
// row's visible keys go in chunks of 64, one key per lane: each lane forms
// its key's full dot product (the query vector sits in LDS, read as
// broadcasts), the wave reduces the chunk's maximum and sum, and then the
// lanes switch to head-dim elements for P V, taking each key's probability
// from its lane with a uniform readlane.  The softmax runs online over the
// chunks in fp32.
#include "rba_internal.h"

namespace rba {
namespace {

constexpr int kRowsPerBlock = 4;     // waves (query rows) per work-group

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int sh = 32; sh > 0; sh >>= 1) x = fmaxf(x, __shfl_xor(x, sh));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int sh = 32; sh > 0; sh >>= 1) x += __shfl_xor(x, sh);
  return x;
}

// Attention of one query row at position t over keys [lo, t] of sequence
// row `trow` of the block table.  q_lds holds the query (D floats, this
// wave's own LDS slice); brow is the row's bias.  Returns the row output
// elements lane + 64*e (e < D/64) unnormalised, with the row max m and sum l.
template <int D>
__device__ __forceinline__ void attend_row_f32(const float *q_lds, const float *kp, const float *vp,
                                               const int32_t *trow, int Hkv, int g, int P, int lp,
                                               int t, int lo, const float *brow, int R,
                                               float sm_scale, float (&acc)[D / 64], float &m,
                                               float &l) {
  constexpr int E = D / 64;
  const int lane = threadIdx.x & 63;
  m = -INFINITY;
  l = 0.f;
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  auto row_of = [&](const float *pool, int s) {
    const int page = trow[s >> lp];
    return pool + (((size_t)page * Hkv + g) * P + (s & (P - 1))) * D;
  };
  for (int c0 = lo; c0 <= t; c0 += 64) {
    // scores: one key per lane
    const int s = c0 + lane;
    const bool vis = s <= t;
    float x = -INFINITY;
    if (vis) {
      const float4 *kr = reinterpret_cast<const float4 *>(row_of(kp, s));
      const float4 *qv = reinterpret_cast<const float4 *>(q_lds);
      float dot = 0.f;
#pragma unroll
      for (int i = 0; i < D / 4; ++i) {
        const float4 k4 = kr[i];
        const float4 q4 = qv[i];
        dot = fmaf(q4.x, k4.x, dot);
        dot = fmaf(q4.y, k4.y, dot);
        dot = fmaf(q4.z, k4.z, dot);
        dot = fmaf(q4.w, k4.w, dot);
      }
      x = fmaf(dot, sm_scale, brow[min(t - s, R - 1)]);
    }
    const float mn = fmaxf(m, wave_max(x));
    const float alpha = expf(m - mn);      // m = -inf on the first chunk: alpha = 0
    const float p = vis ? expf(x - mn) : 0.f;
    l = l * alpha + wave_sum(p);
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] *= alpha;
    m = mn;
    // P V: lanes over head-dim elements, keys of the chunk in turn
    const int nk = min(64, t - c0 + 1);
    for (int j = 0; j < nk; ++j) {
      const float pj = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, p), j));
      const float *vr = row_of(vp, c0 + j);
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] = fmaf(pj, vr[lane + 64 * e], acc[e]);
    }
  }
}

template <int D>
__global__ __launch_bounds__(64 * kRowsPerBlock) void prefill_f32_kernel(PrefillArgs a) {
  constexpr int E = D / 64;
  __shared__ __align__(16) float q_sh[kRowsPerBlock][D];
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int b = blockIdx.z;
  const int h = blockIdx.y;
  const int tok0 = a.cu_seqlens[b];
  const int L = a.cu_seqlens[b + 1] - tok0;
  const int i = blockIdx.x * kRowsPerBlock + wave;
  if (i >= L) return;
  // this call's L tokens are the last L of the n_k keys held for the
  // sequence (n_k = L without history): token i sits at position t
  const int n_k = a.seq_lens != nullptr ? max(a.seq_lens[b], L) : L;
  const int t = n_k - L + i;
  const int W = a.window;
  const size_t row = ((size_t)tok0 + i) * a.Hq + h;
  const float *qp = static_cast<const float *>(a.q) + row * D;
#pragma unroll
  for (int e = 0; e < E; ++e) q_sh[wave][lane + 64 * e] = qp[lane + 64 * e];
  __builtin_amdgcn_wave_barrier();   // the wave's own LDS slice: in-order within the wave
  float acc[E], m, l;
  attend_row_f32<D>(q_sh[wave], static_cast<const float *>(a.k_pool),
                    static_cast<const float *>(a.v_pool), a.block_table + (size_t)b * a.max_pages,
                    a.Hkv, h / a.G, a.page_size, a.log2_page, t,
                    (W > 0) ? max(0, t - W + 1) : 0, static_cast<const float *>(a.bias) + row * a.R,
                    a.R, a.sm_scale, acc, m, l);
  float *op = static_cast<float *>(a.out) + row * D;
  const float inv = 1.0f / l;
#pragma unroll
  for (int e = 0; e < E; ++e) op[lane + 64 * e] = acc[e] * inv;
  if (a.lse != nullptr && lane == 0) a.lse[row] = m + logf(l);
}

template <int D>
__global__ __launch_bounds__(64 * kRowsPerBlock) void decode_f32_kernel(DecodeArgs a) {
  constexpr int E = D / 64;
  __shared__ __align__(16) float q_sh[kRowsPerBlock][D];
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const size_t orow = (size_t)blockIdx.x * kRowsPerBlock + wave;   // b * Hq + h
  if (orow >= (size_t)a.num_seqs * a.Hq) return;
  const int b = (int)(orow / a.Hq);
  const int h = (int)(orow % a.Hq);
  const int n = a.seq_lens[b];
  const float *qp = static_cast<const float *>(a.q) + orow * D;
#pragma unroll
  for (int e = 0; e < E; ++e) q_sh[wave][lane + 64 * e] = qp[lane + 64 * e];
  __builtin_amdgcn_wave_barrier();
  float acc[E], m = -INFINITY, l = 0.f;
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  if (n > 0) {
    const int t = n - 1;
    attend_row_f32<D>(q_sh[wave], static_cast<const float *>(a.k_pool),
                      static_cast<const float *>(a.v_pool),
                      a.block_table + (size_t)b * a.max_pages, a.Hkv, h / a.G, a.page_size,
                      a.log2_page, t, (a.window > 0) ? max(0, n - a.window) : 0,
                      static_cast<const float *>(a.bias) + orow * a.R, a.R, a.sm_scale, acc, m, l);
  }
  // a sequence with no key gets a zero row and lse = -inf
  const float inv = l > 0.f ? 1.0f / l : 0.f;
  float *op = static_cast<float *>(a.out) + orow * D;
#pragma unroll
  for (int e = 0; e < E; ++e) op[lane + 64 * e] = acc[e] * inv;
  if (a.lse != nullptr && lane == 0) a.lse[orow] = l > 0.f ? m + logf(l) : -INFINITY;
}

}  // namespace

hipError_t launch_prefill_f32(const PrefillArgs &a, int head_dim, hipStream_t s) {
  // grid: (groups of kRowsPerBlock queries, head, sequence); a.num_qtiles
  // holds the group count
  dim3 grid(a.num_qtiles, a.Hq, a.num_seqs), block(64 * kRowsPerBlock);
  if (head_dim == 128) {
    hipLaunchKernelGGL(prefill_f32_kernel<128>, grid, block, 0, s, a);
  } else if (head_dim == 64) {
    hipLaunchKernelGGL(prefill_f32_kernel<64>, grid, block, 0, s, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_decode_f32(const DecodeArgs &a, int head_dim, hipStream_t s) {
  const long long rows = (long long)a.num_seqs * a.Hq;
  dim3 grid((unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock)), block(64 * kRowsPerBlock);
  if (head_dim == 128) {
    hipLaunchKernelGGL(decode_f32_kernel<128>, grid, block, 0, s, a);
  } else if (head_dim == 64) {
    hipLaunchKernelGGL(decode_f32_kernel<64>, grid, block, 0, s, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace rba
