// attn_f32.hip -- fp32 prefill and decode with a learned relative-position
// bias over a paged KV pool.  A plain path for float32 layers: one thread per
// prefill query row (two passes: row max, then exp-sum and P V), one wave per
// decode row with the head dimension spread over the lanes.  Same semantics as
// the bf16 kernels: score = sm_scale * q.k + bias[t,h,min(t-s,R-1)] over
// s <= t (and t - s < window on local layers), keys read through
// page = table[s / page_size], never past seq_len (TensorRT-LLM PR #17062
// "Support Inkling-NVFP4 model", Description, Architecture list; TensorRT-LLM
// PR #17860 "Inkling attn backend cleanup fake registry", the commit that
// borrows the framework page table).
#include "rba_internal.h"

namespace rba {
namespace {

template <int D>
__global__ __launch_bounds__(64) void prefill_f32_kernel(PrefillArgs a) {
  const int b = blockIdx.z;
  const int h = blockIdx.y;
  const int tok0 = a.cu_seqlens[b];
  const int L = a.cu_seqlens[b + 1] - tok0;
  const int i = blockIdx.x * 64 + threadIdx.x;
  if (i >= L) return;
  // this call's L tokens are the last L of the n_k keys held for the
  // sequence (n_k = L without history): token i sits at position t
  const int n_k = a.seq_lens != nullptr ? max(a.seq_lens[b], L) : L;
  const int t = n_k - L + i;
  const int g = h / a.G;
  const int R = a.R, W = a.window, P = a.page_size, lp = a.log2_page;
  const float *qp = static_cast<const float *>(a.q);
  const float *kp = static_cast<const float *>(a.k_pool);
  const float *vp = static_cast<const float *>(a.v_pool);
  const float *bp = static_cast<const float *>(a.bias);
  const int32_t *trow = a.block_table + (size_t)b * a.max_pages;
  const size_t row = ((size_t)tok0 + i) * a.Hq + h;

  float q[D];
#pragma unroll
  for (int i = 0; i < D; ++i) q[i] = qp[row * D + i];
  const float *brow = bp + row * R;
  const int lo = (W > 0) ? max(0, t - W + 1) : 0;

  auto key_ptr = [&](const float *pool, int s) {
    const int page = trow[s >> lp];
    return pool + (((size_t)page * a.Hkv + g) * P + (s & (P - 1))) * D;
  };
  auto score = [&](int s) {
    const float *kr = key_ptr(kp, s);
    float dot = 0.f;
#pragma unroll
    for (int i = 0; i < D; ++i) dot = fmaf(q[i], kr[i], dot);
    return fmaf(dot, a.sm_scale, brow[min(t - s, R - 1)]);
  };

  float m = -INFINITY;
  for (int s = lo; s <= t; ++s) m = fmaxf(m, score(s));
  float acc[D];
#pragma unroll
  for (int i = 0; i < D; ++i) acc[i] = 0.f;
  float l = 0.f;
  for (int s = lo; s <= t; ++s) {
    const float p = expf(score(s) - m);
    l += p;
    const float *vr = key_ptr(vp, s);
#pragma unroll
    for (int i = 0; i < D; ++i) acc[i] = fmaf(p, vr[i], acc[i]);
  }
  float *op = static_cast<float *>(a.out) + row * D;
  const float inv = 1.0f / l;
#pragma unroll
  for (int i = 0; i < D; ++i) op[i] = acc[i] * inv;
  if (a.lse != nullptr) a.lse[row] = m + logf(l);
}

template <int D>
__global__ __launch_bounds__(64) void decode_f32_kernel(DecodeArgs a) {
  constexpr int E = D / 64;
  const int lane = threadIdx.x;
  const size_t orow = blockIdx.x;               // b * Hq + h
  const int b = (int)(orow / a.Hq);
  const int h = (int)(orow % a.Hq);
  const int g = h / a.G;
  const int n = a.seq_lens[b];
  const int t = n - 1;
  const int R = a.R, W = a.window, P = a.page_size, lp = a.log2_page;
  const float *qp = static_cast<const float *>(a.q);
  const float *kp = static_cast<const float *>(a.k_pool);
  const float *vp = static_cast<const float *>(a.v_pool);
  const float *bp = static_cast<const float *>(a.bias);
  const int32_t *trow = a.block_table + (size_t)b * a.max_pages;
  float q[E], acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    q[e] = qp[orow * D + lane * E + e];
    acc[e] = 0.f;
  }
  const float *brow = bp + orow * R;
  const int lo = (W > 0) ? max(0, n - W) : 0;
  float m = -INFINITY, l = 0.f;
  for (int s = lo; s < n; ++s) {
    const int page = trow[s >> lp];
    const size_t off = (((size_t)page * a.Hkv + g) * P + (s & (P - 1))) * D + lane * E;
    float dot = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) dot = fmaf(q[e], kp[off + e], dot);
#pragma unroll
    for (int sh = 32; sh > 0; sh >>= 1) dot += __shfl_xor(dot, sh);
    const float x = fmaf(dot, a.sm_scale, brow[min(t - s, R - 1)]);
    const float mn = fmaxf(m, x);
    const float alpha = expf(m - mn);   // m = -inf on the first key: alpha = 0
    const float p = expf(x - mn);
    l = l * alpha + p;
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = fmaf(p, vp[off + e], acc[e] * alpha);
    m = mn;
  }
  const float inv = l > 0.f ? 1.0f / l : 0.f;
  float *op = static_cast<float *>(a.out) + orow * D + lane * E;
#pragma unroll
  for (int e = 0; e < E; ++e) op[e] = acc[e] * inv;
  if (a.lse != nullptr && lane == 0) a.lse[orow] = l > 0.f ? m + logf(l) : -INFINITY;
}

}  // namespace

hipError_t launch_prefill_f32(const PrefillArgs &a, int head_dim, hipStream_t s) {
  // grid: (query blocks of 64, head, sequence); a.num_qtiles holds the block count
  dim3 grid(a.num_qtiles, a.Hq, a.num_seqs), block(64);
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
  dim3 grid((unsigned)((long long)a.num_seqs * a.Hq)), block(64);
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
