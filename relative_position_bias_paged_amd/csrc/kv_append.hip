// kv_append.hip -- write the keys and values of new tokens into their pool
// pages, and the reverse gather.  Sequence b holds seq_lens[b] keys after the
// call, its L_b new tokens being the last L_b positions, so new token i of
// sequence b goes to position seq_lens[b] - L_b + i: pool page
// table[b][pos / page_size], slot pos % page_size (the page-table addressing
// of the TensorRT-LLM PR #17860 page, the commit that borrows the framework
// page table: positional entries, bounded by the sequence length).  The
// gather reads the same slots back into token rows, through the same
// indexing, so a gather of whole sequences de-pages the cache.
//
// One thread per 16-byte chunk of a new token's row, for a group of two KV
// heads: the sequence lookup and the page read serve both rows, and all four
// loads (K and V of both heads) are in flight before the first store.  The
// lanes of a chunk run cover consecutive tokens, so a page's slots are written
// by consecutive lanes.  The new rows are read once, with streaming loads.
// Larger head groups were measured slower: more rows per thread puts more
// writes of one wave 16 KB apart, at the same position in different pages.
// A position outside the table or a page id outside the pool is a broken
// caller contract: that token's rows are not written.
#include "rba_internal.h"

namespace rba {
namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kHeadGroup = 2;

// Block: 256 threads = (256 / chunks) tokens x chunks 16-byte chunks; grid.y
// runs over the head groups.  GATHER reverses the copy: pool slots to rows.
template <bool GATHER>
__global__ __launch_bounds__(256) void kv_append_kernel(AppendArgs a, int log2_chunks) {
  const int c = threadIdx.x & ((1 << log2_chunks) - 1);
  const int tok = blockIdx.x * (256 >> log2_chunks) + (threadIdx.x >> log2_chunks);
  if (tok >= a.total_new) return;
  // sequence of the token: the largest b with cu_new[b] <= tok
  int lo = 0, hi = a.num_seqs;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (a.cu_new[mid] <= tok) lo = mid;
    else hi = mid;
  }
  const int b = lo;
  const int first = a.cu_new[b];
  const int pos = a.seq_lens[b] - (a.cu_new[b + 1] - first) + (tok - first);
  if (pos < 0 || pos >= a.max_pages * a.page_size) return;
  const int page = a.block_table[(size_t)b * a.max_pages + (pos >> a.log2_page)];
  if (page < 0 || page >= a.num_pages) return;
  const int h0 = blockIdx.y * kHeadGroup;
  const int nh = min(kHeadGroup, a.Hkv - h0);
  const size_t rb = (size_t)a.row_bytes;
  const size_t src = ((size_t)tok * a.Hkv + h0) * rb + c * 16;
  const size_t dst = (((size_t)page * a.Hkv + h0) * a.page_size + (pos & (a.page_size - 1))) * rb +
                     c * 16;
  const size_t row_step = rb;                             // next head, same token
  const size_t head_step = (size_t)a.page_size * rb;     // next head, same slot
  char *kr = static_cast<char *>(a.k_rows) + src;
  char *vr = static_cast<char *>(a.v_rows) + src;
  char *kp = static_cast<char *>(a.k_pool) + dst;
  char *vp = static_cast<char *>(a.v_pool) + dst;
  u32x4_t kv[kHeadGroup], vv[kHeadGroup];
  if constexpr (GATHER) {
#pragma unroll
    for (int j = 0; j < kHeadGroup; ++j)
      if (j < nh) {
        kv[j] = *reinterpret_cast<const u32x4_t *>(kp + j * head_step);
        vv[j] = *reinterpret_cast<const u32x4_t *>(vp + j * head_step);
      }
#pragma unroll
    for (int j = 0; j < kHeadGroup; ++j)
      if (j < nh) {
        *reinterpret_cast<u32x4_t *>(kr + j * row_step) = kv[j];
        *reinterpret_cast<u32x4_t *>(vr + j * row_step) = vv[j];
      }
  } else {
#pragma unroll
    for (int j = 0; j < kHeadGroup; ++j)
      if (j < nh) {
        kv[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(kr + j * row_step));
        vv[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(vr + j * row_step));
      }
#pragma unroll
    for (int j = 0; j < kHeadGroup; ++j)
      if (j < nh) {
        *reinterpret_cast<u32x4_t *>(kp + j * head_step) = kv[j];
        *reinterpret_cast<u32x4_t *>(vp + j * head_step) = vv[j];
      }
  }
}

}  // namespace

hipError_t launch_kv_append(const AppendArgs &a, bool gather, hipStream_t s) {
  const int chunks = a.row_bytes / 16;
  int log2_chunks = 0;
  while ((1 << log2_chunks) < chunks) ++log2_chunks;
  if (a.row_bytes % 16 != 0 || (1 << log2_chunks) != chunks || chunks > 256)
    return hipErrorInvalidValue;
  const int tokens_per_block = 256 >> log2_chunks;
  const long long bx = ((long long)a.total_new + tokens_per_block - 1) / tokens_per_block;
  const long long by = ((long long)a.Hkv + kHeadGroup - 1) / kHeadGroup;
  if (bx <= 0 || by <= 0) return hipSuccess;
  if (bx > 0x7fffffffLL || by > 65535) return hipErrorInvalidValue;
  const dim3 grid((unsigned)bx, (unsigned)by);
  if (gather) hipLaunchKernelGGL(kv_append_kernel<true>, grid, dim3(256), 0, s, a, log2_chunks);
  else hipLaunchKernelGGL(kv_append_kernel<false>, grid, dim3(256), 0, s, a, log2_chunks);
  return hipGetLastError();
}

}  // namespace rba
