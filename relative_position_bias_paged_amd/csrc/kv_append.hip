// kv_append.hip -- write the keys and values of new tokens into their pool
// pages.  Sequence b holds seq_lens[b] keys after the call, its L_b new
// tokens being the last L_b positions, so new token i of sequence b goes to
// position seq_lens[b] - L_b + i: pool page table[b][pos / page_size], slot
// pos % page_size (the page-table addressing of the TensorRT-LLM PR #17860
// page, the commit that borrows the framework page table: positional
// entries, bounded by the sequence length).
//
// One thread per 16-byte chunk of a new (token, KV head) row, so a row is
// written by consecutive lanes.  A position outside the table or a page id
// outside the pool is a broken caller contract: that chunk is not written.
#include "rba_internal.h"

namespace rba {
namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void kv_append_kernel(AppendArgs a) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  const int chunks = a.row_bytes / 16;                 // 16-byte chunks per (token, head) row
  if (i >= (long long)a.total_new * a.Hkv * chunks) return;
  const int c = (int)(i % chunks);
  const long long r = i / chunks;
  const int h = (int)(r % a.Hkv);
  const int tok = (int)(r / a.Hkv);
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
  const size_t dst = (((size_t)page * a.Hkv + h) * a.page_size + (pos & (a.page_size - 1))) *
                         a.row_bytes + (size_t)c * 16;
  const size_t src = ((size_t)tok * a.Hkv + h) * a.row_bytes + (size_t)c * 16;
  const u32x4_t kv = *reinterpret_cast<const u32x4_t *>(static_cast<const char *>(a.k_new) + src);
  const u32x4_t vv = *reinterpret_cast<const u32x4_t *>(static_cast<const char *>(a.v_new) + src);
  *reinterpret_cast<u32x4_t *>(static_cast<char *>(a.k_pool) + dst) = kv;
  *reinterpret_cast<u32x4_t *>(static_cast<char *>(a.v_pool) + dst) = vv;
}

}  // namespace

hipError_t launch_kv_append(const AppendArgs &a, hipStream_t s) {
  const long long threads = (long long)a.total_new * a.Hkv * (a.row_bytes / 16);
  const long long blocks = (threads + 255) / 256;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(kv_append_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace rba
