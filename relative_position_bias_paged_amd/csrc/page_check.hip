// page_check.hip -- debug check of a positional page table (key position s
// of sequence b in pool page table[b][s / page_size], the addressing of the
// TensorRT-LLM PR #17860 page, the commit that borrows the framework page
// table: positional entries bounded by the sequence length).
//
// Counts the entries a call could reach that do not name a pool page: an
// index at or past max_pages_per_seq, or a page id outside [0, num_pages).
// The attention and append kernels do not check the pages they read; this
// is how a caller checks a table in a debug run without trapping the device.
#include "rba_internal.h"

namespace rba {
namespace {

__global__ void clear_count_kernel(int32_t *count) {
  if (threadIdx.x == 0 && blockIdx.x == 0) *count = 0;
}

// One work-group per sequence; its threads stride over the sequence's
// reachable entries.  Entries past the table are counted without reading it.
__global__ __launch_bounds__(256) void check_table_kernel(PageCheckArgs a) {
  __shared__ int32_t wg_count;
  if (threadIdx.x == 0) wg_count = 0;
  __syncthreads();
  const int b = blockIdx.x;
  const long long n = max(a.seq_lens[b], 0);
  if (n > 0) {
    const long long lo = a.window > 0 ? max(0LL, n - a.max_new - a.window + 1) : 0;
    const long long j_lo = lo >> a.log2_page, j_hi = (n - 1) >> a.log2_page;
    int32_t local = 0;
    for (long long j = j_lo + threadIdx.x; j <= j_hi; j += blockDim.x) {
      if (j >= a.max_pages) {
        ++local;
        continue;
      }
      const int32_t page = a.block_table[(size_t)b * a.max_pages + j];
      if (page < 0 || page >= a.num_pages) ++local;
    }
    if (local != 0) atomicAdd(&wg_count, local);
  }
  __syncthreads();
  if (threadIdx.x == 0 && wg_count != 0) atomicAdd(a.bad, wg_count);
}

}  // namespace

hipError_t launch_page_check(const PageCheckArgs &a, hipStream_t s) {
  hipLaunchKernelGGL(clear_count_kernel, dim3(1), dim3(64), 0, s, a.bad);
  if (a.num_seqs > 0)
    hipLaunchKernelGGL(check_table_kernel, dim3((unsigned)a.num_seqs), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace rba
