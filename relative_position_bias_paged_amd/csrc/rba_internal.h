// Internal declarations shared by the host entry points and the kernels of
// librba.  Not part of the public ABI (include/rba.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rba {

// Arguments of the prefill kernels.  Pointers are device pointers.
struct PrefillArgs {
  const void *q;             // [T][Hq][D]
  const int32_t *cu_seqlens; // [B+1]
  const void *k_pool;        // [num_pages][Hkv][P][D]
  const void *v_pool;
  const int32_t *block_table; // [B][max_pages]
  const int32_t *seq_lens;    // prefill: keys held per sequence, this call's included (null: none before it)
  const void *bias;          // [T][Hq][R] (null in the fused variant)
  const void *rel_r;         // fused variant: [T][Hq][d_rel]
  const void *w_rel_t;       // fused variant: [R][d_rel], W^T
  void *out;                 // [T][Hq][D]
  float *lse;                // [T][Hq] or null
  int32_t num_seqs, Hq, Hkv, G, max_pages, page_size, log2_page;
  int32_t window, R;
  int32_t d_rel;             // fused variant: 16 or 32 (0 otherwise)
  int32_t total_tokens;      // T: rows of q, out and bias
  int32_t waves;             // waves per work-group (bf16 kernel: 4 or 8)
  int32_t hpw;               // query heads per work-group (divides G and waves)
  int32_t num_qtiles;        // query tiles per (sequence, head group)
  int32_t num_blocks;        // total work-groups of the launch
  float sm_scale;
};

// Arguments of the decode kernels.
struct DecodeArgs {
  const void *q;             // [B][Hq][D]
  const void *k_pool;
  const void *v_pool;
  const int32_t *block_table;
  const int32_t *seq_lens;   // [B]
  const void *bias;          // [B][Hq][R]
  void *out;                 // [B][Hq][D]
  float *lse;                // [B][Hq] or null
  float *part_o;             // [B][Hq][S][D] when S > 1
  float *part_lse;           // [B][Hq][S]   when S > 1
  // When S > 1: the (sequence, partition) items largest first, as written by
  // the plan kernel: {b * S + partition, seq_lens[b]}, then {-1, 0} for the
  // partitions that hold no key.  Null: the grid order is used as it is.
  int2 *plan;
  int32_t plan_shift;        // plan buckets: (chunk_pages - pages) >> plan_shift
  int32_t num_seqs, Hq, Hkv, G, max_pages, page_size, log2_page;
  int32_t window, R;
  int32_t num_splits;        // S
  int32_t chunk_pages;       // pages per partition
  int32_t head_groups;       // query-head groups per KV head: ceil(G / hpw)
  int32_t hpw;               // query heads per wave (decode_bf16_kernel: 4)
  // Query tokens per sequence: 1 for single-token decode.  With q_len > 1
  // (decode_multi_kernel) q, bias and out hold q_len rows per sequence,
  // row b * q_len + i at position n_b - q_len + i, n_b = max(seq_lens[b],
  // q_len); part_o is then [B * q_len][Hq][S][D], part_lse [B * q_len][Hq][S].
  int32_t q_len;
  float sm_scale;
};

// Arguments of the K/V append kernel (and of its reverse, the gather).
struct AppendArgs {
  void *k_rows;               // [total_new][Hkv][D]: read by the append,
  void *v_rows;               // written by the gather
  const int32_t *cu_new;      // [B+1] over the new tokens
  const int32_t *seq_lens;    // [B] keys held after the append
  const int32_t *block_table; // [B][max_pages]
  void *k_pool;               // [num_pages][Hkv][P][D]
  void *v_pool;
  int32_t total_new, num_seqs, Hkv, max_pages, page_size, log2_page, num_pages;
  int32_t row_bytes;          // head_dim * element size, a multiple of 16
};

// Arguments of the page-table check.
struct PageCheckArgs {
  const int32_t *block_table; // [B][max_pages]
  const int32_t *seq_lens;    // [B] keys held
  int32_t *bad;               // [1] count written
  int32_t num_seqs, max_pages, log2_page, num_pages, window, max_new;
};

hipError_t launch_prefill_bf16(const PrefillArgs &a, int head_dim, hipStream_t s);
hipError_t launch_prefill_fused(const PrefillArgs &a, int head_dim, hipStream_t s);
hipError_t launch_kv_append(const AppendArgs &a, bool gather, hipStream_t s);
hipError_t launch_decode_bf16(const DecodeArgs &a, int head_dim, hipStream_t s);
hipError_t launch_merge(const DecodeArgs &a, int head_dim, bool bf16_out, hipStream_t s);
hipError_t launch_decode_plan(const DecodeArgs &a, hipStream_t s);
hipError_t launch_prefill_f32(const PrefillArgs &a, int head_dim, hipStream_t s);
hipError_t launch_decode_f32(const DecodeArgs &a, int head_dim, hipStream_t s);
hipError_t launch_decode_multi(const DecodeArgs &a, int head_dim, hipStream_t s);
hipError_t launch_page_check(const PageCheckArgs &a, hipStream_t s);

}  // namespace rba
