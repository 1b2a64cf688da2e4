/*
 * rba.h -- C ABI of librba: paged attention with a learned relative-position
 * bias, for AMD Instinct MI355X (gfx950).
 *
 * What the library computes.  For query position t of a sequence, query head
 * h and every key position s of the same sequence,
 *
 *   score(t,s) = sm_scale * <q[t,h,:], k[s,g,:]> + bias[t,h,min(t-s, R-1)]
 *   visible    = s <= t  and  (window <= 0  or  t - s < window)
 *   out[t,h,:] = sum over visible s of softmax_s(score) * v[s,g,:]
 *
 * with g = h / (Hq / Hkv) and R = rel_extent.  Sources: TensorRT-LLM PR #17062
 * "Support Inkling-NVFP4 model" -- Description, Architecture list (no RoPE;
 * the position signal is a learned bias per (query token, head, relative
 * distance) added before softmax; local layers use a causal sliding window,
 * global layers are full causal), and its review comment on _build_rel_logits
 * (the bias tensor is [T, heads, rel_extent]); TensorRT-LLM PR #17860 "Inkling
 * attn backend cleanup fake registry" -- the commit making both Triton entry
 * points assert num_heads % num_kv_heads (query head -> KV head is
 * h // kv_group_num), and the commit borrowing the framework page table (keys
 * are addressed as page = table[k_pos // page_size]; entries past a
 * sequence's last page are never read because every access is bounded by
 * k_pos < seq_len).
 *
 * General conventions (every entry point):
 *  - All tensor pointers are DEVICE pointers to caller-owned memory.  The
 *    library never allocates, frees or synchronises; work is enqueued on
 *    `stream` (NULL = the null stream) and the call returns immediately.
 *  - Host-side argument checks run before anything is enqueued; on any error
 *    nothing is enqueued and the output is untouched.  Device contents (page
 *    ids, sequence lengths) are never read by the host: keeping them in range
 *    is the caller's contract (page ids in [0, num_pages) for every page
 *    that holds a key below seq_len).
 *  - Tensor pointers must be 16-byte aligned; all tensors are contiguous,
 *    row-major in the shapes given.
 *  - No C++ exception crosses the ABI.  Apart from rba_decode_noalloc's
 *    per-device workspace (see there), the library holds no mutable global
 *    state; calls on different streams may run concurrently.
 */
#ifndef RBA_H
#define RBA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum rba_status {
  RBA_OK = 0,
  RBA_ERR_INVALID_ARG = 1, /* a null pointer, an inconsistent size, Hq % Hkv != 0,
                              page_size not a power of two, rel_extent < 1, ... */
  RBA_ERR_UNSUPPORTED = 2, /* valid, but not a shape/dtype the library's kernels
                              run (see each call) */
  RBA_ERR_WORKSPACE = 3,   /* workspace null or smaller than required */
  RBA_ERR_HIP = 4          /* the HIP runtime reported an error at launch */
} rba_status;

typedef enum rba_dtype {
  RBA_BF16 = 0, /* q, k, v, bias and out in bfloat16 (fp32 accumulation) */
  RBA_F32 = 1   /* q, k, v, bias and out in float32 */
} rba_dtype;

/*
 * Page table.  Key position s of sequence b lives in pool page
 * block_table[b * max_pages_per_seq + s / page_size], slot s % page_size.
 * The table is positional: entry j always describes key positions
 * j*page_size .. j*page_size + page_size - 1.  Entries at or past
 * ceil(seq_lens[b] / page_size) are never read (0 by convention).
 */
typedef struct rba_page_table {
  const int32_t *block_table; /* device, [num_seqs][max_pages_per_seq] */
  const int32_t *seq_lens;    /* device, [num_seqs]: keys held per sequence,
                                 the keys of this call's tokens included
                                 (prefill: may be NULL when every sequence
                                 holds exactly its new tokens) */
  int32_t num_seqs;
  int32_t max_pages_per_seq;
  int32_t page_size;          /* power of two, 16 .. 1024 */
  int32_t num_pages;          /* pool size in pages */
} rba_page_table;

/*
 * Paged KV pool.  K and V are separate pools of identical shape
 * [num_pages][num_kv_heads][page_size][head_dim]: inside one page, each KV
 * head's page_size x head_dim block is contiguous.
 */
typedef struct rba_kv_cache {
  const void *k_pool;
  const void *v_pool;
  int32_t num_kv_heads;
  int32_t head_dim;           /* bf16: 64 or 128; f32: 64 or 128 */
  rba_dtype dtype;            /* also the dtype of q, bias and out */
} rba_kv_cache;

/*
 * Per-layer scalars (the three the pages name: sm_scale, rel_extent and the
 * window, with window <= 0 meaning full causal like window_left = -1).
 */
typedef struct rba_attn_params {
  int32_t num_q_heads;        /* Hq, a multiple of num_kv_heads */
  int32_t window;             /* > 0: key visible iff 0 <= t - s < window;
                                 <= 0: full causal */
  int32_t rel_extent;         /* R >= 1: buckets per bias row; distances
                                 >= R-1 share bucket R-1 */
  float sm_scale;             /* > 0, finite; multiplies q.k, not the bias */
} rba_attn_params;

/*
 * Prefill: every token of this call is a query.  Sequence b holds n_b =
 * pt->seq_lens[b] keys in the pool, the keys of its L_b new tokens included
 * (already written); the new tokens are its last L_b positions, so token
 * cu_seqlens[b]+i sits at position n_b - L_b + i and sees the keys before
 * it (chunked prefill, or several new tokens of a decode step).  With
 * n_b == L_b (or seq_lens NULL) this is a plain prefill of whole sequences.
 * Source of the semantics: the TensorRT-LLM PR #17062 page, Description,
 * Architecture list (bias per query token, head and distance); the
 * positions follow from the keys being the sequence's history.
 *
 *  q           [total_tokens][Hq][head_dim]; sequence b owns tokens
 *              cu_seqlens[b] .. cu_seqlens[b+1]-1
 *  cu_seqlens  device int32 [num_seqs + 1], non-decreasing, cu[0] = 0,
 *              cu[num_seqs] = total_tokens
 *  pt->seq_lens  n_b >= L_b (device data, not checked on the host; a value
 *              below L_b is read as L_b), n_b <= max_pages_per_seq *
 *              page_size
 *  max_seqlen  host bound on max_b L_b (sizes the grid)
 *  bias        [total_tokens][Hq][rel_extent]
 *  out         [total_tokens][Hq][head_dim] (written)
 *  lse         NULL or float [total_tokens][Hq]: natural-log sum of
 *              exp(score) over the visible keys (written)
 *
 * RBA_ERR_INVALID_ARG if a pointer is null or misaligned, a count is
 * negative, Hq % Hkv != 0, page_size is not a power of two, rel_extent < 1,
 * sm_scale is not finite and positive, or max_seqlen exceeds
 * max_pages_per_seq * page_size.  RBA_ERR_UNSUPPORTED for a head_dim or
 * page_size outside the ranges above, or (bf16) for one pool page of all KV
 * heads, Hkv * page_size * head_dim * 2 bytes, above 4 GiB - 1, for
 * max_pages_per_seq * page_size of 2^29 keys or more, or (bf16) for 32 bias
 * rows of one head, (31 * Hq + 1) * rel_extent elements, of 2 GiB or more.
 * total_tokens == 0 or num_seqs == 0 is a no-op returning RBA_OK.
 */
rba_status rba_prefill(const void *q, const int32_t *cu_seqlens,
                       int32_t total_tokens, int32_t max_seqlen,
                       const rba_kv_cache *kv, const rba_page_table *pt,
                       const void *bias, const rba_attn_params *params,
                       void *out, float *lse, hipStream_t stream);

/*
 * Prefill with the bias formed on the fly from its projection instead of
 * read from a [T][Hq][R] tensor:
 *   bias[t,h,d] = sum_k rel_r[t,h,k] * W[k,d],   d = 0 .. R-1,
 * the product the TensorRT-LLM PR #17062 page's review comment on
 * _build_rel_logits materialises per layer (r [T, heads, d_rel] times
 * rel_logits_proj [d_rel, rel_extent]); everything else as rba_prefill.
 * The products are accumulated in fp32 from the bf16 inputs and rounded
 * to bf16 before they join the score (the page's fp32 tensor, emitted in
 * bf16 as its review suggests), the clamped bucket d = R-1 of distances at
 * or beyond R-1 included: the result is that of rba_prefill given the bf16
 * bias tensor the product would materialise.
 *
 *  rel_r    bf16 [total_tokens][Hq][d_rel], 16-byte aligned
 *  w_rel_t  bf16 [rel_extent][d_rel]: W transposed (distance-major),
 *           16-byte aligned; a weight, laid out once
 *  d_rel    16 or 32 (the pages leave it open)
 *
 * bf16 pools only.  Errors as rba_prefill, plus RBA_ERR_INVALID_ARG for
 * d_rel <= 0 and RBA_ERR_UNSUPPORTED for an fp32 pool or another d_rel.
 */
rba_status rba_prefill_fused(const void *q, const int32_t *cu_seqlens,
                             int32_t total_tokens, int32_t max_seqlen,
                             const rba_kv_cache *kv, const rba_page_table *pt,
                             const void *rel_r, const void *w_rel_t,
                             int32_t d_rel, const rba_attn_params *params,
                             void *out, float *lse, hipStream_t stream);

/*
 * Number of key-range partitions rba_decode will use for these arguments
 * (num_splits == 0 picks one from the host bound max_seq_len; otherwise the
 * requested count, capped at 256).  Returns 0 on invalid arguments.
 */
int32_t rba_decode_num_splits(const rba_kv_cache *kv, const rba_page_table *pt,
                              int32_t max_seq_len,
                              const rba_attn_params *params,
                              int32_t num_splits);

/*
 * Bytes of device workspace rba_decode needs for these arguments (0 when it
 * runs without partitions).  Returns 0 on invalid arguments as well.
 *
 * The arguments are those of the decode call itself (the pool and page
 * table, max_seq_len and the layer parameters), not only (num_seqs, Hq,
 * head_dim, num_splits): with num_splits == 0 the partition count is
 * planned from max_seq_len, the page size and the window, and the workspace
 * also holds the largest-first order of the (sequence, partition) items.
 */
size_t rba_decode_workspace_size(const rba_kv_cache *kv,
                                 const rba_page_table *pt, int32_t max_seq_len,
                                 const rba_attn_params *params,
                                 int32_t num_splits);

/*
 * Single-token decode: one query per sequence at position seq_lens[b] - 1,
 * attending the seq_lens[b] keys in the pool (its own key included).  The
 * score is the one of rba_prefill (TensorRT-LLM PR #17062 page, Description,
 * Architecture list); the key count per sequence comes from the cache, as in
 * the TensorRT-LLM PR #17860 page's commit moving the model onto the
 * framework's hooks (the KV lengths are the cached token counts), and keys
 * are read through the positional page table of that page's commit that
 * borrows the framework page table.  With
 * more than one partition the visible key range of each sequence is cut into
 * page-aligned partitions, each partition's normalised partial output and
 * log-sum-exp go to the workspace, and a second kernel merges them with
 * weights exp(lse_j - max_j lse_j).  A one-work-group kernel launched first
 * orders the (sequence, partition) pairs largest first from seq_lens on the
 * device, into the workspace, so that the grid hands out the longest
 * partitions first; the order changes no result.
 *
 *  q           [num_seqs][Hq][head_dim]
 *  max_seq_len host bound on max_b seq_lens[b] (sizes the grid)
 *  bias        [num_seqs][Hq][rel_extent]: the bias row of each query
 *  num_splits  0 = automatic, else the partition count (capped at 256)
 *  workspace   device memory of rba_decode_workspace_size() bytes, 256-byte
 *              aligned (may be NULL when that size is 0); contents on entry
 *              are ignored
 *  out         [num_seqs][Hq][head_dim] (written)
 *  lse         NULL or float [num_seqs][Hq] (written): natural-log sum of
 *              exp(score) over the visible keys, the quantity the split-K
 *              merge combines; callers that merge further (e.g. partial
 *              results from several devices) need it
 *
 * Errors as for rba_prefill, plus RBA_ERR_WORKSPACE.  A sequence with
 * seq_lens[b] == 0 gets a zero output row and lse = -inf.
 */
rba_status rba_decode(const void *q, const rba_kv_cache *kv,
                      const rba_page_table *pt, int32_t max_seq_len,
                      const void *bias, const rba_attn_params *params,
                      int32_t num_splits, void *workspace,
                      size_t workspace_bytes, void *out, float *lse,
                      hipStream_t stream);

/* Largest workspace rba_decode_noalloc can use: 64 MiB per GPU. */
#define RBA_DECODE_SCRATCH_BYTES (64u << 20)

/*
 * rba_decode for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the
 * same computation, kernels and results as rba_decode, with the workspace
 * taken from a static device array of RBA_DECODE_SCRATCH_BYTES that every
 * GPU the library runs on holds until the process ends.  The call allocates
 * and frees nothing; its first call on a device looks up that device's
 * array (work must be enqueued on a stream of the current device).
 *
 * Every call on one GPU shares that GPU's array, so calls that may overlap
 * on one GPU (different streams, or different host threads) race: order
 * them.  Nothing in the array needs to start at zero (every byte read in a
 * call is written earlier in the same call), so the previous call's
 * contents are harmless.
 *
 * Arguments and errors as rba_decode without the workspace; a call whose
 * workspace (rba_decode_workspace_size) would exceed RBA_DECODE_SCRATCH_BYTES
 * returns RBA_ERR_WORKSPACE before anything is enqueued (fewer partitions,
 * or rba_decode with a caller workspace, fit such a call).
 */
rba_status rba_decode_noalloc(const void *q, const rba_kv_cache *kv,
                              const rba_page_table *pt, int32_t max_seq_len,
                              const void *bias, const rba_attn_params *params,
                              int32_t num_splits, void *out, float *lse,
                              hipStream_t stream);

/*
 * Decode of q_len new tokens per sequence at once (q_len 1..16), the pass
 * that verifies the drafted tokens of a multi-token-prediction step (the
 * vLLM PR #48768 "Add Inkling multi-depth MTP support [5/N]" page: the
 * target model checks every depth's drafts in one forward pass).  Sequence
 * b holds n_b = seq_lens[b] keys, the keys of its q_len new tokens included
 * (a value below q_len is read as q_len); token b*q_len + i sits at position
 * n_b - q_len + i and attends the keys before it as in rba_prefill over a
 * history.  The result equals that prefill's; the work is split as in
 * rba_decode: page-aligned partitions of the keys any of the sequence's
 * queries sees, one pass that writes each partition's normalised partial
 * output and log-sum-exp, and the merge.  Each K/V tile is loaded once for
 * all the sequence's tokens of up to 16 / q_len query heads.
 *
 *  q           [num_seqs * q_len][Hq][head_dim], sequence b's tokens at rows
 *              b*q_len .. b*q_len + q_len - 1
 *  q_len       tokens per sequence, 1 .. 16 (1 is rba_decode)
 *  bias        [num_seqs * q_len][Hq][rel_extent]: each token's own row
 *  out         [num_seqs * q_len][Hq][head_dim] (written)
 *  lse         NULL or float [num_seqs * q_len][Hq] (written)
 *  workspace   rba_decode_multi_workspace_size() bytes, 256-byte aligned
 *              (NULL when that is 0); contents on entry are ignored
 *
 * Errors as rba_decode; RBA_ERR_UNSUPPORTED for q_len > 16, and for fp32
 * pools with q_len > 1 (rba_prefill over a history computes those).
 */
rba_status rba_decode_multi(const void *q, int32_t q_len, const rba_kv_cache *kv,
                            const rba_page_table *pt, int32_t max_seq_len,
                            const void *bias, const rba_attn_params *params,
                            int32_t num_splits, void *workspace,
                            size_t workspace_bytes, void *out, float *lse,
                            hipStream_t stream);

/* Partition count and workspace bytes of rba_decode_multi (0 on invalid
 * arguments), as rba_decode_num_splits / rba_decode_workspace_size. */
int32_t rba_decode_multi_num_splits(int32_t q_len, const rba_kv_cache *kv,
                                    const rba_page_table *pt, int32_t max_seq_len,
                                    const rba_attn_params *params, int32_t num_splits);
size_t rba_decode_multi_workspace_size(int32_t q_len, const rba_kv_cache *kv,
                                       const rba_page_table *pt, int32_t max_seq_len,
                                       const rba_attn_params *params, int32_t num_splits);

/*
 * Append: write the keys and values of new tokens into their pool pages, so
 * that a following rba_prefill or rba_decode reads them.  Sequence b holds
 * n_b = pt->seq_lens[b] keys after the call, and its L_b new tokens
 * (cu_new[b] .. cu_new[b+1]-1) are its last L_b positions: new token i goes
 * to position n_b - L_b + i, pool page
 * block_table[b * max_pages_per_seq + pos / page_size], slot
 * pos % page_size (the positional page table of the TensorRT-LLM PR #17860
 * page, the commit that borrows the framework page table).  Nothing else of
 * the pools is written.
 *
 *  k_new, v_new  [total_new][num_kv_heads][head_dim], the pool dtype,
 *                16-byte aligned
 *  cu_new        device int32 [num_seqs + 1], non-decreasing, cu[0] = 0,
 *                cu[num_seqs] = total_new
 *  pt->seq_lens  device, required; n_b >= L_b.  A position past
 *                max_pages_per_seq * page_size, or a table entry outside
 *                [0, num_pages), leaves that token's rows unwritten.
 *
 * The call reads no device data on the host and allocates nothing, so it
 * can be captured in a HIP graph together with the decode that follows.
 * RBA_ERR_INVALID_ARG for a null or misaligned pointer, a negative count,
 * a page_size that is not a power of two; RBA_ERR_UNSUPPORTED for a
 * head_dim or page_size outside the ranges of rba_prefill.  total_new == 0
 * or num_seqs == 0 is a no-op returning RBA_OK.
 */
rba_status rba_kv_append(const void *k_new, const void *v_new, const int32_t *cu_new,
                         int32_t total_new, const rba_kv_cache *kv,
                         const rba_page_table *pt, hipStream_t stream);

/*
 * The reverse of rba_kv_append: reads the K and V rows of given positions
 * back out of the pool pages.  Row i of sequence b (cu_rows[b] <= i <
 * cu_rows[b+1], L_b = cu_rows[b+1] - cu_rows[b] rows) is position
 * n_b - L_b + (i - cu_rows[b]) with n_b = pt->seq_lens[b], read from pool
 * page block_table[b * max_pages_per_seq + pos / page_size], slot
 * pos % page_size: the slots rba_kv_append writes for the same arguments
 * (the positional page table of the TensorRT-LLM PR #17860 page).  With
 * cu_rows the prefix sums of seq_lens it de-pages every sequence whole, into
 * the logical [sum n_b][num_kv_heads][head_dim] layout: a check of the
 * page-table addressing, and an export path for a cache.
 *
 *  k_out, v_out  [total_rows][num_kv_heads][head_dim], the pool dtype,
 *                16-byte aligned, written
 *  cu_rows       device int32 [num_seqs + 1], non-decreasing, cu[0] = 0,
 *                cu[num_seqs] = total_rows
 *  pt->seq_lens  device, required; n_b >= L_b.  A position past
 *                max_pages_per_seq * page_size, or a table entry outside
 *                [0, num_pages), leaves that row of k_out and v_out
 *                unwritten.
 *
 * Nothing is allocated and no device data is read on the host.  Errors as
 * for rba_kv_append; total_rows == 0 or num_seqs == 0 is a no-op returning
 * RBA_OK.
 */
rba_status rba_kv_gather(void *k_out, void *v_out, const int32_t *cu_rows, int32_t total_rows,
                         const rba_kv_cache *kv, const rba_page_table *pt, hipStream_t stream);

/*
 * Debug check of a page table against the calls that will read it: counts,
 * on the device, the table entries a call could reach that do not name a
 * pool page.  For sequence b holding n_b = seq_lens[b] keys, a call with up
 * to max_new new tokens per sequence reads key positions lo_b .. n_b - 1,
 * with lo_b = 0 on a full-causal layer (window <= 0) and
 * max(0, n_b - max_new - window + 1) on a windowed one (rba_decode: max_new
 * 1), i.e. entries lo_b / page_size .. (n_b - 1) / page_size.  An entry is
 * bad if its index is at or past max_pages_per_seq or its page id is outside
 * [0, num_pages) (the positional table of the TensorRT-LLM PR #17860 page).
 * The attention and append kernels do not check the pages they read (a bad
 * reachable entry is a broken caller contract); this call is how a caller
 * checks a table in a debug run, without trapping the device.
 *
 *  pt           seq_lens and block_table required (device); a negative n_b
 *               counts as no keys
 *  max_new      >= 1
 *  bad_entries  device int32[1], written with the count; the call clears
 *               it on the stream first (no memset), so it needs no zeroing
 *
 * Nothing is allocated and no device data is read on the host, so the call
 * can be captured in a HIP graph.  RBA_ERR_INVALID_ARG for a null pointer, a
 * negative count, max_new < 1 or a page_size that is not a power of two.
 */
rba_status rba_check_page_table(const rba_page_table *pt, int32_t window, int32_t max_new,
                                int32_t *bad_entries, hipStream_t stream);

/*
 * Pages per sequence of a window-only pool for a layer with the given
 * window: a call that appends or queries at most max_new positions of a
 * sequence reads keys from at most window + max_new - 1 consecutive
 * positions, which span at most ceil((window + max_new - 1) / page_size) + 1
 * pages.  A pool that gives each sequence a ring of that many pages, with
 * block_table entry j = ring[j % ring_pages] (entries stay positional),
 * holds every key the kernels read for that layer: its memory is
 * O(window + max_new) per sequence instead of O(sequence length) (the
 * window-sized cache the vLLM PR #48768 page notes for its MLX port).
 * Returns 0 for window <= 0 (a full-causal layer needs every page), a page
 * size that is not a power of two, or max_new < 1.  Host only.
 */
int32_t rba_window_ring_pages(int32_t window, int32_t page_size, int32_t max_new);

/*
 * The positional block table of a window-only pool (rba_window_ring_pages):
 * block_table[b][j] = rings[b][j % ring_pages] for j < max_pages_per_seq.
 * HOST memory: rings int32 [num_seqs][ring_pages], block_table int32
 * [num_seqs][max_pages_per_seq] (written; the caller copies it to the
 * device).  The table is caller metadata built once per sequence; no kernel
 * is involved.  RBA_ERR_INVALID_ARG for a negative count, ring_pages < 1 or a
 * null pointer with a non-empty table.
 */
rba_status rba_ring_block_table(const int32_t *rings, int32_t num_seqs, int32_t ring_pages,
                                int32_t max_pages_per_seq, int32_t *block_table);

/* Static, human-readable name of a status code. */
const char *rba_status_string(rba_status status);

#ifdef __cplusplus
}
#endif

#endif /* RBA_H */
