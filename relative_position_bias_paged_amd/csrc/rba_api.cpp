// rba_api.cpp -- host entry points of librba (declared in include/rba.h).
//
// Every call validates its host-side arguments, sizes the launch from host
// scalars only (never reading device memory, so calls can be enqueued from
// any context, including graph capture), and enqueues the kernels on the
// caller's stream.  Nothing here allocates, frees or synchronises.
#include "rba.h"

#include <climits>
#include <cmath>
#include <cstdint>
#include <mutex>

#include "rba_internal.h"

#define RBA_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

// Waves per bf16 prefill work-group on local (windowed) and global layers.
// Every K/V tile a work-group loads serves 32 (head, query) rows per wave.
#ifndef RBA_PREFILL_WAVES_LOCAL
#define RBA_PREFILL_WAVES_LOCAL 4
#endif
#ifndef RBA_PREFILL_WAVES_GLOBAL
#define RBA_PREFILL_WAVES_GLOBAL 8
#endif
constexpr int kF32Rows = 4;          // queries (one wave each) per fp32 prefill work-group
constexpr int kMaxSplits = 256;
constexpr int kAutoChunkPages = 64;  // automatic partitions hold about this many pages
constexpr long long kAutoMinWaves = 2048;

bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

int ilog2(int x) {
  int l = 0;
  while ((1 << l) < x) ++l;
  return l;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

rba_status check_layer(const rba_kv_cache *kv, const rba_page_table *pt,
                       const rba_attn_params *p) {
  if (kv == nullptr || pt == nullptr || p == nullptr) return RBA_ERR_INVALID_ARG;
  if (kv->dtype != RBA_BF16 && kv->dtype != RBA_F32) return RBA_ERR_INVALID_ARG;
  if (kv->num_kv_heads <= 0 || p->num_q_heads <= 0) return RBA_ERR_INVALID_ARG;
  if (p->num_q_heads % kv->num_kv_heads != 0) return RBA_ERR_INVALID_ARG;
  if (kv->head_dim <= 0) return RBA_ERR_INVALID_ARG;
  if (!is_pow2(pt->page_size)) return RBA_ERR_INVALID_ARG;
  if (p->rel_extent < 1) return RBA_ERR_INVALID_ARG;
  if (!(p->sm_scale > 0.0f) || !std::isfinite(p->sm_scale)) return RBA_ERR_INVALID_ARG;
  if (pt->num_seqs < 0 || pt->max_pages_per_seq < 0 || pt->num_pages < 0)
    return RBA_ERR_INVALID_ARG;
  if (kv->head_dim != 64 && kv->head_dim != 128) return RBA_ERR_UNSUPPORTED;
  if (pt->page_size < 16 || pt->page_size > 1024) return RBA_ERR_UNSUPPORTED;
  return RBA_OK;
}

bool pool_ok(const rba_kv_cache *kv, const rba_page_table *pt) {
  return kv->k_pool != nullptr && kv->v_pool != nullptr && pt->block_table != nullptr &&
         aligned16(kv->k_pool) && aligned16(kv->v_pool) && pt->num_pages > 0 &&
         pt->max_pages_per_seq > 0;
}

// Upper bound on the pages the queries of one sequence touch: with q_len
// queries at positions n - q_len .. n - 1, the visible keys
// [max(0, n - q_len - window + 1), n) span at most ceil(visible / P) pages,
// plus one when a window start falls inside a page.
int decode_pages_max(const rba_page_table *pt, int max_seq_len, int window, int q_len = 1) {
  const long long P = pt->page_size;
  long long visible = max_seq_len;
  if (window > 0 && (long long)window + q_len - 1 < visible) visible = (long long)window + q_len - 1;
  long long pages = (visible + P - 1) / P + (window > 0 ? 1 : 0);
  if (pages < 1) pages = 1;
  const long long cap = (max_seq_len + P - 1) / P;
  if (pages > cap && cap > 0) pages = cap;
  return (int)pages;
}

struct SplitPlan {
  int splits;
  int chunk_pages;
};

// Query heads per decode wave: 4 for single-token decode; with q_len > 1,
// as many as fit the 16 matrix rows of a wave with their q_len tokens each.
int decode_heads_per_wave(int G, int q_len) {
  if (q_len <= 1) return 4;
  const int fit = 16 / q_len;
  return fit < G ? fit : G;
}

SplitPlan plan_splits(const rba_kv_cache *kv, const rba_page_table *pt, int max_seq_len,
                      const rba_attn_params *p, int num_splits, int q_len = 1) {
  if (kv->dtype == RBA_F32) return {1, 1 << 30};
  const int pm = decode_pages_max(pt, max_seq_len, p->window, q_len);
  int s;
  if (num_splits > 0) {
    s = num_splits;
  } else {
    s = (pm + kAutoChunkPages - 1) / kAutoChunkPages;
    const int G = p->num_q_heads / kv->num_kv_heads;
    const int hpw = decode_heads_per_wave(G, q_len);
    const long long base = (long long)pt->num_seqs * kv->num_kv_heads * ((G + hpw - 1) / hpw);
    if (base > 0 && base * s < kAutoMinWaves) s = (int)((kAutoMinWaves + base - 1) / base);
  }
  if (s > kMaxSplits) s = kMaxSplits;
  if (s > pm) s = pm;
  if (s < 1) s = 1;
  const int chunk = (pm + s - 1) / s;
  s = (pm + chunk - 1) / chunk;  // drop partitions that could never hold a page
  return {s, chunk};
}

// Decode workspace with S > 1 partitions, each part starting 256-byte aligned:
// partial outputs fp32 [B][Hq][S][D], their LSE fp32 [B][Hq][S], and the
// largest-first plan of the B*S (sequence, partition) items, two int32 each.
struct WorkspaceLayout {
  size_t lse_off, plan_off, bytes;
};

size_t pad256(size_t x) { return (x + 255) & ~(size_t)255; }

WorkspaceLayout workspace_layout(const rba_kv_cache *kv, const rba_page_table *pt,
                                 const rba_attn_params *p, int splits, int q_len = 1) {
  if (splits <= 1) return {0, 0, 0};
  const size_t rows = (size_t)pt->num_seqs * q_len * p->num_q_heads;
  const size_t lse_off = pad256(rows * splits * kv->head_dim * sizeof(float));
  const size_t plan_off = pad256(lse_off + rows * splits * sizeof(float));
  return {lse_off, plan_off, plan_off + (size_t)pt->num_seqs * splits * 2 * sizeof(int32_t)};
}

size_t workspace_bytes_for(const rba_kv_cache *kv, const rba_page_table *pt,
                           const rba_attn_params *p, int splits, int q_len = 1) {
  return workspace_layout(kv, pt, p, splits, q_len).bytes;
}

}  // namespace

RBA_EXPORT const char *rba_status_string(rba_status status) {
  switch (status) {
    case RBA_OK: return "RBA_OK";
    case RBA_ERR_INVALID_ARG: return "RBA_ERR_INVALID_ARG";
    case RBA_ERR_UNSUPPORTED: return "RBA_ERR_UNSUPPORTED";
    case RBA_ERR_WORKSPACE: return "RBA_ERR_WORKSPACE";
    case RBA_ERR_HIP: return "RBA_ERR_HIP";
  }
  return "RBA_UNKNOWN_STATUS";
}

namespace {

// Shared by rba_prefill (bias tensor given) and rba_prefill_fused (bias
// formed from rel_r and w_rel_t, d_rel > 0).
rba_status prefill_impl(const void *q, const int32_t *cu_seqlens, int32_t total_tokens,
                        int32_t max_seqlen, const rba_kv_cache *kv, const rba_page_table *pt,
                        const void *bias, const void *rel_r, const void *w_rel_t, int32_t d_rel,
                        const rba_attn_params *params, void *out, float *lse, hipStream_t stream) {
  const bool fused = d_rel != 0;
  rba_status st = check_layer(kv, pt, params);
  if (st != RBA_OK) return st;
  if (total_tokens < 0 || max_seqlen < 0 || d_rel < 0) return RBA_ERR_INVALID_ARG;
  if (fused && (kv->dtype != RBA_BF16 || (d_rel != 16 && d_rel != 32))) return RBA_ERR_UNSUPPORTED;
  if (total_tokens == 0 || pt->num_seqs == 0 || max_seqlen == 0) return RBA_OK;
  if (q == nullptr || cu_seqlens == nullptr || out == nullptr) return RBA_ERR_INVALID_ARG;
  if (fused ? (rel_r == nullptr || w_rel_t == nullptr || !aligned16(rel_r) || !aligned16(w_rel_t))
            : (bias == nullptr || !aligned16(bias)))
    return RBA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(out) || !pool_ok(kv, pt)) return RBA_ERR_INVALID_ARG;
  if (lse != nullptr && (reinterpret_cast<uintptr_t>(lse) & 3u) != 0) return RBA_ERR_INVALID_ARG;
  if ((long long)max_seqlen > (long long)pt->max_pages_per_seq * pt->page_size)
    return RBA_ERR_INVALID_ARG;
  // key positions stay below 2^29, and a wave's 32 bias rows (Hq * rel_extent
  // elements apart) span under 2 GiB: the bias stage's 32-bit offsets rely on both
  if ((long long)pt->max_pages_per_seq * pt->page_size >= (1LL << 29)) return RBA_ERR_UNSUPPORTED;
  if (!fused && kv->dtype == RBA_BF16 &&
      (31LL * params->num_q_heads * params->rel_extent + params->rel_extent + 256) * 2 > INT_MAX)
    return RBA_ERR_UNSUPPORTED;

  rba::PrefillArgs a{};
  a.q = q;
  a.cu_seqlens = cu_seqlens;
  a.k_pool = kv->k_pool;
  a.v_pool = kv->v_pool;
  a.block_table = pt->block_table;
  a.seq_lens = pt->seq_lens;       // null: the queries are all the keys
  a.bias = fused ? nullptr : bias;
  a.rel_r = fused ? rel_r : nullptr;
  a.w_rel_t = fused ? w_rel_t : nullptr;
  a.d_rel = d_rel;
  a.out = out;
  a.lse = lse;
  a.num_seqs = pt->num_seqs;
  a.Hq = params->num_q_heads;
  a.Hkv = kv->num_kv_heads;
  a.G = a.Hq / a.Hkv;
  a.max_pages = pt->max_pages_per_seq;
  a.page_size = pt->page_size;
  a.log2_page = ilog2(pt->page_size);
  a.window = params->window > 0 ? params->window : 0;
  a.R = params->rel_extent;
  a.total_tokens = total_tokens;
  a.sm_scale = params->sm_scale;

  hipError_t err;
  if (kv->dtype == RBA_BF16) {
    // Query heads of one KV head share a work-group (and its K/V tiles):
    // the largest of 8, 4, 2, 1 that divides both G and the wave count.
    // The fused variant takes the local wave count only where G is even (its
    // 4-wave work-groups need two heads or more), else 8 waves.
    a.waves = (a.window > 0 && (!fused || a.G % 2 == 0)) ? RBA_PREFILL_WAVES_LOCAL
                                                          : RBA_PREFILL_WAVES_GLOBAL;
    a.hpw = 1;
    while (a.hpw * 2 <= a.waves && a.G % (a.hpw * 2) == 0) a.hpw *= 2;
    const int qm = 32 * (a.waves / a.hpw);       // queries per head per work-group
    a.num_qtiles = (max_seqlen + qm - 1) / qm;
    const long long blocks = (long long)a.num_seqs * a.Hkv * (a.G / a.hpw) * a.num_qtiles;
    if (blocks > 0x7fffffffLL) return RBA_ERR_UNSUPPORTED;
    // the kernel forms page offsets as (32-bit page id) x (32-bit page bytes)
    if ((long long)a.Hkv * a.page_size * kv->head_dim * 2 > 0xffffffffLL) return RBA_ERR_UNSUPPORTED;
    a.num_blocks = (int32_t)blocks;
    err = fused ? rba::launch_prefill_fused(a, kv->head_dim, stream)
                : rba::launch_prefill_bf16(a, kv->head_dim, stream);
  } else {
    a.num_qtiles = (max_seqlen + kF32Rows - 1) / kF32Rows;
    if (a.Hq > 65535 || a.num_seqs > 65535) return RBA_ERR_UNSUPPORTED;
    a.num_blocks = a.num_qtiles;
    err = rba::launch_prefill_f32(a, kv->head_dim, stream);
  }
  return err == hipSuccess ? RBA_OK : RBA_ERR_HIP;
}

}  // namespace

RBA_EXPORT rba_status rba_prefill(const void *q, const int32_t *cu_seqlens, int32_t total_tokens,
                                  int32_t max_seqlen, const rba_kv_cache *kv,
                                  const rba_page_table *pt, const void *bias,
                                  const rba_attn_params *params, void *out, float *lse,
                                  hipStream_t stream) {
  return prefill_impl(q, cu_seqlens, total_tokens, max_seqlen, kv, pt, bias, nullptr, nullptr, 0,
                      params, out, lse, stream);
}

RBA_EXPORT rba_status rba_prefill_fused(const void *q, const int32_t *cu_seqlens,
                                        int32_t total_tokens, int32_t max_seqlen,
                                        const rba_kv_cache *kv, const rba_page_table *pt,
                                        const void *rel_r, const void *w_rel_t, int32_t d_rel,
                                        const rba_attn_params *params, void *out, float *lse,
                                        hipStream_t stream) {
  if (d_rel <= 0) return RBA_ERR_INVALID_ARG;
  return prefill_impl(q, cu_seqlens, total_tokens, max_seqlen, kv, pt, nullptr, rel_r, w_rel_t,
                      d_rel, params, out, lse, stream);
}

// Validation and launch shared by rba_kv_append and rba_kv_gather: the same
// rows <-> pool slots mapping, copied in either direction.
static rba_status kv_rows_copy(void *k_rows, void *v_rows, const int32_t *cu, int32_t total,
                               const rba_kv_cache *kv, const rba_page_table *pt, bool gather,
                               hipStream_t stream) {
  if (kv == nullptr || pt == nullptr) return RBA_ERR_INVALID_ARG;
  if (kv->dtype != RBA_BF16 && kv->dtype != RBA_F32) return RBA_ERR_INVALID_ARG;
  if (kv->num_kv_heads <= 0 || kv->head_dim <= 0) return RBA_ERR_INVALID_ARG;
  if (!is_pow2(pt->page_size)) return RBA_ERR_INVALID_ARG;
  if (total < 0 || pt->num_seqs < 0 || pt->max_pages_per_seq < 0 || pt->num_pages < 0)
    return RBA_ERR_INVALID_ARG;
  if (kv->head_dim != 64 && kv->head_dim != 128) return RBA_ERR_UNSUPPORTED;
  if (pt->page_size < 16 || pt->page_size > 1024) return RBA_ERR_UNSUPPORTED;
  if (total == 0 || pt->num_seqs == 0) return RBA_OK;
  if (k_rows == nullptr || v_rows == nullptr || cu == nullptr || pt->seq_lens == nullptr ||
      !aligned16(k_rows) || !aligned16(v_rows) || !pool_ok(kv, pt))
    return RBA_ERR_INVALID_ARG;
  rba::AppendArgs a{};
  a.k_rows = k_rows;
  a.v_rows = v_rows;
  a.cu_new = cu;
  a.seq_lens = pt->seq_lens;
  a.block_table = pt->block_table;
  a.k_pool = const_cast<void *>(kv->k_pool);
  a.v_pool = const_cast<void *>(kv->v_pool);
  a.total_new = total;
  a.num_seqs = pt->num_seqs;
  a.Hkv = kv->num_kv_heads;
  a.max_pages = pt->max_pages_per_seq;
  a.page_size = pt->page_size;
  a.log2_page = ilog2(pt->page_size);
  a.num_pages = pt->num_pages;
  a.row_bytes = kv->head_dim * (kv->dtype == RBA_BF16 ? 2 : 4);
  return rba::launch_kv_append(a, gather, stream) == hipSuccess ? RBA_OK : RBA_ERR_HIP;
}

RBA_EXPORT rba_status rba_kv_append(const void *k_new, const void *v_new, const int32_t *cu_new,
                                    int32_t total_new, const rba_kv_cache *kv,
                                    const rba_page_table *pt, hipStream_t stream) {
  return kv_rows_copy(const_cast<void *>(k_new), const_cast<void *>(v_new), cu_new, total_new, kv,
                      pt, false, stream);
}

RBA_EXPORT rba_status rba_kv_gather(void *k_out, void *v_out, const int32_t *cu_rows,
                                    int32_t total_rows, const rba_kv_cache *kv,
                                    const rba_page_table *pt, hipStream_t stream) {
  return kv_rows_copy(k_out, v_out, cu_rows, total_rows, kv, pt, true, stream);
}

RBA_EXPORT rba_status rba_check_page_table(const rba_page_table *pt, int32_t window,
                                           int32_t max_new, int32_t *bad_entries,
                                           hipStream_t stream) {
  if (pt == nullptr || bad_entries == nullptr || max_new < 1) return RBA_ERR_INVALID_ARG;
  if (!is_pow2(pt->page_size) || pt->num_seqs < 0 || pt->max_pages_per_seq < 0 ||
      pt->num_pages < 0)
    return RBA_ERR_INVALID_ARG;
  if (pt->num_seqs > 0 && (pt->seq_lens == nullptr ||
                           (pt->max_pages_per_seq > 0 && pt->block_table == nullptr)))
    return RBA_ERR_INVALID_ARG;
  rba::PageCheckArgs a{};
  a.block_table = pt->block_table;
  a.seq_lens = pt->seq_lens;
  a.bad = bad_entries;
  a.num_seqs = pt->num_seqs;
  a.max_pages = pt->max_pages_per_seq;
  a.log2_page = ilog2(pt->page_size);
  a.num_pages = pt->num_pages;
  a.window = window > 0 ? window : 0;
  a.max_new = max_new;
  return rba::launch_page_check(a, stream) == hipSuccess ? RBA_OK : RBA_ERR_HIP;
}

RBA_EXPORT int32_t rba_window_ring_pages(int32_t window, int32_t page_size, int32_t max_new) {
  if (window <= 0 || max_new < 1 || !is_pow2(page_size)) return 0;
  const long long span = (long long)window + max_new - 1;      // consecutive key positions read
  const long long pages = (span + page_size - 1) / page_size + 1;
  return pages > 0x7fffffffLL ? 0 : (int32_t)pages;
}

RBA_EXPORT rba_status rba_ring_block_table(const int32_t *rings, int32_t num_seqs,
                                           int32_t ring_pages, int32_t max_pages_per_seq,
                                           int32_t *block_table) {
  if (num_seqs < 0 || ring_pages < 1 || max_pages_per_seq < 0) return RBA_ERR_INVALID_ARG;
  if (num_seqs == 0 || max_pages_per_seq == 0) return RBA_OK;
  if (rings == nullptr || block_table == nullptr) return RBA_ERR_INVALID_ARG;
  for (int32_t b = 0; b < num_seqs; ++b)
    for (int32_t j = 0; j < max_pages_per_seq; ++j)
      block_table[(size_t)b * max_pages_per_seq + j] = rings[(size_t)b * ring_pages + j % ring_pages];
  return RBA_OK;
}

RBA_EXPORT int32_t rba_decode_num_splits(const rba_kv_cache *kv, const rba_page_table *pt,
                                         int32_t max_seq_len, const rba_attn_params *params,
                                         int32_t num_splits) {
  if (check_layer(kv, pt, params) != RBA_OK || max_seq_len < 0 || num_splits < 0) return 0;
  return plan_splits(kv, pt, max_seq_len, params, num_splits).splits;
}

RBA_EXPORT size_t rba_decode_workspace_size(const rba_kv_cache *kv, const rba_page_table *pt,
                                            int32_t max_seq_len, const rba_attn_params *params,
                                            int32_t num_splits) {
  if (check_layer(kv, pt, params) != RBA_OK || max_seq_len < 0 || num_splits < 0) return 0;
  const SplitPlan sp = plan_splits(kv, pt, max_seq_len, params, num_splits);
  return workspace_bytes_for(kv, pt, params, sp.splits);
}

namespace {

// Host-side checks of a decode call.  On RBA_OK, *sp holds the partition
// plan and *need the workspace bytes it takes (0 without partitions).
rba_status decode_check(const void *q, const rba_kv_cache *kv, const rba_page_table *pt,
                        int32_t max_seq_len, const void *bias, const rba_attn_params *params,
                        int32_t num_splits, void *out, float *lse, SplitPlan *sp, size_t *need,
                        int q_len = 1) {
  rba_status st = check_layer(kv, pt, params);
  if (st != RBA_OK) return st;
  if (max_seq_len < 0 || num_splits < 0 || q_len < 1) return RBA_ERR_INVALID_ARG;
  if (q_len > 16 || (q_len > 1 && kv->dtype != RBA_BF16)) return RBA_ERR_UNSUPPORTED;
  *sp = plan_splits(kv, pt, max_seq_len, params, num_splits, q_len);
  *need = 0;
  if (pt->num_seqs == 0) return RBA_OK;
  if (q == nullptr || bias == nullptr || out == nullptr || pt->seq_lens == nullptr)
    return RBA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(bias) || !aligned16(out) || !pool_ok(kv, pt))
    return RBA_ERR_INVALID_ARG;
  if (lse != nullptr && (reinterpret_cast<uintptr_t>(lse) & 3u) != 0) return RBA_ERR_INVALID_ARG;
  if ((long long)max_seq_len > (long long)pt->max_pages_per_seq * pt->page_size)
    return RBA_ERR_INVALID_ARG;
  // every sequence holds its q_len new tokens' keys: the kernels read a
  // shorter length as q_len, which max_seq_len (and the table) must cover
  if (q_len > 1 && max_seq_len < q_len) return RBA_ERR_INVALID_ARG;
  if ((long long)pt->num_seqs * q_len * params->num_q_heads > 0x7fffffffLL) return RBA_ERR_UNSUPPORTED;
  *need = workspace_bytes_for(kv, pt, params, sp->splits, q_len);
  return RBA_OK;
}

// Enqueues a checked decode call (decode_check returned RBA_OK).
rba_status decode_launch(const void *q, const rba_kv_cache *kv, const rba_page_table *pt,
                         const void *bias, const rba_attn_params *params, const SplitPlan &sp,
                         size_t need, void *workspace, void *out, float *lse,
                         hipStream_t stream, int q_len = 1) {
  rba::DecodeArgs a{};
  a.q = q;
  a.k_pool = kv->k_pool;
  a.v_pool = kv->v_pool;
  a.block_table = pt->block_table;
  a.seq_lens = pt->seq_lens;
  a.bias = bias;
  a.out = out;
  a.lse = lse;
  a.num_seqs = pt->num_seqs;
  a.Hq = params->num_q_heads;
  a.Hkv = kv->num_kv_heads;
  a.G = a.Hq / a.Hkv;
  a.max_pages = pt->max_pages_per_seq;
  a.page_size = pt->page_size;
  a.log2_page = ilog2(pt->page_size);
  a.window = params->window > 0 ? params->window : 0;
  a.R = params->rel_extent;
  a.sm_scale = params->sm_scale;
  a.num_splits = sp.splits;
  a.chunk_pages = sp.chunk_pages;
  a.q_len = q_len;
  a.hpw = decode_heads_per_wave(a.G, q_len);
  a.head_groups = (a.G + a.hpw - 1) / a.hpw;
  if (need > 0) {
    const WorkspaceLayout wl = workspace_layout(kv, pt, params, sp.splits, q_len);
    char *base = static_cast<char *>(workspace);
    a.part_o = reinterpret_cast<float *>(base);
    a.part_lse = reinterpret_cast<float *>(base + wl.lse_off);
    if (kv->dtype == RBA_BF16) {
      a.plan = reinterpret_cast<int2 *>(base + wl.plan_off);
      a.plan_shift = 0;
      while (((sp.chunk_pages - 1) >> a.plan_shift) > 255) ++a.plan_shift;
    }
  }

  hipError_t err;
  if (kv->dtype == RBA_F32) {
    err = rba::launch_decode_f32(a, kv->head_dim, stream);
  } else {
    const long long items = (long long)a.num_seqs * a.Hkv * a.num_splits * a.head_groups;
    if (items > 0x7fffffffLL) return RBA_ERR_UNSUPPORTED;
    if (a.plan != nullptr) {
      if ((long long)a.num_seqs * a.num_splits > 0x7fffffffLL) return RBA_ERR_UNSUPPORTED;
      err = rba::launch_decode_plan(a, stream);
      if (err != hipSuccess) return RBA_ERR_HIP;
    }
    err = q_len > 1 ? rba::launch_decode_multi(a, kv->head_dim, stream)
                    : rba::launch_decode_bf16(a, kv->head_dim, stream);
    if (err == hipSuccess && sp.splits > 1) err = rba::launch_merge(a, kv->head_dim, true, stream);
  }
  return err == hipSuccess ? RBA_OK : RBA_ERR_HIP;
}

}  // namespace

// Workspace of rba_decode_noalloc: one static array per GPU, held until the
// process ends.  Host code never uses its name as an address (in host code
// it is a stand-in, not device memory): each device's address comes from
// hipGetSymbolAddress, taken once per device with that device current.
static __device__ __align__(256) unsigned char scratch[RBA_DECODE_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::once_flag scratch_once[kMaxDevices];
void *scratch_addr[kMaxDevices];
hipError_t scratch_err[kMaxDevices];

hipError_t scratch_for_current_device(void **ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(scratch_once[dev], [dev] {
    void *p = nullptr;
    scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    scratch_addr[dev] = scratch_err[dev] == hipSuccess ? p : nullptr;
  });
  *ptr = scratch_addr[dev];
  return scratch_err[dev];
}

}  // namespace

RBA_EXPORT rba_status rba_decode(const void *q, const rba_kv_cache *kv, const rba_page_table *pt,
                                 int32_t max_seq_len, const void *bias,
                                 const rba_attn_params *params, int32_t num_splits,
                                 void *workspace, size_t workspace_bytes, void *out, float *lse,
                                 hipStream_t stream) {
  SplitPlan sp;
  size_t need;
  const rba_status st =
      decode_check(q, kv, pt, max_seq_len, bias, params, num_splits, out, lse, &sp, &need);
  if (st != RBA_OK || pt->num_seqs == 0) return st;
  if (need > 0) {
    if (workspace == nullptr || workspace_bytes < need ||
        (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
      return RBA_ERR_WORKSPACE;
  }
  return decode_launch(q, kv, pt, bias, params, sp, need, workspace, out, lse, stream);
}

RBA_EXPORT rba_status rba_decode_noalloc(const void *q, const rba_kv_cache *kv,
                                         const rba_page_table *pt, int32_t max_seq_len,
                                         const void *bias, const rba_attn_params *params,
                                         int32_t num_splits, void *out, float *lse,
                                         hipStream_t stream) {
  SplitPlan sp;
  size_t need;
  const rba_status st =
      decode_check(q, kv, pt, max_seq_len, bias, params, num_splits, out, lse, &sp, &need);
  if (st != RBA_OK || pt->num_seqs == 0) return st;
  if (need > (size_t)RBA_DECODE_SCRATCH_BYTES) return RBA_ERR_WORKSPACE;
  void *ws = nullptr;
  if (need > 0 && scratch_for_current_device(&ws) != hipSuccess) return RBA_ERR_HIP;
  return decode_launch(q, kv, pt, bias, params, sp, need, ws, out, lse, stream);
}

RBA_EXPORT int32_t rba_decode_multi_num_splits(int32_t q_len, const rba_kv_cache *kv,
                                               const rba_page_table *pt, int32_t max_seq_len,
                                               const rba_attn_params *params, int32_t num_splits) {
  if (check_layer(kv, pt, params) != RBA_OK || max_seq_len < 0 || num_splits < 0 || q_len < 1 ||
      q_len > 16)
    return 0;
  return plan_splits(kv, pt, max_seq_len, params, num_splits, q_len).splits;
}

RBA_EXPORT size_t rba_decode_multi_workspace_size(int32_t q_len, const rba_kv_cache *kv,
                                                  const rba_page_table *pt, int32_t max_seq_len,
                                                  const rba_attn_params *params,
                                                  int32_t num_splits) {
  if (check_layer(kv, pt, params) != RBA_OK || max_seq_len < 0 || num_splits < 0 || q_len < 1 ||
      q_len > 16)
    return 0;
  const SplitPlan sp = plan_splits(kv, pt, max_seq_len, params, num_splits, q_len);
  return workspace_bytes_for(kv, pt, params, sp.splits, q_len);
}

RBA_EXPORT rba_status rba_decode_multi(const void *q, int32_t q_len, const rba_kv_cache *kv,
                                       const rba_page_table *pt, int32_t max_seq_len,
                                       const void *bias, const rba_attn_params *params,
                                       int32_t num_splits, void *workspace,
                                       size_t workspace_bytes, void *out, float *lse,
                                       hipStream_t stream) {
  SplitPlan sp;
  size_t need;
  const rba_status st = decode_check(q, kv, pt, max_seq_len, bias, params, num_splits, out, lse,
                                     &sp, &need, q_len);
  if (st != RBA_OK || pt->num_seqs == 0) return st;
  if (need > 0) {
    if (workspace == nullptr || workspace_bytes < need ||
        (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
      return RBA_ERR_WORKSPACE;
  }
  return decode_launch(q, kv, pt, bias, params, sp, need, workspace, out, lse, stream, q_len);
}
