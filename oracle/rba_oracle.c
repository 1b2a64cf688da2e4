/*
 * rba_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow, obviously-correct CPU reference for paged attention with a
 * learned relative-position bias.  Only tests/, the smoke check and the
 * cpu_baseline leg of bench.py may load this library; the product path never
 * does.  It shares no code, header, table or helper with the HIP library.
 *
 * What is computed (one query row at a time, in fp64, on the inputs exactly
 * as stored -- bf16 and fp32 widen to double without rounding):
 *
 *   score[s] = sm_scale * <q[t,h,:], k[s,g,:]> + bias[t,h,min(t-s, R-1)]
 *                                       if s <= t and (W <= 0 or t-s < W)
 *   score[s] = -inf                     otherwise
 *   p[s]     = exp(score[s] - max score),  l = sum p,
 *   out[t,h] = sum_s p[s] v[s,g,:] / l,    lse[t,h] = max score + ln l
 *
 * Sources (TensorRT-LLM PR #17062 "Support Inkling-NVFP4 model", and
 * TensorRT-LLM PR #17860 "Inkling attn backend cleanup fake registry"):
 *  - the bias is added before the softmax and is indexed by
 *    (query token, head, relative distance): PR #17062, Description,
 *    "Architecture" list, first item;
 *  - local layers attend a causal sliding window, global layers are full
 *    causal (window_left = -1): PR #17062 "Architecture", second item, and the
 *    PR #17860 commit that tests the sm_scale / rel_extent / window_left
 *    hand-off;
 *  - the bias tensor is [T, heads, rel_extent], one row per query token and
 *    head, rel_extent = 1024 on a global layer: PR #17062 review comment on
 *    _build_rel_logits; it is projected per query token, not a per-head bucket
 *    table: PR #17860, the commit that moves four hand-rolled pieces onto the
 *    framework's existing hooks, item 2;
 *  - query head h reads KV head h / (Hq / Hkv), Hq divisible by Hkv:
 *    PR #17860 commit that makes both Triton entry points assert it;
 *  - distances past the last bucket share bucket R-1 (clamp) and the bias is
 *    added to the already-scaled q.k: the plainest reading of "rel_extent"
 *    together with the per-distance indexing above.
 *
 * The reference reads K and V from logical (un-paged) tensors, token-major,
 * so it never touches a page table.
 *
 * Parity of every function here is pinned by the CPU tests in tests/
 * (brute force, closed forms, invariants, library special cases).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_F32 0
#define ORC_BF16 1
#define ORC_F64 2 /* bias rows formed here (rba_oracle_prefill_projected) */

/* Widen element i of a tensor stored as fp32 or bf16 to double (exact). */
static double elem(const void *base, int dtype, int64_t i) {
  if (dtype == ORC_F64) return ((const double *)base)[i];
  if (dtype == ORC_F32) return (double)((const float *)base)[i];
  uint32_t bits = (uint32_t)((const uint16_t *)base)[i] << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

/*
 * One output row.  t is the query position inside its sequence, n_keys the
 * number of keys held for the sequence (keys 0 .. n_keys-1).  q_row, bias_row
 * are element offsets of the query vector and of the bias row; kv0 is the
 * element offset of key 0 / head 0 in the logical K and V tensors, whose row
 * stride is Hkv*D.  scores is scratch of n_keys doubles.
 */
static void attend_row(int dtype, const void *q, int64_t q_row, const void *k,
                       const void *v, int64_t kv0, int Hkv, int D, int g,
                       int64_t t, int64_t n_keys, const void *bias,
                       int bias_dtype, int64_t bias_row, int R, int W,
                       double sm_scale, double *scores, double *out,
                       double *lse) {
  const int64_t kv_stride = (int64_t)Hkv * D;
  double m = -INFINITY;
  for (int64_t s = 0; s < n_keys; ++s) {
    int visible = (s <= t) && (W <= 0 || t - s < W);
    if (!visible) {
      scores[s] = -INFINITY;
      continue;
    }
    double dot = 0.0;
    for (int i = 0; i < D; ++i)
      dot += elem(q, dtype, q_row + i) *
             elem(k, dtype, kv0 + s * kv_stride + (int64_t)g * D + i);
    int64_t d = t - s;
    if (d > R - 1) d = R - 1;
    scores[s] = sm_scale * dot + elem(bias, bias_dtype, bias_row + d);
    if (scores[s] > m) m = scores[s];
  }
  for (int i = 0; i < D; ++i) out[i] = 0.0;
  if (m == -INFINITY) { /* no visible key: defined as a zero row */
    if (lse) *lse = -INFINITY;
    return;
  }
  double l = 0.0;
  for (int64_t s = 0; s < n_keys; ++s) {
    if (scores[s] == -INFINITY) continue;
    double p = exp(scores[s] - m);
    l += p;
    for (int i = 0; i < D; ++i)
      out[i] += p * elem(v, dtype, kv0 + s * kv_stride + (int64_t)g * D + i);
  }
  for (int i = 0; i < D; ++i) out[i] /= l;
  if (lse) *lse = m + log(l);
}

static int set_threads(int num_threads) {
#ifdef _OPENMP
  if (num_threads > 0) omp_set_num_threads(num_threads);
  return omp_get_max_threads();
#else
  (void)num_threads;
  return 1;
#endif
}

/*
 * Prefill: every sequence b holds tokens cu_seqlens[b] .. cu_seqlens[b+1]-1,
 * each token is a query at position t = token - cu_seqlens[b] and also the key
 * at that position.  q [T,Hq,D], k/v [T,Hkv,D], bias [T,Hq,R].
 * rows: optional list of n_rows (token, head) pairs; NULL means all T*Hq rows
 * in (token, head) order.  out [n_rows, D] fp64, lse [n_rows] fp64 (nullable).
 * Returns the number of threads used, or -1 on a bad argument.
 */
int rba_oracle_prefill(int dtype, const void *q, const void *k, const void *v,
                       const void *bias, const int64_t *cu_seqlens,
                       int num_seqs, int Hq, int Hkv, int D, int R, int W,
                       double sm_scale, const int64_t *rows, int64_t n_rows,
                       double *out, double *lse, int num_threads) {
  if (Hkv <= 0 || Hq % Hkv != 0 || D <= 0 || R < 1 || num_seqs < 0) return -1;
  const int G = Hq / Hkv;
  const int64_t T = cu_seqlens[num_seqs];
  int64_t max_len = 0;
  for (int b = 0; b < num_seqs; ++b)
    if (cu_seqlens[b + 1] - cu_seqlens[b] > max_len)
      max_len = cu_seqlens[b + 1] - cu_seqlens[b];
  if (!rows) n_rows = T * Hq;
  int used = set_threads(num_threads);
  int bad = 0;
#pragma omp parallel
  {
    double *scores = (double *)malloc(sizeof(double) * (size_t)(max_len + 1));
#pragma omp for schedule(dynamic, 4)
    for (int64_t r = 0; r < n_rows; ++r) {
      int64_t tok = rows ? rows[2 * r] : r / Hq;
      int h = rows ? (int)rows[2 * r + 1] : (int)(r % Hq);
      if (tok < 0 || tok >= T || h < 0 || h >= Hq) {
#pragma omp atomic write
        bad = 1;
        continue;
      }
      int b = 0;
      while (cu_seqlens[b + 1] <= tok) ++b;
      int64_t start = cu_seqlens[b];
      int64_t len = cu_seqlens[b + 1] - start;
      attend_row(dtype, q, (tok * Hq + h) * (int64_t)D, k, v,
                 start * (int64_t)Hkv * D, Hkv, D, h / G, tok - start, len,
                 bias, dtype, (tok * Hq + h) * (int64_t)R, R, W, sm_scale, scores,
                 out + r * (int64_t)D, lse ? lse + r : NULL);
    }
    free(scores);
  }
  return bad ? -1 : used;
}

/*
 * Decode: one query per sequence, at position n_b - 1, where n_b is the number
 * of keys held for sequence b (the current token's key included).
 * q [B,Hq,D]; k/v hold the keys of all B sequences back to back, sequence b at
 * rows cu_kv[b] .. cu_kv[b+1]-1 of a [sum n_b, Hkv, D] tensor; bias [B,Hq,R].
 * rows: optional (sequence, head) pairs; NULL means all B*Hq rows.
 */
int rba_oracle_decode(int dtype, const void *q, const void *k, const void *v,
                      const void *bias, const int64_t *cu_kv, int num_seqs,
                      int Hq, int Hkv, int D, int R, int W, double sm_scale,
                      const int64_t *rows, int64_t n_rows, double *out,
                      double *lse, int num_threads) {
  if (Hkv <= 0 || Hq % Hkv != 0 || D <= 0 || R < 1 || num_seqs < 0) return -1;
  const int G = Hq / Hkv;
  int64_t max_len = 0;
  for (int b = 0; b < num_seqs; ++b)
    if (cu_kv[b + 1] - cu_kv[b] > max_len) max_len = cu_kv[b + 1] - cu_kv[b];
  if (!rows) n_rows = (int64_t)num_seqs * Hq;
  int used = set_threads(num_threads);
  int bad = 0;
#pragma omp parallel
  {
    double *scores = (double *)malloc(sizeof(double) * (size_t)(max_len + 1));
#pragma omp for schedule(dynamic, 1)
    for (int64_t r = 0; r < n_rows; ++r) {
      int64_t b = rows ? rows[2 * r] : r / Hq;
      int h = rows ? (int)rows[2 * r + 1] : (int)(r % Hq);
      if (b < 0 || b >= num_seqs || h < 0 || h >= Hq) {
#pragma omp atomic write
        bad = 1;
        continue;
      }
      int64_t n = cu_kv[b + 1] - cu_kv[b];
      attend_row(dtype, q, (b * Hq + h) * (int64_t)D, k, v,
                 cu_kv[b] * (int64_t)Hkv * D, Hkv, D, h / G, n - 1, n, bias,
                 dtype, (b * Hq + h) * (int64_t)R, R, W, sm_scale, scores,
                 out + r * (int64_t)D, lse ? lse + r : NULL);
    }
    free(scores);
  }
  return bad ? -1 : used;
}

/*
 * Prefill over a cached history (chunked prefill; several new tokens of a
 * decode step).  Sequence b holds n_b keys, rows cu_kv[b] .. cu_kv[b+1]-1 of
 * the logical K and V tensors [sum n_b, Hkv, D], the keys of this call's
 * tokens included.  Its L_b = cu_q[b+1] - cu_q[b] query tokens are the last
 * L_b positions: query token cu_q[b] + i sits at position n_b - L_b + i and
 * sees the keys the definition above gives for that position.
 * q [sum L_b, Hq, D], bias [sum L_b, Hq, R] (one row per query token).
 * rows: optional (query token, head) pairs; NULL means all rows.
 * Returns -1 on a bad argument, including some L_b > n_b.
 */
int rba_oracle_prefill_history(int dtype, const void *q, const void *k,
                               const void *v, const void *bias,
                               const int64_t *cu_q, const int64_t *cu_kv,
                               int num_seqs, int Hq, int Hkv, int D, int R,
                               int W, double sm_scale, const int64_t *rows,
                               int64_t n_rows, double *out, double *lse,
                               int num_threads) {
  if (Hkv <= 0 || Hq % Hkv != 0 || D <= 0 || R < 1 || num_seqs < 0) return -1;
  const int G = Hq / Hkv;
  const int64_t T = cu_q[num_seqs];
  int64_t max_keys = 0;
  for (int b = 0; b < num_seqs; ++b) {
    const int64_t L = cu_q[b + 1] - cu_q[b], n = cu_kv[b + 1] - cu_kv[b];
    if (L < 0 || n < L) return -1;
    if (n > max_keys) max_keys = n;
  }
  if (!rows) n_rows = T * Hq;
  int used = set_threads(num_threads);
  int bad = 0;
#pragma omp parallel
  {
    double *scores = (double *)malloc(sizeof(double) * (size_t)(max_keys + 1));
#pragma omp for schedule(dynamic, 4)
    for (int64_t r = 0; r < n_rows; ++r) {
      int64_t tok = rows ? rows[2 * r] : r / Hq;
      int h = rows ? (int)rows[2 * r + 1] : (int)(r % Hq);
      if (tok < 0 || tok >= T || h < 0 || h >= Hq) {
#pragma omp atomic write
        bad = 1;
        continue;
      }
      int b = 0;
      while (cu_q[b + 1] <= tok) ++b;
      const int64_t n = cu_kv[b + 1] - cu_kv[b];
      const int64_t L = cu_q[b + 1] - cu_q[b];
      const int64_t pos = n - L + (tok - cu_q[b]);
      attend_row(dtype, q, (tok * Hq + h) * (int64_t)D, k, v,
                 cu_kv[b] * (int64_t)Hkv * D, Hkv, D, h / G, pos, n, bias,
                 dtype, (tok * Hq + h) * (int64_t)R, R, W, sm_scale, scores,
                 out + r * (int64_t)D, lse ? lse + r : NULL);
    }
    free(scores);
  }
  return bad ? -1 : used;
}

/*
 * Round a double to the nearest value of the given storage type, ties to
 * even: fp32 by the C conversion (round-to-nearest-even), bf16 (8 significant
 * bits, 8 exponent bits like fp32) directly from the double, so there is no
 * double rounding through fp32.
 */
static double round_to_dtype(double x, int dtype) {
  if (dtype == ORC_F32) return (double)(float)x;
  if (dtype != ORC_BF16 || x == 0.0 || !isfinite(x)) return x;
  int e;
  frexp(x, &e);                        /* x = m * 2^e, 0.5 <= |m| < 1 */
  if (e < -125) e = -125;              /* bf16 subnormals: fixed spacing 2^-133 */
  const double ulp = ldexp(1.0, e - 8);
  const double r = nearbyint(x / ulp) * ulp;   /* default mode: ties to even */
  return fabs(r) > 0x1.fep127 ? copysign(INFINITY, r) : r;
}

/*
 * Prefill with the bias given by its projection instead of a tensor:
 *
 *   bias[t,h,d] = round(sum_k r[t,h,k] * w[k,d]),   d = 0 .. R-1,
 *
 * r [sum L_b, Hq, d_rel] one row per query token, w [d_rel, R]: the product
 * the TensorRT-LLM PR #17062 page's review comment on _build_rel_logits forms
 * (r of shape [T, heads, d_rel] times rel_logits_proj [d_rel, rel_extent],
 * giving the [T, heads, rel_extent] bias, which that comment suggests
 * emitting in bf16).  The bias is the tensor that product materialises in the
 * layer's dtype (the dtype of q, as for the streamed bias): each entry is
 * formed here in fp64 from the stored r and w and rounded once to that dtype,
 * ties to even; then the row is attended exactly as rba_oracle_prefill_history
 * does with its bias tensor.  cu_kv NULL: no history, every sequence's keys
 * are its query tokens (rba_oracle_prefill).  rows, out, lse and the return
 * value as there.
 */
int rba_oracle_prefill_projected(int dtype, const void *q, const void *k,
                                 const void *v, const void *r, const void *w,
                                 const int64_t *cu_q, const int64_t *cu_kv,
                                 int num_seqs, int Hq, int Hkv, int D, int R,
                                 int W, int d_rel, double sm_scale,
                                 const int64_t *rows, int64_t n_rows,
                                 double *out, double *lse, int num_threads) {
  if (Hkv <= 0 || Hq % Hkv != 0 || D <= 0 || R < 1 || d_rel < 1 || num_seqs < 0)
    return -1;
  const int G = Hq / Hkv;
  const int64_t T = cu_q[num_seqs];
  int64_t max_keys = 0;
  for (int b = 0; b < num_seqs; ++b) {
    const int64_t L = cu_q[b + 1] - cu_q[b];
    const int64_t n = cu_kv ? cu_kv[b + 1] - cu_kv[b] : L;
    if (L < 0 || n < L) return -1;
    if (n > max_keys) max_keys = n;
  }
  if (!rows) n_rows = T * Hq;
  int used = set_threads(num_threads);
  int bad = 0;
#pragma omp parallel
  {
    double *scores = (double *)malloc(sizeof(double) * (size_t)(max_keys + 1));
    double *brow = (double *)malloc(sizeof(double) * (size_t)R);
#pragma omp for schedule(dynamic, 4)
    for (int64_t i = 0; i < n_rows; ++i) {
      int64_t tok = rows ? rows[2 * i] : i / Hq;
      int h = rows ? (int)rows[2 * i + 1] : (int)(i % Hq);
      if (tok < 0 || tok >= T || h < 0 || h >= Hq) {
#pragma omp atomic write
        bad = 1;
        continue;
      }
      int b = 0;
      while (cu_q[b + 1] <= tok) ++b;
      const int64_t L = cu_q[b + 1] - cu_q[b];
      const int64_t n = cu_kv ? cu_kv[b + 1] - cu_kv[b] : L;
      const int64_t kv_first = cu_kv ? cu_kv[b] : cu_q[b];
      const int64_t pos = n - L + (tok - cu_q[b]);
      const int64_t r_row = (tok * Hq + h) * (int64_t)d_rel;
      for (int d = 0; d < R; ++d) {
        double acc = 0.0;
        for (int kk = 0; kk < d_rel; ++kk)
          acc += elem(r, dtype, r_row + kk) * elem(w, dtype, (int64_t)kk * R + d);
        brow[d] = round_to_dtype(acc, dtype);
      }
      attend_row(dtype, q, (tok * Hq + h) * (int64_t)D, k, v,
                 kv_first * (int64_t)Hkv * D, Hkv, D, h / G, pos, n, brow,
                 ORC_F64, 0, R, W, sm_scale, scores, out + i * (int64_t)D,
                 lse ? lse + i : NULL);
    }
    free(brow);
    free(scores);
  }
  return bad ? -1 : used;
}
