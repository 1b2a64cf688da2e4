/*
 * c_abi_check.c -- TEST INFRASTRUCTURE: the C ABI used from plain C.
 *
 * Device memory comes from hipMalloc, inputs from a fixed xorshift stream;
 * no Python and no torch.  A decode (with its workspace) and a prefill over a
 * shuffled page table run through librba.so, then the CPU oracle library
 * computes the same rows from the logical (un-paged) K/V, and every output
 * element is compared to the bf16 bar (max |d| <= 2e-2, sum|d| / sum|ref|
 * <= 5e-3).  Exit status 0 when every check passes.
 *
 * Built by __graft_entry__.build() with gcc against include/rba.h, librba.so
 * and the oracle's library.
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "rba.h"

/* the oracle's entry points (oracle/rba_oracle.c; dtype 1 = bf16) */
int rba_oracle_decode(int dtype, const void *q, const void *k, const void *v, const void *bias,
                      const int64_t *cu_kv, int num_seqs, int Hq, int Hkv, int D, int R, int W,
                      double sm_scale, const int64_t *rows, int64_t n_rows, double *out,
                      double *lse, int num_threads);
int rba_oracle_prefill(int dtype, const void *q, const void *k, const void *v, const void *bias,
                       const int64_t *cu_seqlens, int num_seqs, int Hq, int Hkv, int D, int R,
                       int W, double sm_scale, const int64_t *rows, int64_t n_rows, double *out,
                       double *lse, int num_threads);

enum { B = 3, HQ = 8, HKV = 2, D = 128, P = 16, R = 64 };
static const int LENS[B] = {1, 100, 333};

#define HIP_OK(x)                                                              \
  do {                                                                         \
    hipError_t e_ = (x);                                                       \
    if (e_ != hipSuccess) {                                                    \
      fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));                  \
      exit(2);                                                                 \
    }                                                                          \
  } while (0)

static uint32_t state = 0x9e3779b9u;
static float frand(void) { /* xorshift32, uniform in [-1, 1) */
  state ^= state << 13;
  state ^= state >> 17;
  state ^= state << 5;
  return (float)((state >> 8) * (1.0 / 16777216.0)) * 2.0f - 1.0f;
}

static uint16_t to_bf16(float f) { /* round to nearest, ties to even */
  uint32_t u;
  memcpy(&u, &f, 4);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

static float from_bf16(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

static uint16_t *rand_bf16(size_t n) {
  uint16_t *p = (uint16_t *)malloc(n * 2);
  for (size_t i = 0; i < n; ++i) p[i] = to_bf16(frand());
  return p;
}

static void *to_device(const void *h, size_t bytes) {
  void *d = NULL;
  HIP_OK(hipMalloc(&d, bytes));
  HIP_OK(hipMemcpy(d, h, bytes, hipMemcpyHostToDevice));
  return d;
}

/* Compares n bf16 device results with the oracle; returns 0 when in bar. */
static int compare(const char *what, const void *d_out, const double *ref, size_t n) {
  uint16_t *g = (uint16_t *)malloc(n * 2);
  HIP_OK(hipMemcpy(g, d_out, n * 2, hipMemcpyDeviceToHost));
  double max_abs = 0, sum_d = 0, sum_r = 0;
  int finite = 1;
  for (size_t i = 0; i < n; ++i) {
    const double x = from_bf16(g[i]);
    if (!isfinite(x)) finite = 0;
    const double d = fabs(x - ref[i]);
    if (d > max_abs) max_abs = d;
    sum_d += d;
    sum_r += fabs(ref[i]);
  }
  free(g);
  const double mean_rel = sum_d / (sum_r > 0 ? sum_r : 1);
  const int ok = finite && max_abs <= 2e-2 && mean_rel <= 5e-3;
  printf("%s: max|d| %.3e  mean rel %.3e  %s\n", what, max_abs, mean_rel, ok ? "ok" : "FAIL");
  return ok ? 0 : 1;
}

int main(void) {
  int T = 0, pages_needed = 0, max_len = 0;
  for (int b = 0; b < B; ++b) {
    T += LENS[b];
    pages_needed += (LENS[b] + P - 1) / P;
    if (LENS[b] > max_len) max_len = LENS[b];
  }
  const int num_pages = pages_needed + 3;  /* 32: 7 is coprime to it */
  const int max_pages = (max_len + P - 1) / P;

  /* logical K/V [T][HKV][D], sequences back to back */
  uint16_t *k_log = rand_bf16((size_t)T * HKV * D), *v_log = rand_bf16((size_t)T * HKV * D);
  /* pools [num_pages][HKV][P][D], unused slots NaN; pages assigned by a permutation */
  const size_t pool_elems = (size_t)num_pages * HKV * P * D;
  uint16_t *k_pool = (uint16_t *)malloc(pool_elems * 2), *v_pool = (uint16_t *)malloc(pool_elems * 2);
  for (size_t i = 0; i < pool_elems; ++i) k_pool[i] = v_pool[i] = 0x7fc0; /* NaN */
  int32_t *table = (int32_t *)calloc((size_t)B * max_pages, 4);
  int32_t lens[B], cu[B + 1];
  int64_t cu64[B + 1];
  int next = 0, tok0 = 0;
  cu[0] = 0;
  cu64[0] = 0;
  for (int b = 0; b < B; ++b) {
    lens[b] = LENS[b];
    cu[b + 1] = cu[b] + LENS[b];
    cu64[b + 1] = cu[b + 1];
    for (int j = 0; j < (LENS[b] + P - 1) / P; ++j) table[b * max_pages + j] = (7 * next++ + 2) % num_pages;
    for (int s = 0; s < LENS[b]; ++s)
      for (int g = 0; g < HKV; ++g) {
        const size_t dst = (((size_t)table[b * max_pages + s / P] * HKV + g) * P + s % P) * D;
        const size_t src = ((size_t)(tok0 + s) * HKV + g) * D;
        memcpy(k_pool + dst, k_log + src, D * 2);
        memcpy(v_pool + dst, v_log + src, D * 2);
      }
    tok0 += LENS[b];
  }

  { /* the page assignment is a permutation: every page used at most once */
    int *used = (int *)calloc((size_t)num_pages, sizeof(int));
    for (int i = 0; i < B * max_pages; ++i)
      if (i % max_pages < (LENS[i / max_pages] + P - 1) / P && used[table[i]]++) {
        fprintf(stderr, "page %d assigned twice\n", table[i]);
        return 2;
      }
    free(used);
  }
  rba_kv_cache kv = {to_device(k_pool, pool_elems * 2), to_device(v_pool, pool_elems * 2), HKV, D,
                     RBA_BF16};
  rba_page_table pt = {(const int32_t *)to_device(table, (size_t)B * max_pages * 4),
                       (const int32_t *)to_device(lens, sizeof lens), B, max_pages, P, num_pages};
  const double scale = 1.0 / sqrt((double)D);
  int fails = 0;

  for (int wi = 0; wi < 2; ++wi) {
    const int W = wi == 0 ? 0 : 100;
    rba_attn_params prm = {HQ, W, R, (float)scale};
    char what[64];

    /* decode: one query per sequence at position n - 1, automatic partitions */
    uint16_t *q = rand_bf16((size_t)B * HQ * D), *bias = rand_bf16((size_t)B * HQ * R);
    void *d_q = to_device(q, (size_t)B * HQ * D * 2), *d_bias = to_device(bias, (size_t)B * HQ * R * 2);
    void *d_out = NULL, *ws = NULL;
    HIP_OK(hipMalloc(&d_out, (size_t)B * HQ * D * 2));
    const size_t ws_bytes = rba_decode_workspace_size(&kv, &pt, max_len, &prm, 0);
    if (ws_bytes) HIP_OK(hipMalloc(&ws, ws_bytes));
    rba_status st = rba_decode(d_q, &kv, &pt, max_len, d_bias, &prm, 0, ws, ws_bytes, d_out, NULL, NULL);
    HIP_OK(hipDeviceSynchronize());
    double *ref = (double *)malloc((size_t)B * HQ * D * sizeof(double));
    if (st != RBA_OK ||
        rba_oracle_decode(1, q, k_log, v_log, bias, cu64, B, HQ, HKV, D, R, W, scale, NULL, 0, ref,
                          NULL, 0) < 0) {
      printf("decode W=%d: status %s\n", W, rba_status_string(st));
      fails++;
    } else {
      snprintf(what, sizeof what, "decode W=%d", W);
      fails += compare(what, d_out, ref, (size_t)B * HQ * D);
    }
    free(ref);
    free(q);
    free(bias);
    HIP_OK(hipFree(d_q));
    HIP_OK(hipFree(d_bias));
    HIP_OK(hipFree(d_out));
    if (ws) HIP_OK(hipFree(ws));

    /* prefill: every token a query over its own sequence's keys */
    q = rand_bf16((size_t)T * HQ * D);
    bias = rand_bf16((size_t)T * HQ * R);
    d_q = to_device(q, (size_t)T * HQ * D * 2);
    d_bias = to_device(bias, (size_t)T * HQ * R * 2);
    void *d_cu = to_device(cu, sizeof cu);
    HIP_OK(hipMalloc(&d_out, (size_t)T * HQ * D * 2));
    st = rba_prefill(d_q, (const int32_t *)d_cu, T, max_len, &kv, &pt, d_bias, &prm, d_out, NULL, NULL);
    HIP_OK(hipDeviceSynchronize());
    ref = (double *)malloc((size_t)T * HQ * D * sizeof(double));
    if (st != RBA_OK ||
        rba_oracle_prefill(1, q, k_log, v_log, bias, cu64, B, HQ, HKV, D, R, W, scale, NULL, 0, ref,
                           NULL, 0) < 0) {
      printf("prefill W=%d: status %s\n", W, rba_status_string(st));
      fails++;
    } else {
      snprintf(what, sizeof what, "prefill W=%d", W);
      fails += compare(what, d_out, ref, (size_t)T * HQ * D);
    }
    free(ref);
    free(q);
    free(bias);
    HIP_OK(hipFree(d_q));
    HIP_OK(hipFree(d_bias));
    HIP_OK(hipFree(d_cu));
    HIP_OK(hipFree(d_out));
  }

  /* an argument error is reported, and nothing is launched */
  rba_attn_params bad = {HQ + 1, 0, R, (float)scale};
  const rba_status st = rba_prefill(NULL, NULL, 0, 0, &kv, &pt, NULL, &bad, NULL, NULL, NULL);
  printf("bad head count: %s\n", rba_status_string(st));
  if (st != RBA_ERR_INVALID_ARG) fails++;
  printf(fails ? "FAILED %d\n" : "all ok\n", fails);
  return fails ? 1 : 0;
}
