/*
 * A plain C caller of libsolattn (no Python, no PyTorch): device buffers from
 * the HIP runtime, q, k, v filled with bf16 values from an integer hash plus
 * a smooth function of the token position, the pooling pass and the sparse
 * forward through the C ABI at tau = 8 and tau = +inf, and a few rows of the
 * tau = +inf output checked against dense softmax attention computed here in
 * double precision (tau = +inf keeps every key block).
 *
 *   sol_attn_example [N]      (default 4096; B = 1, H = 2, d = 128)
 *
 * Exit status 0 when every call succeeds and the checked rows agree within
 * 2e-2; the kept-block statistics of the tau = 8 call are printed.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "sol_attn.h"

#define CHECK_HIP(x)                                                           \
  do {                                                                         \
    hipError_t e_ = (x);                                                       \
    if (e_ != hipSuccess) {                                                    \
      fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));           \
      return 1;                                                                \
    }                                                                          \
  } while (0)
#define CHECK_SOL(x)                                                           \
  do {                                                                         \
    int r_ = (x);                                                              \
    if (r_ != SOL_OK) {                                                        \
      fprintf(stderr, "%s failed: %s\n", #x, sol_attn_strerror(r_));           \
      return 1;                                                                \
    }                                                                          \
  } while (0)

static uint16_t to_bf16(float f) {  /* round to nearest even */
  uint32_t u;
  memcpy(&u, &f, 4);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
static double from_bf16(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}
static float hash_unit(uint64_t x) {  /* splitmix64 -> [-1, 1) */
  x += 0x9e3779b97f4a7c15ull;
  x = (x ^ (x >> 30)) * 0xbf58476d1ce4e5b9ull;
  x = (x ^ (x >> 27)) * 0x94d049bb133111ebull;
  x ^= x >> 31;
  return (float)((double)(x >> 11) * (1.0 / 4503599627370496.0) - 1.0);
}

int main(int argc, char** argv) {
  const int B = 1, H = 2, d = 128, Bq = 64, Bk = 64;
  const int N = argc > 1 ? atoi(argv[1]) : 4096;
  if (N <= 0) return 2;
  const size_t n = (size_t)B * H * N * d;
  uint16_t* hq = malloc(n * 2);
  uint16_t* hk = malloc(n * 2);
  uint16_t* hv = malloc(n * 2);
  float* hout = malloc(n * 4);
  if (!hq || !hk || !hv || !hout) return 1;
  for (size_t i = 0; i < n; ++i) {
    const size_t t = (i / d) % (size_t)N;
    const int c = (int)(i % d);
    const float pos = 2.f * sinf(0.01f * (float)t * (float)(1 + c % 7));  /* neighbouring tokens alike */
    hq[i] = to_bf16(hash_unit(3 * i) + pos);
    hk[i] = to_bf16(hash_unit(3 * i + 1) + pos);
    hv[i] = to_bf16(hash_unit(3 * i + 2));
  }
  const int Nk = (N + Bk - 1) / Bk;
  void *q, *k, *v, *out, *kpool, *vmean, *ws;
  sol_attn_stats* stats;
  const size_t ws_bytes = sol_attn_workspace_bytes(B, H, N, d, Bq, Bk);
  if (ws_bytes == 0) return 1;
  CHECK_HIP(hipMalloc(&q, n * 2));
  CHECK_HIP(hipMalloc(&k, n * 2));
  CHECK_HIP(hipMalloc(&v, n * 2));
  CHECK_HIP(hipMalloc(&out, n * 4));
  CHECK_HIP(hipMalloc(&kpool, (size_t)B * H * Nk * d * 4));
  CHECK_HIP(hipMalloc(&vmean, (size_t)B * H * Nk * d * 4));
  CHECK_HIP(hipMalloc(&ws, ws_bytes));
  CHECK_HIP(hipMalloc((void**)&stats, sizeof(sol_attn_stats)));
  CHECK_HIP(hipMemcpy(q, hq, n * 2, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(k, hk, n * 2, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(v, hv, n * 2, hipMemcpyHostToDevice));

  /* tau = 8: the sparse path, with statistics */
  CHECK_SOL(sol_attn_forward(q, k, v, out, B, H, N, d, Bq, Bk, 8.0f, 0u, stats, kpool, vmean, ws, ws_bytes, NULL));
  sol_attn_stats st;
  CHECK_HIP(hipMemcpy(&st, stats, sizeof st, hipMemcpyDeviceToHost));
  printf("tau=8: kept %llu of %llu key blocks (%.2f%%), per query block %u..%u\n", st.kept_blocks, st.total_blocks,
         100.0 * (double)st.kept_blocks / (double)st.total_blocks, st.min_kept, st.max_kept);
  if (st.total_blocks != (unsigned long long)B * H * Nk * Nk || st.min_kept < 1) return 1;

  /* tau = +inf: dense attention, checked on a few rows of each head */
  CHECK_SOL(sol_attn_forward(q, k, v, out, B, H, N, d, Bq, Bk, INFINITY, 0u, NULL, kpool, vmean, ws, ws_bytes, NULL));
  CHECK_HIP(hipMemcpy(hout, out, n * 4, hipMemcpyDeviceToHost));
  double* logit = malloc((size_t)N * sizeof(double));
  if (!logit) return 1;
  const int rows[4] = {0, N / 3, N / 2 + 1, N - 1};
  double worst = 0.0;
  int finite = 1;
  for (int h = 0; h < H; ++h)
    for (int ri = 0; ri < 4; ++ri) {
      const size_t base = (size_t)h * N * d;
      const int r = rows[ri];
      double m = -INFINITY;
      for (int t = 0; t < N; ++t) {
        double s = 0.0;
        for (int c = 0; c < d; ++c) s += from_bf16(hq[base + (size_t)r * d + c]) * from_bf16(hk[base + (size_t)t * d + c]);
        logit[t] = s / sqrt((double)d);
        if (logit[t] > m) m = logit[t];
      }
      double den = 0.0;
      for (int t = 0; t < N; ++t) den += exp(logit[t] - m);
      for (int c = 0; c < d; ++c) {
        double num = 0.0;
        for (int t = 0; t < N; ++t) num += exp(logit[t] - m) * from_bf16(hv[base + (size_t)t * d + c]);
        const double err = fabs(num / den - (double)hout[base + (size_t)r * d + c]);
        if (!isfinite(err)) finite = 0;
        else if (err > worst) worst = err;
      }
    }
  printf("tau=inf: max abs error %.3e on %d checked rows%s\n", worst, 4 * H, finite ? "" : " (non-finite values)");
  CHECK_HIP(hipFree(q));
  CHECK_HIP(hipFree(k));
  CHECK_HIP(hipFree(v));
  CHECK_HIP(hipFree(out));
  CHECK_HIP(hipFree(kpool));
  CHECK_HIP(hipFree(vmean));
  CHECK_HIP(hipFree(ws));
  CHECK_HIP(hipFree(stats));
  free(hq);
  free(hk);
  free(hv);
  free(hout);
  free(logit);
  return finite && worst <= 2e-2 ? 0 : 1;
}
