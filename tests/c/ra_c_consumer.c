/*
 * A plain C consumer of the library's C ABI (include/ra.h): no Python, no C++.
 *
 * It runs one rank's causal zigzag share with Q = 0 through ra_rank_forward. With
 * every score zero the softmax weights of a row are uniform over its allowed keys, so
 * lse = ln(number of allowed keys) and out = the mean of their V rows ("Ring Attention
 * and Ulysses shard a sequence two different ways, ...", section "Ring Attention:
 * point-to-point rotation, and an online softmax that never sees the whole row at
 * once": the fold equals full-row softmax). The host recomputes both from the zigzag
 * positions ("What do you do about long sequences and sparse models?", section "What
 * breaks the load balance?") and compares every row. It also checks that an invalid
 * call returns an error code and leaves a message. Prints "ok" and exits 0 on success.
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "ra.h"

#define CHECK_HIP(x)                                                        \
  do {                                                                      \
    hipError_t e_ = (x);                                                    \
    if (e_ != hipSuccess) {                                                 \
      fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));        \
      return 2;                                                             \
    }                                                                       \
  } while (0)

static uint16_t to_bf16(float f) {   /* round to nearest even */
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

/* Global position of row t of owner i's share: zigzag chunks i and 2c-1-i of m tokens. */
static int position(int i, int t, int m, int c) { return t < m ? i * m + t : (2 * c - 1 - i) * m + (t - m); }

int main(void) {
  const int B = 1, hq = 4, hkv = 2, d = 128, c = 3, rank = 1, n = 200, m = n / 2;
  const size_t nq_el = (size_t)B * hq * n * d, kv_el = (size_t)c * B * hkv * n * d;
  uint16_t* hv = malloc(kv_el * 2);
  uint16_t* hout = malloc(nq_el * 2);
  float* hlse = malloc((size_t)B * hq * n * 4);
  float* vf = malloc(kv_el * 4);
  if (!hv || !hout || !hlse || !vf) return 2;
  srand(7);
  for (size_t i = 0; i < kv_el; ++i) {
    hv[i] = to_bf16((float)rand() / RAND_MAX - 0.5f);
    vf[i] = from_bf16(hv[i]);
  }
  void *q, *k, *v, *out;
  float* lse;
  CHECK_HIP(hipMalloc(&q, nq_el * 2));
  CHECK_HIP(hipMalloc(&k, kv_el * 2));
  CHECK_HIP(hipMalloc(&v, kv_el * 2));
  CHECK_HIP(hipMalloc(&out, nq_el * 2));
  CHECK_HIP(hipMalloc((void**)&lse, (size_t)B * hq * n * 4));
  CHECK_HIP(hipMemset(q, 0, nq_el * 2));
  CHECK_HIP(hipMemset(k, 0x3f, kv_el * 2));   /* any finite keys: Q = 0 ignores them */
  CHECK_HIP(hipMemcpy(v, hv, kv_el * 2, hipMemcpyHostToDevice));

  int rc = ra_rank_forward(q, k, v, out, lse, B, hq, hkv, n, n, d, c, rank, 1, 1, 0, c, RA_BF16, NULL);
  if (rc != RA_OK) {
    fprintf(stderr, "ra_rank_forward: %d %s\n", rc, ra_last_error());
    return 1;
  }
  CHECK_HIP(hipDeviceSynchronize());
  CHECK_HIP(hipMemcpy(hout, out, nq_el * 2, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(hlse, lse, (size_t)B * hq * n * 4, hipMemcpyDeviceToHost));

  double max_out = 0, max_lse = 0;
  for (int h = 0; h < hq; ++h) {
    const int g = h / (hq / hkv);
    for (int t = 0; t < n; ++t) {
      const int pq = position(rank, t, m, c);
      double sum[128] = {0};
      long count = 0;
      for (int j = 0; j < c; ++j)
        for (int r = 0; r < n; ++r) {
          if (position(j, r, m, c) > pq) continue;
          const float* vr = vf + (((size_t)j * B * hkv + g) * n + r) * d;
          for (int x = 0; x < d; ++x) sum[x] += vr[x];
          ++count;
        }
      const double dl = fabs(hlse[h * n + t] - log((double)count));
      if (dl > max_lse) max_lse = dl;
      for (int x = 0; x < d; ++x) {
        const double o = from_bf16(hout[((size_t)h * n + t) * d + x]);
        const double e = fabs(o - sum[x] / count);
        if (e > max_out) max_out = e;
      }
    }
  }
  printf("Q = 0 share: max |out - prefix mean| %.3g, max |lse - ln count| %.3g\n", max_out, max_lse);

  /* an invalid call: rank outside [0, c) */
  const int bad = ra_rank_forward(q, k, v, out, lse, B, hq, hkv, n, n, d, c, c, 1, 1, 0, c, RA_BF16, NULL);
  const int bad_ok = bad == RA_ERR_ARG && strlen(ra_last_error()) > 0;

  hipFree(q);
  hipFree(k);
  hipFree(v);
  hipFree(out);
  hipFree(lse);
  free(hv);
  free(hout);
  free(hlse);
  free(vf);
  if (max_out > 2e-2 || max_lse > 1e-3 || !bad_ok) {
    printf("FAILED (invalid call returned %d)\n", bad);
    return 1;
  }
  printf("ok\n");
  return 0;
}
