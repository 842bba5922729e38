/*
 * The library used from plain C through include/tp.h alone: the Megatron MLP
 * pair (column-parallel W1, row-parallel W2, fixed-order sum of the partials)
 * with one tp_mlp call, then the same three steps as separate calls
 * (tp_col_linear, tp_row_linear, tp_reduce_partials). Device memory comes from
 * the HIP runtime's C API. The inputs are small integers, so every product and
 * sum is exact in fp32, and the program checks both results element by element
 * against the same product computed here in double precision.
 * Exit status 0: both results exact; 1: a mismatch; 2: a call failed.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "tp.h"

enum { M = 40, D = 64, F = 96, NSHARD = 4 };

static uint16_t bf16_bits(int v) {
  const float f = (float)v;
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  return (uint16_t)(u >> 16); /* exact: small integers have 8 significant bits at most */
}

static uint32_t lcg = 12345u;
static int small_int(void) {
  lcg = lcg * 1664525u + 1013904223u;
  return (int)((lcg >> 16) % 5u) - 2; /* -2 .. 2 */
}

#define HIP_OK(call)                                                    \
  do {                                                                  \
    if ((call) != hipSuccess) {                                         \
      fprintf(stderr, "HIP call failed: %s (line %d)\n", #call, __LINE__); \
      return 2;                                                         \
    }                                                                   \
  } while (0)

#define TP_OK_OR_FAIL(call)                                                          \
  do {                                                                               \
    const tp_status st_ = (call);                                                    \
    if (st_ != TP_OK) {                                                              \
      fprintf(stderr, "%s returned %s (line %d)\n", #call, tp_status_string(st_), __LINE__); \
      return 2;                                                                      \
    }                                                                                \
  } while (0)

static tp_matrix mat(void* ptr, int32_t dtype, int64_t rows, int64_t cols, int64_t ld, int64_t shard_stride) {
  tp_matrix m;
  memset(&m, 0, sizeof m);
  m.ptr = ptr;
  m.dtype = dtype;
  m.rows = rows;
  m.cols = cols;
  m.ld = ld;
  m.shard_stride = shard_stride;
  return m;
}

static int compare(const float* got, const double* ref, const char* what) {
  int bad = 0;
  for (int i = 0; i < M * D; ++i)
    if ((double)got[i] != ref[i]) {
      if (bad < 5) fprintf(stderr, "%s: element %d is %g, expected %g\n", what, i, got[i], ref[i]);
      ++bad;
    }
  return bad;
}

int main(void) {
  static int x[M][D], w1[D][F], w2[F][D];
  static uint16_t xb[M * D], w1b[D * F], w2b[F * D];
  static double h[M][F], ref[M * D];
  static float got[M * D];
  for (int i = 0; i < M; ++i)
    for (int k = 0; k < D; ++k) xb[i * D + k] = bf16_bits(x[i][k] = small_int());
  for (int k = 0; k < D; ++k)
    for (int f = 0; f < F; ++f) w1b[k * F + f] = bf16_bits(w1[k][f] = small_int());
  for (int f = 0; f < F; ++f)
    for (int c = 0; c < D; ++c) w2b[f * D + c] = bf16_bits(w2[f][c] = small_int());
  for (int i = 0; i < M; ++i)
    for (int f = 0; f < F; ++f) {
      double s = 0;
      for (int k = 0; k < D; ++k) s += (double)x[i][k] * w1[k][f];
      h[i][f] = s;
    }
  for (int i = 0; i < M; ++i)
    for (int c = 0; c < D; ++c) {
      double s = 0;
      for (int f = 0; f < F; ++f) s += h[i][f] * w2[f][c];
      ref[i * D + c] = s;
    }

  void *dx, *dw1, *dw2, *dy, *dh, *dp, *ws;
  HIP_OK(hipMalloc(&dx, sizeof xb));
  HIP_OK(hipMalloc(&dw1, sizeof w1b));
  HIP_OK(hipMalloc(&dw2, sizeof w2b));
  HIP_OK(hipMalloc(&dy, sizeof got));
  HIP_OK(hipMalloc(&dh, (size_t)M * F * 2));
  HIP_OK(hipMalloc(&dp, (size_t)NSHARD * M * D * 4));
  HIP_OK(hipMemcpy(dx, xb, sizeof xb, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dw1, w1b, sizeof w1b, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dw2, w2b, sizeof w2b, hipMemcpyHostToDevice));

  const tp_matrix X = mat(dx, TP_BF16, M, D, D, 0);
  const tp_matrix W1 = mat(dw1, TP_BF16, D, F, F, 0);
  const tp_matrix W2 = mat(dw2, TP_BF16, F, D, D, 0);
  const tp_matrix Y = mat(dy, TP_F32, M, D, D, 0);

  /* one call: query the workspace size, then run */
  size_t ws_bytes = 0;
  TP_OK_OR_FAIL(tp_mlp(&X, &W1, &W2, NSHARD, 0, NSHARD, TP_ACT_NONE, NULL, &ws_bytes, &Y, NULL));
  HIP_OK(hipMalloc(&ws, ws_bytes > 0 ? ws_bytes : 1));
  TP_OK_OR_FAIL(tp_mlp(&X, &W1, &W2, NSHARD, 0, NSHARD, TP_ACT_NONE, ws, &ws_bytes, &Y, NULL));
  HIP_OK(hipDeviceSynchronize());
  HIP_OK(hipMemcpy(got, dy, sizeof got, hipMemcpyDeviceToHost));
  int bad = compare(got, ref, "tp_mlp");

  /* the same three steps as separate calls: H stays column-partitioned, P holds one partial per shard */
  HIP_OK(hipMemset(dy, 0, sizeof got));
  const tp_matrix H = mat(dh, TP_BF16, M, F, F, 0);
  const tp_matrix P = mat(dp, TP_F32, M, D, D, (int64_t)M * D);
  TP_OK_OR_FAIL(tp_col_linear(&X, &W1, NSHARD, 0, NSHARD, TP_ACT_NONE, &H, NULL));
  TP_OK_OR_FAIL(tp_row_linear(&H, &W2, NSHARD, 0, NSHARD, &P, NULL));
  TP_OK_OR_FAIL(tp_reduce_partials(&P, NSHARD, TP_SPLIT_ROWS, &Y, NULL));
  HIP_OK(hipDeviceSynchronize());
  HIP_OK(hipMemcpy(got, dy, sizeof got, hipMemcpyDeviceToHost));
  bad += compare(got, ref, "three calls");

  hipFree(dx); hipFree(dw1); hipFree(dw2); hipFree(dy); hipFree(dh); hipFree(dp); hipFree(ws);
  printf("c interface: tp_mlp and the three-call form on [%d, %d] x [%d, %d] x [%d, %d], N = %d: %s\n", M, D, D, F,
         F, D, NSHARD, bad ? "MISMATCH" : "exact");
  return bad ? 1 : 0;
}
