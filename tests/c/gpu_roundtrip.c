/* The C ABI used from plain C on the GPU, with no Python and no PyTorch:
 * device buffers from hipMalloc, one arnfp8_run (ragged 37 x 7176, P = 5,
 * residual read and written out of place) and one arn_sum_bf16 on the null
 * stream, each checked against the CPU oracle linked from oracle/; then the
 * same fused call split over 4 workgroups per row with a hipMalloc'd
 * workspace (arnfp8_run_split), against the oracle too, and its
 * allocation-free form, bitwise against the split call.  Test
 * infrastructure.  Exit status 0 = pass. */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "arnfp8.h"
#include "arnfp8_oracle.h"

enum { ROWS = 37, COLS = 7176, P = 5 };
#define N ((size_t)ROWS * COLS)

static int failures = 0;

static void fail(const char *what) {
  printf("FAIL %s\n", what);
  ++failures;
}

/* splitmix64: the inputs' random bits. */
static uint64_t rng_state = 0x1234567ull;
static uint64_t next64(void) {
  uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

/* A bf16 bit pattern with a random sign, a biased exponent in [lo, hi] and a
 * random 7-bit mantissa: finite values drawn directly in the format. */
static uint16_t random_bf16(int lo, int hi, int positive) {
  const uint64_t r = next64();
  const uint16_t sign = positive ? 0 : (uint16_t)((r >> 63) << 15);
  const uint16_t exp = (uint16_t)(lo + (int)((r >> 8) % (uint64_t)(hi - lo + 1)));
  return (uint16_t)(sign | (exp << 7) | (r & 0x7F));
}

static int ordered_fp8(uint8_t c) { return (c & 0x80) ? -(int)(c & 0x7F) : (int)(c & 0x7F); }

#define CHECK_HIP(call)                                         \
  do {                                                          \
    if ((call) != hipSuccess) {                                 \
      printf("FAIL hip call %s\n", #call);                      \
      return 2;                                                 \
    }                                                           \
  } while (0)

int main(void) {
  uint16_t *x[P], *res = malloc(2 * N), *gamma = malloc(2 * COLS);
  uint16_t *res_out = malloc(2 * N), *res_ref = malloc(2 * N);
  uint16_t *sum = malloc(2 * N), *sum_ref = malloc(2 * N);
  uint8_t *q = malloc(N), *q_ref = malloc(N);
  float *s = malloc(4 * ROWS), *s_ref = malloc(4 * ROWS);
  uint16_t *res_split = malloc(2 * N), *res_na = malloc(2 * N);
  uint8_t *q_split = malloc(N), *q_na = malloc(N);
  float *s_split = malloc(4 * ROWS), *s_na = malloc(4 * ROWS);
  for (int p = 0; p < P; ++p) {
    x[p] = malloc(2 * N);
    for (size_t i = 0; i < N; ++i) x[p][i] = random_bf16(118, 128, 0);
  }
  for (size_t i = 0; i < N; ++i) res[i] = random_bf16(120, 127, 0);
  for (int j = 0; j < COLS; ++j) gamma[j] = random_bf16(126, 127, 1);

  void *dx[P], *dres, *dres_out, *dq, *ds, *dgamma, *dsum;
  void *dres_split, *dq_split, *ds_split, *dws, *dres_na, *dq_na, *ds_na;
  for (int p = 0; p < P; ++p) {
    CHECK_HIP(hipMalloc(&dx[p], 2 * N));
    CHECK_HIP(hipMemcpy(dx[p], x[p], 2 * N, hipMemcpyHostToDevice));
  }
  CHECK_HIP(hipMalloc(&dres, 2 * N));
  CHECK_HIP(hipMalloc(&dres_out, 2 * N));
  CHECK_HIP(hipMalloc(&dq, N));
  CHECK_HIP(hipMalloc(&ds, 4 * ROWS));
  CHECK_HIP(hipMalloc(&dgamma, 2 * COLS));
  CHECK_HIP(hipMalloc(&dsum, 2 * N));
  const int64_t ws_bytes = arnfp8_split_workspace_bytes(ROWS);
  CHECK_HIP(hipMalloc(&dres_split, 2 * N));
  CHECK_HIP(hipMalloc(&dq_split, N));
  CHECK_HIP(hipMalloc(&ds_split, 4 * ROWS));
  CHECK_HIP(hipMalloc(&dws, (size_t)ws_bytes));
  CHECK_HIP(hipMemset(dws, 0, (size_t)ws_bytes));
  CHECK_HIP(hipMalloc(&dres_na, 2 * N));
  CHECK_HIP(hipMalloc(&dq_na, N));
  CHECK_HIP(hipMalloc(&ds_na, 4 * ROWS));
  CHECK_HIP(hipMemcpy(dres, res, 2 * N, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(dgamma, gamma, 2 * COLS, hipMemcpyHostToDevice));

  const void *inputs[P];
  for (int p = 0; p < P; ++p) inputs[p] = dx[p];
  int st = arnfp8_run(inputs, dres, dres_out, dq, (float *)ds, dgamma, 1e-6f, 0.0f, 1200.0f, ROWS,
                      COLS, P, NULL);
  if (st != ARNFP8_OK) fail(arnfp8_status_string(st));
  st = arn_sum_bf16(inputs, dsum, ROWS, COLS, P, NULL);
  if (st != ARNFP8_OK) fail(arnfp8_status_string(st));
  /* An error path from C: a misaligned output is refused before any launch. */
  if (arnfp8_run(inputs, dres, dres_out, (char *)dq + 8, (float *)ds, dgamma, 1e-6f, 0.0f,
                 1200.0f, ROWS, COLS, P, NULL) != ARNFP8_MISALIGNED)
    fail("misaligned output accepted");
  const arnfp8_split_opts four = {4, 0};
  st = arnfp8_run_split(inputs, dres, dres_split, dq_split, (float *)ds_split, dgamma, 1e-6f, 0.0f,
                        1200.0f, ROWS, COLS, P, dws, ws_bytes, NULL, &four);
  if (st != ARNFP8_OK) fail(arnfp8_status_string(st));
  st = arnfp8_run_split_noalloc(inputs, dres, dres_na, dq_na, (float *)ds_na, dgamma, 1e-6f, 0.0f,
                                1200.0f, ROWS, COLS, P, NULL, &four);
  if (st != ARNFP8_OK) fail(arnfp8_status_string(st));
  CHECK_HIP(hipDeviceSynchronize());
  CHECK_HIP(hipMemcpy(res_split, dres_split, 2 * N, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(q_split, dq_split, N, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(s_split, ds_split, 4 * ROWS, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(res_na, dres_na, 2 * N, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(q_na, dq_na, N, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(s_na, ds_na, 4 * ROWS, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(res_out, dres_out, 2 * N, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(q, dq, N, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(s, ds, 4 * ROWS, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(sum, dsum, 2 * N, hipMemcpyDeviceToHost));

  const uint16_t *xs[P];
  for (int p = 0; p < P; ++p) xs[p] = x[p];
  if (oracle_arnfp8(xs, P, res, res_ref, q_ref, s_ref, gamma, 1e-6f, 0.0f, 1200.0f, ROWS, COLS))
    fail("oracle_arnfp8");
  if (oracle_sum_bf16(xs, P, sum_ref, ROWS, COLS)) fail("oracle_sum_bf16");

  if (memcmp(res_out, res_ref, 2 * N) != 0) fail("residual_out differs from the oracle");
  if (memcmp(sum, sum_ref, 2 * N) != 0) fail("sum differs from the oracle");
  for (int i = 0; i < ROWS; ++i)
    if (!(fabs((double)s[i] / (double)s_ref[i] - 1.0) <= 1e-5)) {
      fail("scale differs from the oracle by more than 1e-5 relative");
      break;
    }
  size_t exact = 0;
  int worst = 0;
  for (size_t i = 0; i < N; ++i) {
    if ((q[i] & 0x7F) == 0x7F) worst = 99; /* NaN code */
    const int d = abs(ordered_fp8(q[i]) - ordered_fp8(q_ref[i]));
    if (d > worst) worst = d;
    exact += d == 0;
  }
  if (worst > 1) fail("fp8 code more than one step from the oracle (or NaN)");
  if ((double)exact / (double)N < 0.999) fail("fewer than 99.9% of fp8 codes exactly equal");

  /* The split call against the oracle, and the allocation-free call bitwise
   * against the split call. */
  if (memcmp(res_split, res_ref, 2 * N) != 0) fail("split residual_out differs from the oracle");
  for (int i = 0; i < ROWS; ++i)
    if (!(fabs((double)s_split[i] / (double)s_ref[i] - 1.0) <= 1e-5)) {
      fail("split scale differs from the oracle by more than 1e-5 relative");
      break;
    }
  size_t exact_split = 0;
  int worst_split = 0;
  for (size_t i = 0; i < N; ++i) {
    if ((q_split[i] & 0x7F) == 0x7F) worst_split = 99;
    const int d = abs(ordered_fp8(q_split[i]) - ordered_fp8(q_ref[i]));
    if (d > worst_split) worst_split = d;
    exact_split += d == 0;
  }
  if (worst_split > 1) fail("split fp8 code more than one step from the oracle (or NaN)");
  if ((double)exact_split / (double)N < 0.999) fail("split: fewer than 99.9% of codes exact");
  if (memcmp(res_na, res_split, 2 * N) != 0 || memcmp(q_na, q_split, N) != 0 ||
      memcmp(s_na, s_split, 4 * ROWS) != 0)
    fail("allocation-free split differs from the split call");

  for (int p = 0; p < P; ++p) {
    hipFree(dx[p]);
    free(x[p]);
  }
  hipFree(dres);
  hipFree(dres_out);
  hipFree(dq);
  hipFree(ds);
  hipFree(dgamma);
  hipFree(dsum);
  hipFree(dres_split);
  hipFree(dq_split);
  hipFree(ds_split);
  hipFree(dws);
  hipFree(dres_na);
  hipFree(dq_na);
  hipFree(ds_na);
  free(res_split);
  free(res_na);
  free(q_split);
  free(q_na);
  free(s_split);
  free(s_na);
  free(res);
  free(gamma);
  free(res_out);
  free(res_ref);
  free(sum);
  free(sum_ref);
  free(q);
  free(q_ref);
  free(s);
  free(s_ref);
  printf("gpu_roundtrip: %s (%zu of %zu codes exact, worst %d step)\n", failures ? "FAILED" : "ok",
         exact, N, worst);
  return failures ? 1 : 0;
}
