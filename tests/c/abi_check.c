/* Plain C99 use of the C ABI: compiled with gcc against include/arnfp8.h and
 * linked to libarnfp8.so.  Exercises only calls that return before any launch
 * (validation), so it runs on a machine without a GPU.  Exit status 0 = pass. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "arnfp8.h"

static int failures = 0;

static void expect(const char *what, int got, int want) {
  if (got != want) {
    printf("FAIL %s: got %d (%s), want %d\n", what, got, arnfp8_status_string(got), want);
    ++failures;
  }
}

int main(void) {
  /* Fake, well separated, 16-byte aligned device addresses: validation reads none. */
  const uintptr_t base = (uintptr_t)1 << 40, mb = (uintptr_t)1 << 20;
  const void *inputs[2] = {(const void *)base, (const void *)(base + 10 * mb)};
  void *out = (void *)(base + 100 * mb);
  float *scales = (float *)(base + 200 * mb);
  const void *gamma = (const void *)(base + 300 * mb);
  arnfp8_launch opt;
  memset(&opt, 0, sizeof opt);

  expect("bad cols", arnfp8_run(inputs, NULL, NULL, out, scales, gamma, 1e-6f, 0.0f, 1.0f, 4, 12, 2, NULL), ARNFP8_BAD_SHAPE);
  expect("bad P", arnfp8_run(inputs, NULL, NULL, out, scales, gamma, 1e-6f, 0.0f, 1.0f, 4, 256, 0, NULL), ARNFP8_BAD_P);
  expect("null gamma", arnfp8_run(inputs, NULL, NULL, out, scales, NULL, 1e-6f, 0.0f, 1.0f, 4, 256, 2, NULL), ARNFP8_NULL_POINTER);
  expect("misaligned out", arnfp8_run(inputs, NULL, NULL, (char *)out + 8, scales, gamma, 1e-6f, 0.0f, 1.0f, 4, 256, 2, NULL), ARNFP8_MISALIGNED);
  expect("alias", arnfp8_run(inputs, NULL, (void *)inputs[1], out, scales, gamma, 1e-6f, 0.0f, 1.0f, 4, 256, 2, NULL), ARNFP8_ALIAS);
  expect("rows 0", arnfp8_run(inputs, NULL, NULL, NULL, NULL, NULL, 1e-6f, 0.0f, 1.0f, 0, 256, 2, NULL), ARNFP8_OK);
  expect("negative eps", arnfp8_run(inputs, NULL, NULL, out, scales, gamma, -1.0f, 0.0f, 1.0f, 4, 256, 2, NULL), ARNFP8_BAD_SCALAR);
  expect("zero scale_ub", arnfp8_run(inputs, NULL, NULL, out, scales, gamma, 1e-6f, 0.0f, 0.0f, 4, 256, 2, NULL), ARNFP8_BAD_SCALAR);
  opt.threads = 96;
  expect("bad threads", arnfp8_run_ex(inputs, NULL, NULL, out, scales, gamma, 1e-6f, 0.0f, 1.0f, 4, 256, 2, NULL, &opt), ARNFP8_BAD_CONFIG);
  expect("bad format", arnfp8_run_fmt(inputs, NULL, NULL, out, scales, gamma, 1e-6f, 0.0f, 1.0f, 4, 256, 2, 42, NULL, NULL), ARNFP8_BAD_FORMAT);
  expect("bad share", arnfp8_run_share(inputs, NULL, NULL, out, gamma, 1e-6f, 0.0f, 1.0f, 4, 256, 2, 4, 4, NULL), ARNFP8_BAD_SHARE);
  {
    arnfp8_split_opts sopt = {9, 0};
    void *ws = (void *)(base + 500 * mb);
    expect("split bad parts", arnfp8_run_split(inputs, NULL, NULL, out, scales, gamma, 1e-6f, 0.0f, 1.0f, 4, 256, 2, ws, 512, NULL, &sopt), ARNFP8_BAD_CONFIG);
    sopt.parts = 2;
    expect("split small workspace", arnfp8_run_split(inputs, NULL, NULL, out, scales, gamma, 1e-6f, 0.0f, 1.0f, 4, 256, 2, ws, 511, NULL, &sopt), ARNFP8_BAD_WORKSPACE);
    expect("split rows 0", arnfp8_run_split(inputs, NULL, NULL, NULL, NULL, NULL, 1e-6f, 0.0f, 1.0f, 0, 256, 2, NULL, 0, NULL, &sopt), ARNFP8_OK);
    expect("noalloc too many rows", arnfp8_run_split_noalloc(inputs, NULL, NULL, out, scales, gamma, 1e-6f, 0.0f, 1.0f, ARNFP8_NOALLOC_MAX_ROWS + 1, 256, 2, NULL, &sopt), ARNFP8_BAD_WORKSPACE);
    expect("noalloc rows 0", arnfp8_run_split_noalloc(inputs, NULL, NULL, NULL, NULL, NULL, 1e-6f, 0.0f, 1.0f, 0, 256, 2, NULL, &sopt), ARNFP8_OK);
    if (arnfp8_split_workspace_bytes(4) != 512) {
      printf("FAIL split workspace bytes\n");
      ++failures;
    }
  }
  expect("sum bad shape", arn_sum_bf16(inputs, out, 4, 7, 2, NULL), ARNFP8_BAD_SHAPE);
  expect("convert bad n", arnfp8_convert_f32((const float *)base, out, 12, ARNFP8_FMT_E4M3FN, NULL), ARNFP8_BAD_SHAPE);
  if (arnfp8_stage_bytes(8192, 7168, 8) != 7344128) {
    printf("FAIL stage bytes\n");
    ++failures;
  }
  if (strcmp(arnfp8_status_string(12345), "unknown status") != 0) {
    printf("FAIL status string\n");
    ++failures;
  }
  printf("%s\n", failures ? "abi_check: FAILED" : "abi_check: ok");
  return failures ? 1 : 0;
}
