/* A C99 caller of the library through include/fp8bq.h alone (no HIP headers): links against
 * libfp8bq.so and exercises entry points that return before touching a device — status strings,
 * the version, workspace sizes, plans and argument validation — checking the documented codes.
 * Prints "ok" and exits 0 on success. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "fp8bq.h"

static int failures = 0;
#define EXPECT(cond)                                              \
  do {                                                            \
    if (!(cond)) {                                                \
      fprintf(stderr, "%s:%d: failed: %s\n", __FILE__, __LINE__, #cond); \
      ++failures;                                                 \
    }                                                             \
  } while (0)

int main(void) {
  EXPECT(fp8bq_version() >= 100);
  EXPECT(strncmp(fp8bq_status_string(FP8BQ_OK), "FP8BQ_OK", 8) == 0);
  EXPECT(strncmp(fp8bq_status_string(FP8BQ_ERR_SHAPE), "FP8BQ_ERR_SHAPE", 15) == 0);
  EXPECT(strcmp(fp8bq_status_string(12345), "FP8BQ_ERR_UNKNOWN") == 0);

  int32_t tm = 0, tn = 0, sk = 0;
  EXPECT(fp8bq_gemm_plan(FP8BQ_OP_FPROP, 16384, 11264, 2048, &tm, &tn, &sk) == FP8BQ_OK);
  EXPECT(tm > 0 && tn > 0 && sk >= 1);
  EXPECT(fp8bq_gemm_plan(FP8BQ_OP_FPROP, 16384, 11264, 2048, NULL, &tn, &sk) == FP8BQ_ERR_NULL);
  EXPECT(fp8bq_gemm_workspace_size(FP8BQ_OP_DGRAD, 4096, 2048, 2048) >= (size_t)2048 * 2048);
  EXPECT(fp8bq_quantize_tensor_workspace_size(0, 128) == 0);
  EXPECT(fp8bq_hyperball_workspace_size(256, 256) > 0);

  /* validation happens before any device work: these return without a GPU */
  static uint8_t q[256 * 256];
  static float s[2 * 256];
  static uint16_t x[256 * 256];
  EXPECT(fp8bq_quantize_act_1x128(x, FP8BQ_IN_BF16, 256, 200, 256, FP8BQ_E4M3, q, 256, s, 256, NULL) ==
         FP8BQ_ERR_SHAPE);                                   /* C not a multiple of 128 */
  EXPECT(fp8bq_quantize_act_1x128(x, FP8BQ_IN_BF16, 256, 256, 256, (fp8bq_fp8)7, q, 256, s, 256, NULL) ==
         FP8BQ_ERR_FORMAT);
  EXPECT(fp8bq_quantize_act_1x128(NULL, FP8BQ_IN_BF16, 256, 256, 256, FP8BQ_E4M3, q, 256, s, 256, NULL) ==
         FP8BQ_ERR_NULL);
  EXPECT(fp8bq_quantize_act_1x128(x, FP8BQ_IN_BF16, 0, 256, 256, FP8BQ_E4M3, q, 256, s, 256, NULL) ==
         FP8BQ_OK);                                          /* empty: nothing to do */
  EXPECT(fp8bq_gemm_fprop(256, 256, 200, q, 256, s, 256, FP8BQ_E4M3, q, 256, s, 2, FP8BQ_E4M3, x,
                          FP8BQ_OUT_BF16, 256, NULL, 0, NULL) == FP8BQ_ERR_SHAPE);
  EXPECT(fp8bq_gemm_fprop(256, 256, 256, q, 256, s, 256, FP8BQ_E4M3, q, 256, s, 2, FP8BQ_E4M3, x,
                          FP8BQ_OUT_F32_ACCUM, 256, NULL, 0, NULL) == FP8BQ_ERR_DTYPE);
  float amax = 1.0f, scale = 0.0f;
  static uint8_t ws[8192];
  EXPECT(fp8bq_quantize_tensor_delayed(x, FP8BQ_IN_BF16, 256, 256, 256, FP8BQ_E4M3, &amax, 1.5, q, 256, NULL, 0,
                                       &scale, ws, sizeof ws, NULL) == FP8BQ_ERR_VALUE);
  EXPECT(fp8bq_quantize_tensor_delayed_noalloc(x, FP8BQ_IN_BF16, 256, 256, 256, FP8BQ_E4M3, &amax, 1.5, q, 256,
                                               NULL, 0, &scale, NULL) == FP8BQ_ERR_VALUE);
  EXPECT(fp8bq_quantize_tensor_delayed_noalloc(x, FP8BQ_IN_BF16, 0, 256, 256, FP8BQ_E4M3, &amax, 0.5, q, 256, NULL,
                                               0, &scale, NULL) == FP8BQ_OK);  /* empty: nothing to do */
  static float w[256 * 256];
  EXPECT(fp8bq_hyperball_step(w, 256, x, FP8BQ_IN_BF16, 256, 256, 256, 1e-4, 0.1, 0.0, 0.0, NULL, ws, sizeof ws,
                              NULL) == FP8BQ_ERR_VALUE);     /* eps must be > 0 */
  /* several Hyperball steps: too many jobs, one job's weights on another's gradient, none */
  fp8bq_hyperball_job hj[2] = {{w, 256, x, 256, 256, 256, 0.0, NULL}, {w + 256 * 256 / 2, 256, x, 256, 128, 256, 1.0, NULL}};
  EXPECT(fp8bq_hyperball_batch_workspace_size(FP8BQ_MAX_HYPERBALL_JOBS + 1) == 0);
  EXPECT(fp8bq_hyperball_step_batch(hj, FP8BQ_MAX_HYPERBALL_JOBS + 1, FP8BQ_IN_BF16, 1e-4, 0.1, 1e-8, ws, sizeof ws,
                                    NULL) == FP8BQ_ERR_VALUE);
  static double hws[2 * 3 * 1024];                          /* two jobs' partial sums (16-byte aligned) */
  EXPECT(fp8bq_hyperball_batch_workspace_size(2) <= sizeof hws);
  EXPECT(fp8bq_hyperball_step_batch(hj, 2, FP8BQ_IN_BF16, 1e-4, 0.1, 1e-8, hws, sizeof hws, NULL) ==
         FP8BQ_ERR_OVERLAP);                                  /* job 1's w lies inside job 0's w */
  EXPECT(fp8bq_hyperball_step_batch(hj, 0, FP8BQ_IN_BF16, 1e-4, 0.1, 1e-8, NULL, 0, NULL) == FP8BQ_OK);
  /* the streaming-copy reference: a size not a multiple of 16, overlapping ranges, empty */
  EXPECT(fp8bq_stream_copy(w, q, 100, NULL) == FP8BQ_ERR_SHAPE);
  EXPECT(fp8bq_stream_copy(w, (uint8_t*)w + 256, 1024, NULL) == FP8BQ_ERR_OVERLAP);
  EXPECT(fp8bq_stream_copy(NULL, NULL, 0, NULL) == FP8BQ_OK);
  /* several weights: a job array from C, checked job by job and across jobs */
  static uint8_t qt[256 * 256], q2[256 * 256], qt2[256 * 256];
  static float s2[4];
  fp8bq_weight_job jobs[2] = {{x, 256, 256, 256, q, 256, s, 2, qt, 256}, {x, 256, 256, 256, q2, 256, s2, 2, qt2, 256}};
  EXPECT(fp8bq_quantize_weights_dual(jobs, 0, FP8BQ_IN_BF16, FP8BQ_E4M3, NULL) == FP8BQ_OK);
  EXPECT(fp8bq_quantize_weights_dual(jobs, FP8BQ_MAX_WEIGHT_JOBS + 1, FP8BQ_IN_BF16, FP8BQ_E4M3, NULL) ==
         FP8BQ_ERR_VALUE);
  jobs[1].q = q;                                             /* job 1 would overwrite job 0's codes */
  EXPECT(fp8bq_quantize_weights_dual(jobs, 2, FP8BQ_IN_BF16, FP8BQ_E4M3, NULL) == FP8BQ_ERR_OVERLAP);
  jobs[1].q = q2;
  jobs[1].K = 200;
  EXPECT(fp8bq_quantize_weights_dual(jobs, 2, FP8BQ_IN_BF16, FP8BQ_E4M3, NULL) == FP8BQ_ERR_SHAPE);

  if (failures) return 1;
  printf("ok\n");
  return 0;
}
