/* A plain C11 caller of the prefill path on the GPU.  It builds three packed
 * prompts with a fixed generator, places them in device memory from hipMalloc,
 * calls pa_fill (the prompts into their pages) and pa_prefill in both weight
 * modes through include/pa.h on the default stream, and writes its inputs and
 * results to the file named by its argument, for the Python test to check
 * against the oracle:
 *   q [T][32][64], k, v [T][8][64], block_table [B][8], cu_tokens [B+1],
 *   K and V pools before [16][16][8][64] (bf16 bits), K and V pools after,
 *   out [2][T][32][64] (fp32: bf16-pair weights, fp16 weights).
 * Exit status: 0, or the step that failed (its status printed on stderr). */
#include <stdint.h>
#include <stdio.h>

#include <hip/hip_runtime_api.h>

#include "pa.h"

enum { B = 3, T = 111, HQ = 32, HKV = 8, D = 64, MAXB = 8, PAGES = 16, PT = 16 };
#define POOL_ELEMS ((size_t)PAGES * PT * HKV * D)
#define Q_ELEMS ((size_t)T * HQ * D)
#define KV_ELEMS ((size_t)T * HKV * D)

static uint32_t state = 777u;

/* bf16 bits of a value in +-[0.25, 2): random sign, exponent 125..127, random mantissa */
static uint16_t next_bf16(void) {
  state = state * 1664525u + 1013904223u;
  const uint32_t r = state >> 8;
  const uint32_t sign = r & 1u, exp = 125u + (r >> 1) % 3u, mant = (r >> 3) & 0x7fu;
  return (uint16_t)((sign << 15) | (exp << 7) | mant);
}

static int check(hipError_t e, const char* what) {
  if (e != hipSuccess) {
    fprintf(stderr, "%s: %s\n", what, hipGetErrorString(e));
    return 1;
  }
  return 0;
}

int main(int argc, char** argv) {
  if (argc != 2) {
    fprintf(stderr, "usage: %s out_file\n", argv[0]);
    return 2;
  }
  static uint16_t q[Q_ELEMS], k[KV_ELEMS], v[KV_ELEMS], kp[POOL_ELEMS], vp[POOL_ELEMS];
  static uint16_t kp_after[POOL_ELEMS], vp_after[POOL_ELEMS];
  static float out[2][Q_ELEMS];
  /* prompts of 40, 1 and 70 tokens: pages 9, 3, 14 | 0 | 6, 12, 1, 8, 15 */
  const int32_t bt[B][MAXB] = {{9, 3, 14, -1, -1, -1, -1, -1},
                               {0, -1, -1, -1, -1, -1, -1, -1},
                               {6, 12, 1, 8, 15, -1, -1, -1}};
  const int32_t cu[B + 1] = {0, 40, 41, T};
  for (size_t i = 0; i < Q_ELEMS; ++i) q[i] = next_bf16();
  for (size_t i = 0; i < KV_ELEMS; ++i) k[i] = next_bf16();
  for (size_t i = 0; i < KV_ELEMS; ++i) v[i] = next_bf16();
  for (size_t i = 0; i < POOL_ELEMS; ++i) kp[i] = next_bf16();
  for (size_t i = 0; i < POOL_ELEMS; ++i) vp[i] = next_bf16();

  void *dq, *dk, *dv, *dkp, *dvp, *dbt, *dcu, *dout;
  if (check(hipMalloc(&dq, sizeof q), "hipMalloc") || check(hipMalloc(&dk, sizeof k), "hipMalloc") ||
      check(hipMalloc(&dv, sizeof v), "hipMalloc") || check(hipMalloc(&dkp, sizeof kp), "hipMalloc") ||
      check(hipMalloc(&dvp, sizeof vp), "hipMalloc") || check(hipMalloc(&dbt, sizeof bt), "hipMalloc") ||
      check(hipMalloc(&dcu, sizeof cu), "hipMalloc") || check(hipMalloc(&dout, sizeof out[0]), "hipMalloc"))
    return 4;
  if (check(hipMemcpy(dq, q, sizeof q, hipMemcpyHostToDevice), "copy") ||
      check(hipMemcpy(dk, k, sizeof k, hipMemcpyHostToDevice), "copy") ||
      check(hipMemcpy(dv, v, sizeof v, hipMemcpyHostToDevice), "copy") ||
      check(hipMemcpy(dkp, kp, sizeof kp, hipMemcpyHostToDevice), "copy") ||
      check(hipMemcpy(dvp, vp, sizeof vp, hipMemcpyHostToDevice), "copy") ||
      check(hipMemcpy(dbt, bt, sizeof bt, hipMemcpyHostToDevice), "copy") ||
      check(hipMemcpy(dcu, cu, sizeof cu, hipMemcpyHostToDevice), "copy"))
    return 5;

  int st = pa_fill((const uint16_t*)dk, (const uint16_t*)dv, (uint16_t*)dkp, (uint16_t*)dvp, (const int32_t*)dbt,
                   MAXB, NULL, (const int32_t*)dcu, B, T, HKV, D, PAGES, NULL);
  if (st != PA_OK) {
    fprintf(stderr, "pa_fill: %s\n", pa_status_string(st));
    return 6;
  }
  const int32_t modes[2] = {PA_PREFILL_WEIGHTS_BF16X2, PA_PREFILL_WEIGHTS_FP16};
  for (int c = 0; c < 2; ++c) {
    st = pa_prefill((const uint16_t*)dq, (const uint16_t*)dk, (const uint16_t*)dv, (const int32_t*)dcu, B, T, HQ, HKV,
                    D, 0.125f, modes[c], (float*)dout, NULL);
    if (st != PA_OK) {
      fprintf(stderr, "pa_prefill (weights %d): %s\n", modes[c], pa_status_string(st));
      return 6;
    }
    if (check(hipDeviceSynchronize(), "synchronize") ||
        check(hipMemcpy(out[c], dout, sizeof out[c], hipMemcpyDeviceToHost), "copy back"))
      return 7;
  }
  if (check(hipMemcpy(kp_after, dkp, sizeof kp_after, hipMemcpyDeviceToHost), "copy back") ||
      check(hipMemcpy(vp_after, dvp, sizeof vp_after, hipMemcpyDeviceToHost), "copy back"))
    return 7;

  FILE* f = fopen(argv[1], "wb");
  if (!f) return 8;
  int ok = fwrite(q, sizeof q, 1, f) == 1 && fwrite(k, sizeof k, 1, f) == 1 && fwrite(v, sizeof v, 1, f) == 1 &&
           fwrite(bt, sizeof bt, 1, f) == 1 && fwrite(cu, sizeof cu, 1, f) == 1 &&
           fwrite(kp, sizeof kp, 1, f) == 1 && fwrite(vp, sizeof vp, 1, f) == 1 &&
           fwrite(kp_after, sizeof kp_after, 1, f) == 1 && fwrite(vp_after, sizeof vp_after, 1, f) == 1 &&
           fwrite(out, sizeof out, 1, f) == 1;
  ok = (fclose(f) == 0) && ok;
  hipFree(dq), hipFree(dk), hipFree(dv), hipFree(dkp), hipFree(dvp), hipFree(dbt), hipFree(dcu), hipFree(dout);
  return ok ? 0 : 9;
}
