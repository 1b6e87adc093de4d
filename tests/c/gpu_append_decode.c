/* A plain C11 caller of the library on the GPU.  It builds a small paged state
 * with a fixed generator, places it in device memory from hipMalloc, calls
 * pa_append_decode through include/pa.h on the default stream (the automatic
 * split, then one page per split), then the same two steps planned
 * (pa_decode_plan, pa_decode_planned) and through the allocation-free entry
 * point (pa_append_decode_noalloc), and writes its inputs and results to the
 * file named by its argument, for the Python test to check against the
 * oracle:
 *   q [B][32][64], k_new, v_new [B][8][64], block_table [B][4], seq_lens [B],
 *   K and V pools before [12][16][8][64] (bf16 bits), K and V pools after,
 *   out [6][B][32][64] (fp32: unplanned automatic, unplanned one page,
 *   planned automatic, planned one page, allocation-free automatic,
 *   allocation-free one page).
 * Exit status: 0, or the step that failed (its status printed on stderr). */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "pa.h"

enum { B = 3, HQ = 32, HKV = 8, D = 64, MAXB = 4, PAGES = 12, PT = 16 };
#define POOL_ELEMS ((size_t)PAGES * PT * HKV * D)
#define Q_ELEMS ((size_t)B * HQ * D)
#define NEW_ELEMS ((size_t)B * HKV * D)

static uint32_t state = 12345u;

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
  static uint16_t q[Q_ELEMS], k_new[NEW_ELEMS], v_new[NEW_ELEMS], kp[POOL_ELEMS], vp[POOL_ELEMS];
  static uint16_t kp_after[POOL_ELEMS], vp_after[POOL_ELEMS];
  static float out[6][Q_ELEMS];
  /* three sequences after the append: 37 tokens on pages 7, 2, 10; 16 on page 4; 1 on page 11 */
  const int32_t bt[B][MAXB] = {{7, 2, 10, -1}, {4, -1, -1, -1}, {11, -1, -1, -1}};
  const int32_t lens[B] = {37, 16, 1};
  for (size_t i = 0; i < Q_ELEMS; ++i) q[i] = next_bf16();
  for (size_t i = 0; i < NEW_ELEMS; ++i) k_new[i] = next_bf16();
  for (size_t i = 0; i < NEW_ELEMS; ++i) v_new[i] = next_bf16();
  for (size_t i = 0; i < POOL_ELEMS; ++i) kp[i] = next_bf16();
  for (size_t i = 0; i < POOL_ELEMS; ++i) vp[i] = next_bf16();

  void *dq, *dk_new, *dv_new, *dkp, *dvp, *dbt, *dlens, *dout, *dws, *dplan;
  const size_t ws_bytes = pa_decode_workspace_bytes(B, HQ, D, MAXB, PT);  /* the larger of the two splits */
  const size_t plan_bytes = pa_decode_plan_bytes(B, MAXB, PT) > pa_decode_plan_bytes(B, MAXB, 0)
                                ? pa_decode_plan_bytes(B, MAXB, PT)
                                : pa_decode_plan_bytes(B, MAXB, 0);
  if (ws_bytes == 0 || plan_bytes == 0) return 3;
  if (check(hipMalloc(&dq, sizeof q), "hipMalloc") || check(hipMalloc(&dk_new, sizeof k_new), "hipMalloc") ||
      check(hipMalloc(&dv_new, sizeof v_new), "hipMalloc") || check(hipMalloc(&dkp, sizeof kp), "hipMalloc") ||
      check(hipMalloc(&dvp, sizeof vp), "hipMalloc") || check(hipMalloc(&dbt, sizeof bt), "hipMalloc") ||
      check(hipMalloc(&dlens, sizeof lens), "hipMalloc") || check(hipMalloc(&dout, sizeof out[0]), "hipMalloc") ||
      check(hipMalloc(&dws, ws_bytes), "hipMalloc") || check(hipMalloc(&dplan, plan_bytes), "hipMalloc"))
    return 4;
  if (check(hipMemcpy(dq, q, sizeof q, hipMemcpyHostToDevice), "copy") ||
      check(hipMemcpy(dk_new, k_new, sizeof k_new, hipMemcpyHostToDevice), "copy") ||
      check(hipMemcpy(dv_new, v_new, sizeof v_new, hipMemcpyHostToDevice), "copy") ||
      check(hipMemcpy(dkp, kp, sizeof kp, hipMemcpyHostToDevice), "copy") ||
      check(hipMemcpy(dvp, vp, sizeof vp, hipMemcpyHostToDevice), "copy") ||
      check(hipMemcpy(dbt, bt, sizeof bt, hipMemcpyHostToDevice), "copy") ||
      check(hipMemcpy(dlens, lens, sizeof lens, hipMemcpyHostToDevice), "copy") ||
      check(hipMemset(dws, 0, ws_bytes), "hipMemset"))
    return 5;

  const int32_t partitions[2] = {0, PT};
  for (int c = 0; c < 2; ++c) {
    /* the append writes the same rows both times, so the second call sees the same pools */
    const int st = pa_append_decode((const uint16_t*)dk_new, (const uint16_t*)dv_new, (uint16_t*)dkp, (uint16_t*)dvp,
                                    (const uint16_t*)dq, (const int32_t*)dbt, MAXB, (const int32_t*)dlens, 0.125f,
                                    (float*)dout, B, HQ, HKV, D, PAGES, partitions[c], dws, ws_bytes, NULL);
    if (st != PA_OK) {
      fprintf(stderr, "pa_append_decode (partition %d): %s\n", partitions[c], pa_status_string(st));
      return 6;
    }
    if (check(hipDeviceSynchronize(), "synchronize") ||
        check(hipMemcpy(out[c], dout, sizeof out[c], hipMemcpyDeviceToHost), "copy back"))
      return 7;
  }
  for (int c = 0; c < 2; ++c) {
    /* the same steps with the plan built once, as for the layers of a step */
    int st = pa_decode_plan((const int32_t*)dlens, B, MAXB, partitions[c], dplan, plan_bytes, NULL);
    if (st == PA_OK)
      st = pa_decode_planned((const uint16_t*)dq, (const uint16_t*)dk_new, (const uint16_t*)dv_new, NULL, 0,
                             (uint16_t*)dkp, (uint16_t*)dvp, (const int32_t*)dbt, MAXB, 0.125f, (float*)dout, B, HQ,
                             HKV, D, PAGES, partitions[c], dplan, plan_bytes, dws, ws_bytes, NULL);
    if (st != PA_OK) {
      fprintf(stderr, "planned decode (partition %d): %s\n", partitions[c], pa_status_string(st));
      return 6;
    }
    if (check(hipDeviceSynchronize(), "synchronize") ||
        check(hipMemcpy(out[2 + c], dout, sizeof out[2 + c], hipMemcpyDeviceToHost), "copy back"))
      return 7;
  }
  for (int c = 0; c < 2; ++c) {
    /* the same steps with no workspace: the library's own scratch array */
    const int st = pa_append_decode_noalloc((const uint16_t*)dk_new, (const uint16_t*)dv_new, (uint16_t*)dkp,
                                            (uint16_t*)dvp, (const uint16_t*)dq, (const int32_t*)dbt, MAXB,
                                            (const int32_t*)dlens, 0.125f, (float*)dout, B, HQ, HKV, D, PAGES,
                                            partitions[c], NULL);
    if (st != PA_OK) {
      fprintf(stderr, "pa_append_decode_noalloc (partition %d): %s\n", partitions[c], pa_status_string(st));
      return 6;
    }
    if (check(hipDeviceSynchronize(), "synchronize") ||
        check(hipMemcpy(out[4 + c], dout, sizeof out[4 + c], hipMemcpyDeviceToHost), "copy back"))
      return 7;
  }
  if (check(hipMemcpy(kp_after, dkp, sizeof kp_after, hipMemcpyDeviceToHost), "copy back") ||
      check(hipMemcpy(vp_after, dvp, sizeof vp_after, hipMemcpyDeviceToHost), "copy back"))
    return 7;

  FILE* f = fopen(argv[1], "wb");
  if (!f) return 8;
  int ok = fwrite(q, sizeof q, 1, f) == 1 && fwrite(k_new, sizeof k_new, 1, f) == 1 &&
           fwrite(v_new, sizeof v_new, 1, f) == 1 && fwrite(bt, sizeof bt, 1, f) == 1 &&
           fwrite(lens, sizeof lens, 1, f) == 1 && fwrite(kp, sizeof kp, 1, f) == 1 &&
           fwrite(vp, sizeof vp, 1, f) == 1 && fwrite(kp_after, sizeof kp_after, 1, f) == 1 &&
           fwrite(vp_after, sizeof vp_after, 1, f) == 1 && fwrite(out, sizeof out, 1, f) == 1;
  ok = (fclose(f) == 0) && ok;
  hipFree(dq), hipFree(dk_new), hipFree(dv_new), hipFree(dkp), hipFree(dvp);
  hipFree(dbt), hipFree(dlens), hipFree(dout), hipFree(dws), hipFree(dplan);
  return ok ? 0 : 9;
}
