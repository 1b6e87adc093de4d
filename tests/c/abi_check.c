/* A plain C11 program against the library's C ABI (include/pa.h, include/pa_sched.h):
 * it includes the headers in C, links libpa.so and calls the entry points that
 * need no GPU: status strings, sizing, argument checks that fail before any
 * launch, and the host scheduler end to end.  Prints one "name value" line per
 * check; the Python test compares them. */
#include <stdint.h>
#include <stdio.h>

#include "pa.h"
#include "pa_sched.h"

int main(void) {
  printf("status_shape %s\n", pa_status_string(PA_ERR_SHAPE));
  printf("default_partition %d\n", (int)pa_default_partition_tokens());
  printf("workspace_full %zu\n", pa_decode_workspace_bytes(64, 32, 64, 128, 0));
  printf("workspace_bad %zu\n", pa_decode_workspace_bytes(0, 32, 64, 128, 0));
  /* argument checks reject these before anything is launched */
  printf("append_null %d\n", pa_append(NULL, NULL, NULL, NULL, NULL, 128, NULL, 4, 8, 64, 1024, NULL));
  printf("decode_dims %d\n", pa_decode(NULL, NULL, NULL, NULL, 128, NULL, 0.125f, NULL, 4, 32, 8, 128, 1024, 0,
                                       NULL, 0, NULL));
  printf("prefill_weights %d\n", pa_prefill(NULL, NULL, NULL, NULL, 4, 100, 32, 8, 64, 0.125f, 7, NULL, NULL));
  printf("prefill_empty %d\n", pa_prefill(NULL, NULL, NULL, NULL, 4, 0, 32, 8, 64, 0.125f, PA_PREFILL_WEIGHTS_FP16,
                                          NULL, NULL));
  printf("rope_empty %d\n", pa_rope_append(NULL, NULL, NULL, NULL, 2048, NULL, NULL, NULL, NULL, 128, NULL, 0, 32, 8,
                                            64, 1024, NULL));
  printf("rope_table %d\n", pa_rope_append(NULL, NULL, NULL, NULL, 0, NULL, NULL, NULL, NULL, 128, NULL, 4, 32, 8,
                                            64, 1024, NULL));
  printf("fill_empty %d\n", pa_fill(NULL, NULL, NULL, NULL, NULL, 128, NULL, NULL, 0, 0, 8, 64, 1024, NULL));

  /* the scheduler: two requests that fit a 48-page pool, a third that waits
   * (each call is made before its results are printed) */
  int64_t budget = 0;
  int st0 = pa_sched_budget_pages(40, 64, 2048, 16, &budget);
  printf("budget %d %lld\n", st0, (long long)budget);
  pa_sched* s = NULL;
  st0 = pa_sched_create(48, 2, 2048, 0, &s);
  printf("create %d\n", st0);
  int64_t ids[3] = {-1, -1, -1};
  for (int i = 0; i < 3; ++i) {
    st0 = pa_sched_submit(s, 100, 200, &ids[i]);
    printf("submit%d %d %lld\n", i, st0, (long long)ids[i]);
  }
  int64_t admitted[3] = {-1, -1, -1};
  int32_t n = 0;
  st0 = pa_sched_admit(s, admitted, 3, &n);
  printf("admit %d %d %lld %lld\n", st0, n, (long long)admitted[0], (long long)admitted[1]);
  printf("grow %d\n", pa_sched_grow(s, ids[0], 100));
  int32_t row[8];
  st0 = pa_sched_block_table(s, ids[0], 1, row, 8);
  printf("table %d %d %d %d %d %d %d %d %d\n", st0, row[0], row[1], row[2], row[3], row[4], row[5], row[6], row[7]);
  printf("grow_beyond %d\n", pa_sched_grow(s, ids[0], 400));
  printf("finish %d\n", pa_sched_finish(s, ids[0]));
  st0 = pa_sched_admit(s, admitted, 3, &n);
  printf("admit2 %d %d %lld\n", st0, n, (long long)(n > 0 ? admitted[0] : -1));
  pa_sched_stats st;
  st0 = pa_sched_get_stats(s, &st);
  printf("stats %d %lld %lld %d %d %lld %lld\n", st0, (long long)st.pool_pages, (long long)st.free_pages, st.active,
         st.waiting, (long long)st.admission_waits, (long long)st.completed);
  pa_sched_destroy(s);
  return 0;
}
