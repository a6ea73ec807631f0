/* Drives the C ABI's host-side validation through every error path (and
 * the calls that return before any HIP call: empty batches, queries) in a
 * library whose host code is built with AddressSanitizer and
 * UndefinedBehaviorSanitizer. No call here reaches a HIP API: the pointers
 * are well-aligned fake device addresses that validation never
 * dereferences. Exit status 0 when every call returned what it should. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "gspn.h"
#include "gspn_bench.h"

static int fails = 0;
#define EXPECT(cond) do { if (!(cond)) { fprintf(stderr, "failed: %s (line %d)\n", #cond, __LINE__); ++fails; } } while (0)

#define P(i) ((void*)(uintptr_t)((1ull << 40) + (uint64_t)(i) * (1ull << 32)))

int main(void) {
  const void* lg[3] = {P(1), P(2), P(3)};
  const void* lg_null[3] = {P(1), NULL, P(3)};
  void* dlg[3] = {P(11), P(12), P(13)};
  void* outs5[5] = {P(21), P(22), P(23), P(24), P(25)};
  /* forward */
  EXPECT(gspn_propagate(NULL, lg, P(4), P(5), 1, 1, 8, 8, 15, 0, GSPN_F32, P(6), NULL) == GSPN_E_NULL);
  EXPECT(gspn_propagate(P(0), lg_null, P(4), P(5), 1, 1, 8, 8, 15, 0, GSPN_F32, P(6), NULL) == GSPN_E_NULL);
  EXPECT(gspn_propagate(P(0), lg, P(4), P(5), 1, 1, 0, 8, 15, 0, GSPN_F32, P(6), NULL) == GSPN_E_SHAPE);
  EXPECT(gspn_propagate(P(0), lg, P(4), P(5), 1, 1, 1ll << 31, 8, 15, 0, GSPN_F32, P(6), NULL) == GSPN_E_SHAPE);
  EXPECT(gspn_propagate(P(0), lg, P(4), P(5), INT64_MAX, 2, 8, 8, 15, 0, GSPN_F32, P(6), NULL) == GSPN_E_SHAPE);
  EXPECT(gspn_propagate(P(0), lg, P(4), P(5), 1, 1, 8, 8, 0, 0, GSPN_F32, P(6), NULL) == GSPN_E_DIRMASK);
  EXPECT(gspn_propagate(P(0), lg, P(4), P(5), 1, 1, 8, 8, 16, 0, GSPN_F32, P(6), NULL) == GSPN_E_DIRMASK);
  EXPECT(gspn_propagate(P(0), lg, P(4), P(5), 1, 1, 8, 8, 15, -1, GSPN_F32, P(6), NULL) == GSPN_E_GROUP);
  EXPECT(gspn_propagate(P(0), lg, P(4), P(5), 1, 1, 8, 8, 15, 0, (gspn_dtype)7, P(6), NULL) == GSPN_E_DTYPE);
  EXPECT(gspn_propagate((char*)P(0) + 2, lg, P(4), P(5), 1, 1, 8, 8, 15, 0, GSPN_F32, P(6), NULL) == GSPN_E_ALIGN);
  EXPECT(gspn_propagate(P(0), lg, P(4), P(5), 1, 1, 8, 8, 15, 0, GSPN_F32, (char*)P(0) + 8, NULL) == GSPN_E_ALIAS);
  EXPECT(gspn_propagate(P(0), lg, P(4), P(5), 0, 3, 8, 8, 15, 0, GSPN_F32, P(6), NULL) == GSPN_OK);
  EXPECT(gspn_propagate_ws(P(0), lg, P(4), P(5), 2, 3, 300, 200, 15, 0, GSPN_F32, P(6), NULL, 0, NULL) == GSPN_E_WORKSPACE);
  EXPECT(gspn_propagate_noalloc(P(0), lg, P(4), P(5), 1, 320, 2048, 1024, 15, 0, GSPN_BF16, P(6), NULL) == GSPN_E_WORKSPACE);
  EXPECT(gspn_propagate_noalloc(P(0), lg, P(4), P(5), 0, 3, 8, 8, 15, 0, GSPN_F32, P(6), NULL) == GSPN_OK);
  EXPECT(gspn_propagate_shared_ws(P(0), lg, 4, P(4), P(5), 1, 6, 8, 8, 15, 0, GSPN_F32, P(6), NULL, 0, NULL) == GSPN_E_SHAPE);
  EXPECT(gspn_workspace_bytes(1, 320, 2048, 1024, 15, 0, GSPN_BF16) > 0);
  EXPECT(gspn_workspace_bytes(1, 1, 0, 5, 15, 0, GSPN_F32) == 0);
  EXPECT(gspn_plan_name(64, 96, 56, 56, 15, 0, GSPN_F32)[0] == 'p');
  /* per-direction parameters */
  EXPECT(gspn_propagate_dirs_ws(P(0), lg, P(4), P(5), 3, NULL, 1, 1, 8, 8, 15, 0, GSPN_F32, P(6), NULL, 0, NULL) == GSPN_E_SHAPE);
  EXPECT(gspn_propagate_dirs_ws(P(0), lg, P(4), P(5), 64, (const float*)((char*)P(7) + 2), 1, 1, 8, 8, 15, 0, GSPN_F32, P(6), NULL, 0, NULL) == GSPN_E_ALIGN);
  EXPECT(gspn_workspace_bytes_dirs(1, 2, 100, 100, 15, 0, GSPN_F32) > 0);
  /* backward */
  EXPECT(gspn_propagate_backward(P(0), lg, P(4), P(5), NULL, 1, 1, 8, 8, 15, 0, GSPN_F32, P(10), dlg, P(14), P(15), NULL) == GSPN_E_NULL);
  EXPECT(gspn_propagate_backward(P(0), lg, P(4), P(5), P(9), 1, 1, 8, 8, 15, 0, GSPN_F32, P(0), dlg, P(14), P(15), NULL) == GSPN_E_ALIAS);
  EXPECT(gspn_propagate_backward(P(0), lg, P(4), P(5), P(9), 0, 1, 8, 8, 15, 0, GSPN_F32, P(10), dlg, P(14), P(15), NULL) == GSPN_OK);
  EXPECT(gspn_propagate_backward_ws(P(0), lg, P(4), P(5), P(9), 2, 3, 300, 200, 15, 0, GSPN_F32, P(10), dlg, P(14), P(15), NULL, 0, NULL) == GSPN_E_WORKSPACE);
  EXPECT(gspn_backward_workspace_bytes(1, 320, 2048, 1024, 15, 0, GSPN_BF16) > 0);
  EXPECT(gspn_backward_workspace_bytes_shared(1, 320, 2048, 1024, 1, 15, 0, GSPN_BF16) > 0);
  EXPECT(gspn_backward_workspace_bytes_dirs(1, 2, 100, 100, 15, 0, GSPN_F32) > 0);
  EXPECT(gspn_backward_plan_name(64, 96, 56, 56, 15, 0, GSPN_F32)[0] == 'b');
  EXPECT(gspn_propagate_backward_dirs_ws(P(0), lg, P(4), P(5), 64, NULL, P(9), 1, 1, 8, 8, 15, 0, GSPN_F32, P(0), dlg, P(14), P(15), NULL, NULL, 0, NULL) == GSPN_E_ALIAS);
  /* prologue and module */
  EXPECT(gspn_prologue(P(0), 3, P(1), NULL, P(2), NULL, 1, 4, 8, 8, GSPN_F32, P(20), NULL, NULL) == GSPN_E_NULL);
  EXPECT(gspn_prologue(P(0), 3, P(1), NULL, P(2), NULL, 70000, 4, 8, 8, GSPN_F32, P(20), outs5, NULL) == GSPN_E_SHAPE);
  EXPECT(gspn_prologue(P(0), 3, P(1), NULL, P(2), NULL, 1, 4, 8, 8, GSPN_F32, P(0), outs5, NULL) == GSPN_E_ALIAS);
  EXPECT(gspn_prologue(P(0), 3, P(1), NULL, P(2), NULL, 0, 4, 8, 8, GSPN_F32, P(20), outs5, NULL) == GSPN_OK);
  EXPECT(gspn_module_ws(P(0), 3, P(1), NULL, P(2), NULL, 1, 4, 8, 8, 15, 0, GSPN_F32, P(20), NULL, 0, NULL) == GSPN_E_WORKSPACE);
  EXPECT(gspn_module_workspace_bytes(1, 4, 8, 8, 15, 0, GSPN_F32) > 0);
  /* status text, tracing queries, measurement kernels' argument checks */
  for (int s = 0; s <= 10; ++s) EXPECT(gspn_status_str((gspn_status)s)[0] == 'G');
  EXPECT(gspn_last_error() != NULL);
  EXPECT(gspn_trace_count() >= 0);
  EXPECT(gspn_trace_kernel(-1, NULL) == NULL);
  gspn_trace_events(NULL, 0);
  EXPECT(gspn_abi_version() == 1);
  EXPECT(gspn_noalloc_scratch_bytes() == (size_t)64 << 20);
  EXPECT(gspn_bench_stream(3, 0, P(0), P(1), 4096, 4, NULL) == 1);
  EXPECT(gspn_bench_stream(2, 0, P(0), P(1), 4095, 4, NULL) == 1);
  if (fails) fprintf(stderr, "%d checks failed\n", fails);
  else printf("abi driver: all calls clean\n");
  return fails ? 1 : 0;
}
