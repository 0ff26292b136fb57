/*
 * A plain C caller of libthdcp: only include/thd_cp.h and the HIP runtime's
 * C API, no Python, no PyTorch.  It runs the worked example of the page
 * "Packed Sequence 与上下文并行" (§3.1-§3.8: two rows of eight tokens, CP 2,
 * alignment 4) through the whole path and compares every result with the
 * values that page prints:
 *   pack -> cu_seqlens, cu_seqlens_padded, the packed stream   (§3.2-§3.4)
 *   route build, c->z swap -> the two ranks' zigzag tokens      (§3.5-§3.6)
 *   z->c swap -> the packed stream again
 *   roll in zigzag order -> the ranks' valid masks, 13 in all    (§3.6, §3.8)
 *   the same pack through thd_pack_noalloc (no workspace argument)
 *
 * Usage: thd_worked_example host   (argument checks only; no GPU needed)
 *        thd_worked_example gpu    (the whole example on device 0)
 * Exit status 0 when every check holds.
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "thd_cp.h"

static int failures = 0;

#define CHECK(cond, ...)                      \
  do {                                        \
    if (!(cond)) {                            \
      fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
      fprintf(stderr, __VA_ARGS__);           \
      fprintf(stderr, "\n");                  \
      ++failures;                             \
    }                                         \
  } while (0)

#define HIP_OK(call)                                                     \
  do {                                                                   \
    hipError_t e_ = (call);                                              \
    if (e_ != hipSuccess) {                                              \
      fprintf(stderr, "HIP error %d at %s:%d\n", (int)e_, __FILE__, __LINE__); \
      return 2;                                                          \
    }                                                                    \
  } while (0)

static int host_checks(void) {
  thd_route* r = NULL;
  CHECK(thd_route_create(0, 2, 16, &r) == THD_ERR_ARG, "create with 0 slots");
  CHECK(thd_route_create(4, 0, 16, &r) == THD_ERR_ARG, "create with cp 0");
  CHECK(thd_route_create(4, 2, 16, NULL) == THD_ERR_ARG, "create without an output");
  CHECK(thd_swap(NULL, THD_ZIGZAG_TO_CONTIGUOUS, NULL, NULL, 16, 8, NULL) == THD_ERR_ARG, "swap without a route");
  CHECK(thd_copy(NULL, NULL, 0, NULL) == THD_OK, "empty copy");
  CHECK(thd_pack_workspace_bytes(-1, 8) == -1, "workspace for a negative batch");
  CHECK(strlen(thd_strerror(THD_ERR_CU_DIVISIBLE)) > 0, "strerror");
  /* the pack without a workspace refuses a batch past its static scratch on the host */
  CHECK(thd_pack_noalloc(NULL, 2, 1 << 30, 0, 1, 8, 8, 1, 0, NULL, NULL, NULL, NULL, NULL) == THD_ERR_CAPACITY,
        "pack_noalloc beyond its scratch");
  CHECK(thd_pack_noalloc(NULL, -1, 8, 0, 1, 8, 8, 1, 0, NULL, NULL, NULL, NULL, NULL) == THD_ERR_ARG,
        "pack_noalloc with a negative batch");
  return failures;
}

static int gpu_example(void) {
  /* §3.1: two samples of eight tokens, '_' is PAD and 'E' the EOD token */
  const char* samples = "abcEdeE_fghijE__";
  /* §3.2-§3.4 */
  const int32_t want_cu[4] = {0, 4, 7, 13};
  const int32_t want_cu_pad[4] = {0, 4, 8, 16};
  const char* want_tokens = "abcEdeEPfghijEPP";
  /* §3.6: rank 0's then rank 1's zigzag share, and their valid masks */
  const char* want_zigzag = "aEdPfgPPbceEhijE";
  const uint8_t want_mask[16] = {1, 1, 1, 0, 1, 1, 0, 0, 1, 1, 1, 1, 1, 1, 1, 1};
  enum { B = 2, S = 8, T = 16, MAX_DOCS = 3, SLOTS = MAX_DOCS + 1, CP = 2 };

  int64_t h_rows[B * S], h_out[T];
  for (int i = 0; i < B * S; ++i) h_rows[i] = samples[i];

  hipStream_t stream;
  HIP_OK(hipStreamCreate(&stream));
  int64_t *rows, *packed, *zig, *back, *shifted;
  int32_t *cu, *cu_pad, *status;
  uint8_t *mask, *ws;
  const int64_t ws_bytes = thd_pack_workspace_bytes(B, S);
  HIP_OK(hipMalloc((void**)&rows, sizeof(h_rows)));
  HIP_OK(hipMalloc((void**)&packed, T * 8));
  HIP_OK(hipMalloc((void**)&zig, T * 8));
  HIP_OK(hipMalloc((void**)&back, T * 8));
  HIP_OK(hipMalloc((void**)&shifted, T * 8));
  HIP_OK(hipMalloc((void**)&mask, 2 * T));
  HIP_OK(hipMalloc((void**)&cu, (MAX_DOCS + 2) * 4));
  HIP_OK(hipMalloc((void**)&cu_pad, (MAX_DOCS + 2) * 4));
  HIP_OK(hipMalloc((void**)&status, 8));
  HIP_OK(hipMalloc((void**)&ws, (size_t)ws_bytes));
  HIP_OK(hipMemcpy(rows, h_rows, sizeof(h_rows), hipMemcpyHostToDevice));

  /* pack (§3.3: alignment TP*CP*2 = 4) */
  CHECK(thd_pack(rows, B, S, '_', 'E', 4, T, MAX_DOCS, 'P', ws, ws_bytes, packed, cu, cu_pad, status, stream) ==
            THD_OK, "thd_pack");
  /* route from the padded boundaries, then both swaps of the packed ids */
  thd_route* route = NULL;
  CHECK(thd_route_create(SLOTS, CP, T, &route) == THD_OK, "thd_route_create");
  CHECK(thd_build_route(route, cu_pad, SLOTS, CP, T, stream) == THD_OK, "thd_build_route");
  CHECK(thd_swap(route, THD_CONTIGUOUS_TO_ZIGZAG, packed, zig, T, 8, stream) == THD_OK, "c->z swap");
  CHECK(thd_swap(route, THD_ZIGZAG_TO_CONTIGUOUS, zig, back, T, 8, stream) == THD_OK, "z->c swap");
  CHECK(thd_roll_labels_zigzag(route, packed, cu_pad, cu, SLOTS, T, 1, -1, shifted, mask, status + 1, stream) ==
            THD_OK, "zigzag roll");
  HIP_OK(hipStreamSynchronize(stream));

  int32_t h_cu[MAX_DOCS + 2], h_cu_pad[MAX_DOCS + 2], h_status[2], route_status = -99;
  uint8_t h_mask[2 * T];
  HIP_OK(hipMemcpy(h_cu, cu, sizeof(h_cu), hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(h_cu_pad, cu_pad, sizeof(h_cu_pad), hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(h_status, status, sizeof(h_status), hipMemcpyDeviceToHost));
  CHECK(h_status[0] == THD_OK && h_status[1] == THD_OK, "pack status %d, roll status %d", h_status[0], h_status[1]);
  CHECK(thd_route_status(route, stream, &route_status) == THD_OK && route_status == THD_OK, "route status %d",
        route_status);
  for (int k = 0; k < 4; ++k) {
    CHECK(h_cu[k] == want_cu[k], "cu_seqlens[%d] = %d, want %d", k, h_cu[k], want_cu[k]);
    CHECK(h_cu_pad[k] == want_cu_pad[k], "cu_seqlens_padded[%d] = %d, want %d", k, h_cu_pad[k], want_cu_pad[k]);
  }
  /* slot 3 is the trailing pad-only slot: empty here, the documents fill the budget */
  CHECK(h_cu[4] == 13 && h_cu_pad[4] == 16, "trailing slot %d %d", h_cu[4], h_cu_pad[4]);

  HIP_OK(hipMemcpy(h_out, packed, sizeof(h_out), hipMemcpyDeviceToHost));
  for (int i = 0; i < T; ++i) CHECK(h_out[i] == want_tokens[i], "packed[%d] = %c", i, (char)h_out[i]);

  /* the same pack without a workspace argument (the library's static scratch),
     written over the outputs of the first: the same stream and boundaries */
  HIP_OK(hipMemset(packed, 0, T * 8));
  HIP_OK(hipMemset(cu, 0, (MAX_DOCS + 2) * 4));
  HIP_OK(hipMemset(cu_pad, 0, (MAX_DOCS + 2) * 4));
  CHECK(thd_pack_noalloc(rows, B, S, '_', 'E', 4, T, MAX_DOCS, 'P', packed, cu, cu_pad, status, stream) == THD_OK,
        "thd_pack_noalloc");
  HIP_OK(hipStreamSynchronize(stream));
  HIP_OK(hipMemcpy(h_status, status, 4, hipMemcpyDeviceToHost));
  CHECK(h_status[0] == THD_OK, "pack_noalloc status %d", h_status[0]);
  HIP_OK(hipMemcpy(h_cu, cu, sizeof(h_cu), hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(h_cu_pad, cu_pad, sizeof(h_cu_pad), hipMemcpyDeviceToHost));
  for (int k = 0; k < 4; ++k)
    CHECK(h_cu[k] == want_cu[k] && h_cu_pad[k] == want_cu_pad[k], "pack_noalloc boundary %d", k);
  HIP_OK(hipMemcpy(h_out, packed, sizeof(h_out), hipMemcpyDeviceToHost));
  for (int i = 0; i < T; ++i) CHECK(h_out[i] == want_tokens[i], "pack_noalloc packed[%d] = %c", i, (char)h_out[i]);
  HIP_OK(hipMemcpy(h_out, zig, sizeof(h_out), hipMemcpyDeviceToHost));
  for (int i = 0; i < T; ++i) CHECK(h_out[i] == want_zigzag[i], "zigzag[%d] = %c", i, (char)h_out[i]);
  HIP_OK(hipMemcpy(h_out, back, sizeof(h_out), hipMemcpyDeviceToHost));
  for (int i = 0; i < T; ++i) CHECK(h_out[i] == want_tokens[i], "round trip[%d] = %c", i, (char)h_out[i]);
  HIP_OK(hipMemcpy(h_mask, mask, sizeof(h_mask), hipMemcpyDeviceToHost));
  int valid = 0;
  for (int i = 0; i < T; ++i) {
    CHECK(h_mask[i] == want_mask[i], "valid mask[%d] = %d", i, h_mask[i]);
    valid += h_mask[i];
  }
  CHECK(valid == 13, "valid tokens %d", valid);

  int32_t n_runs = 0, split[CP * CP];
  int32_t by_src[64 * 3], by_dst[64 * 3];
  CHECK(thd_route_copy_out(route, stream, &n_runs, 64, by_src, by_dst, split) == THD_OK, "copy out");
  for (int i = 0; i < CP * CP; ++i) CHECK(split[i] == 4, "split[%d] = %d", i, split[i]);

  thd_route_destroy(route);
  hipFree(rows); hipFree(packed); hipFree(zig); hipFree(back); hipFree(shifted);
  hipFree(mask); hipFree(cu); hipFree(cu_pad); hipFree(status); hipFree(ws);
  HIP_OK(hipStreamDestroy(stream));
  return failures;
}

int main(int argc, char** argv) {
  const int gpu = argc > 1 && strcmp(argv[1], "gpu") == 0;
  int rc = host_checks();
  if (rc == 0 && gpu) rc = gpu_example();
  printf("%s (%d failed checks)\n", rc == 0 ? "OK" : "FAILED", failures);
  return rc == 0 ? 0 : 1;
}
