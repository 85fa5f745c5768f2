/* Host-side checks of the C ABI, built and run under AddressSanitizer by
 * tests/test_host_sanitizer.py (CPU only).  Only calls that do no device work
 * are made: version and error strings, argument checks, workspace sizing,
 * the launch plan, and the forward's argument errors, which are all reported
 * before anything is enqueued.  Exit status 0 when every expectation holds. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "lapattn.h"

static int failures = 0;

#define EXPECT(cond, ...)                                  \
  do {                                                     \
    if (!(cond)) {                                         \
      ++failures;                                          \
      fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
      fprintf(stderr, __VA_ARGS__);                        \
      fprintf(stderr, "\n");                               \
    }                                                      \
  } while (0)

static lapattn_desc_t desc(int B, int H, int gh, int gw, int d, int ph, int pw, int kernel,
                           int dtype) {
  lapattn_desc_t x;
  memset(&x, 0, sizeof x);
  x.B = B;
  x.H = H;
  x.grid_h = gh;
  x.grid_w = gw;
  x.d = d;
  x.pool_h = ph;
  x.pool_w = pw;
  x.kernel = kernel;
  x.dtype = dtype;
  x.flags = 0;
  return x;
}

int main(void) {
  EXPECT(lapattn_version() >= 1, "version %d", lapattn_version());
  for (int s = 0; s >= -11; --s) {
    const char* t = lapattn_strerror(s);
    EXPECT(t != NULL && strlen(t) > 0, "strerror(%d)", s);
  }

  /* the workloads' shapes are valid and have a workspace */
  const lapattn_desc_t ok[] = {
      desc(1, 1, 14, 14, 32, 2, 2, LAPATTN_KERNEL_LAPLACIAN, LAPATTN_F32),
      desc(8, 1, 56, 56, 64, 8, 8, LAPATTN_KERNEL_LAPLACIAN, LAPATTN_F32),
      desc(32, 5, 28, 28, 64, 4, 4, LAPATTN_KERNEL_LAPLACIAN, LAPATTN_BF16),
      desc(1, 2, 128, 128, 64, 16, 16, LAPATTN_KERNEL_LAPLACIAN, LAPATTN_F32),
      desc(16, 2, 56, 56, 64, 8, 8, LAPATTN_KERNEL_GAUSSIAN, LAPATTN_F32),
      desc(1, 1, 4, 4, 16, 1, 1, LAPATTN_KERNEL_LAPLACIAN, LAPATTN_F32),
      desc(300, 1, 10, 14, 32, 2, 2, LAPATTN_KERNEL_GAUSSIAN, LAPATTN_BF16),
  };
  for (size_t i = 0; i < sizeof ok / sizeof ok[0]; ++i) {
    EXPECT(lapattn_check(&ok[i], 16.f, 1e-3f, 20) == LAPATTN_OK, "check of valid shape %zu", i);
    const size_t ws = lapattn_workspace_bytes(&ok[i]);
    EXPECT(ws > 0, "workspace of shape %zu", i);
    EXPECT(lapattn_status_offset(&ok[i]) + 4 <= ws, "status word inside the workspace (%zu)", i);
    EXPECT(lapattn_backward_workspace_bytes(&ok[i], 20) > 0, "backward workspace %zu", i);
    const int mask = lapattn_launches(&ok[i], 0);
    EXPECT(mask > 0 && (mask & (1 << LAPATTN_STAGE_POOL)) && (mask & (1 << LAPATTN_STAGE_MAIN)),
           "launch mask %d of shape %zu", mask, i);
    EXPECT(lapattn_launches(&ok[i], 1) & (1 << LAPATTN_STAGE_OUT), "Q = K uses the output launch (%zu)", i);
  }
  EXPECT(lapattn_block_workspace_bytes(&ok[1], 64) > 0, "block workspace");

  /* argument errors */
  const lapattn_desc_t base = ok[1];
  lapattn_desc_t bad;
  EXPECT(lapattn_check(NULL, 16.f, 1e-3f, 20) == LAPATTN_ERR_NULL, "NULL descriptor");
  bad = base; bad.B = 0;
  EXPECT(lapattn_check(&bad, 16.f, 1e-3f, 20) == LAPATTN_ERR_SHAPE, "B = 0");
  bad = base; bad.d = 48;
  EXPECT(lapattn_check(&bad, 16.f, 1e-3f, 20) == LAPATTN_ERR_SHAPE, "d = 48");
  bad = base; bad.pool_h = 5;
  EXPECT(lapattn_check(&bad, 16.f, 1e-3f, 20) == LAPATTN_ERR_SHAPE, "pool does not divide the grid");
  bad = base; bad.pool_h = 7; bad.pool_w = 7;
  EXPECT(lapattn_check(&bad, 16.f, 1e-3f, 20) == LAPATTN_OK, "m = 64, the largest");
  bad = base; bad.pool_h = 4; bad.pool_w = 8;
  EXPECT(lapattn_check(&bad, 16.f, 1e-3f, 20) == LAPATTN_ERR_M_TOO_LARGE, "m = 98");
  EXPECT(lapattn_check(&base, 0.f, 1e-3f, 20) == LAPATTN_ERR_PARAM, "lambda = 0");
  EXPECT(lapattn_check(&base, NAN, 1e-3f, 20) == LAPATTN_ERR_PARAM, "lambda NaN");
  EXPECT(lapattn_check(&base, 16.f, -1e-3f, 20) == LAPATTN_ERR_PARAM, "eps < 0");
  EXPECT(lapattn_check(&base, 16.f, 1e-3f, 65) == LAPATTN_ERR_PARAM, "iters = 65");
  EXPECT(lapattn_check(&base, 16.f, 1e-3f, -1) == LAPATTN_ERR_PARAM, "iters = -1");
  bad = base; bad.kernel = 2;
  EXPECT(lapattn_check(&bad, 16.f, 1e-3f, 20) == LAPATTN_ERR_PARAM, "kernel 2");
  bad = base; bad.flags = 4u;
  EXPECT(lapattn_check(&bad, 16.f, 1e-3f, 20) == LAPATTN_ERR_PARAM, "unknown flag");
  bad = base; bad.dtype = 7;
  EXPECT(lapattn_check(&bad, 16.f, 1e-3f, 20) == LAPATTN_ERR_DTYPE, "dtype 7");
  bad = base; bad.B = 0;
  EXPECT(lapattn_workspace_bytes(&bad) == 0, "no workspace for an invalid shape");
  EXPECT(lapattn_workspace_bytes(NULL) == 0, "no workspace for NULL");

  /* the forward's argument errors, reported before anything is enqueued
   * (these addresses are never dereferenced) */
  const size_t ws = lapattn_workspace_bytes(&base);
  const size_t io = (size_t)8 * 3136 * 64 * 4;
  char* const q = (char*)(uintptr_t)0x100000000ull;
  char* const k = q + io;
  char* const v = k + io;
  char* const o = v + io;
  char* const w = o + io + 4096;
  EXPECT(lapattn_forward(&base, NULL, k, v, 16.f, 1e-3f, 20, o, w, ws, NULL) == LAPATTN_ERR_NULL,
         "NULL q");
  EXPECT(lapattn_forward(&base, q, k, v, 16.f, 1e-3f, 20, NULL, w, ws, NULL) == LAPATTN_ERR_NULL,
         "NULL out");
  EXPECT(lapattn_forward(&base, q + 4, k, v, 16.f, 1e-3f, 20, o, w, ws, NULL) == LAPATTN_ERR_ALIGN,
         "misaligned q");
  EXPECT(lapattn_forward(&base, q, k, v, 16.f, 1e-3f, 20, o, w, ws - 256, NULL) ==
             LAPATTN_ERR_WORKSPACE,
         "workspace too small");
  EXPECT(lapattn_forward(&base, q, k, v, 16.f, 1e-3f, 20, q + 256, w, ws, NULL) == LAPATTN_ERR_ALIAS,
         "out overlaps q");
  EXPECT(lapattn_forward(&base, q, k, v, 16.f, 1e-3f, 20, w, w, ws, NULL) == LAPATTN_ERR_ALIAS,
         "out overlaps the workspace");
  EXPECT(lapattn_forward(&base, q, k, v, -1.f, 1e-3f, 20, o, w, ws, NULL) == LAPATTN_ERR_PARAM,
         "lambda < 0");
  EXPECT(lapattn_forward_noalloc(&base, q, k, v, 16.f, 1e-3f, 70, o, NULL, NULL) == LAPATTN_ERR_PARAM,
         "noalloc: iters = 70");

  if (failures) {
    fprintf(stderr, "%d failure(s)\n", failures);
    return 1;
  }
  printf("host ABI checks passed\n");
  return 0;
}
