/* Host-side exercise of the C ABI for sanitizer builds (no GPU needed):
 * every entry point's argument validation, the planning queries over a grid
 * of shapes and CU caps, the planner override's parser with well-formed and
 * malformed strings, and the error-message buffer.  Exits non-zero when a
 * call returns something other than an expected status. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "dg.h"

#define P16 ((void*)0x10000)
#define P4 ((void*)0x10004)

static int failures = 0;
static void expect(int got, int want, const char* what) {
  if (got != want) {
    fprintf(stderr, "%s: got %d want %d (%s)\n", what, got, want, dg_get_last_error());
    ++failures;
  }
}
/* on a host without a device, validation passes and the device check fails */
static void expect_ok_or_nodev(int got, const char* what) {
  if (got != DG_OK && got != DG_ERR_DEVICE) {
    fprintf(stderr, "%s: got %d (%s)\n", what, got, dg_get_last_error());
    ++failures;
  }
}

int main(void) {
  void* s = NULL;
  const int64_t Ms[] = {0, 1, 63, 64, 100, 128, 129, 300, 4096, 262400, (int64_t)1 << 31};
  const int64_t NKs[][2] = {{16, 128}, {2112, 7168}, {24576, 1536}, {32768, 512}, {7168, 16384}, {4096, 7168},
                            {7168, 2048}, {400, 640}, {1 << 19, 8192}, {16, 1 << 24}, {100, 128}, {128, 100}};
  const char* forces[] = {NULL, "kernel=wide", "kernel=persistent", "chunk_rows=256", "chunk_rows=1,kernel=wide",
                          "skinny=64x16x7x8", "skinny=128x32x16x4", "skinny=64x16x7", "skinny=99x16x2x4",
                          "skinny=64x16x-3x4", "chunk_rows=-5", "kernel=", ",,,", "garbage=1,chunk_rows=99999999999",
                          "skinny=128x32x1000000x4,chunk_rows=512"};
  const int caps[] = {0, 1, 3, 7, 256, 100000};
  for (size_t f = 0; f < sizeof(forces) / sizeof(forces[0]); ++f) {
    if (forces[f]) setenv("DG_FORCE_CONFIG", forces[f], 1);
    else unsetenv("DG_FORCE_CONFIG");
    for (size_t c = 0; c < sizeof(caps) / sizeof(caps[0]); ++c) {
      dg_set_num_cus(caps[c]);
      for (size_t m = 0; m < sizeof(Ms) / sizeof(Ms[0]); ++m)
        for (size_t k = 0; k < sizeof(NKs) / sizeof(NKs[0]); ++k) {
          const int64_t M = Ms[m], N = NKs[k][0], K = NKs[k][1];
          for (int op = -1; op <= 6; ++op) {
            const char* d = dg_describe_plan(op, M, N, K, 8);
            if (!d) ++failures;
            (void)dg_get_workspace_size(op, M, N, K, 8);
          }
          expect_ok_or_nodev(dg_fp8_gemm_nt(P16, P16, P16, P16, P16, 64, 2112, 7168, NULL, 0, s), "gemm");
          (void)dg_fp8_gemm_nt(P16, P16, P16, P16, P16, M, N, K, P16, 4096, s);
          (void)dg_fp8_gemm_nt_acc(P16, P16, P16, P16, NULL, P16, M, N, K, NULL, 0, s);
          (void)dg_fp8_gemm_nt_ue8m0(P16, P16, P16, P16, P16, M, N, K, NULL, 0, s);
          (void)dg_bf16_gemm_nt(P16, P16, P16, M, N, K, NULL, 0, s);
          (void)dg_fp8_gemm_nt_noalloc(P16, P16, P16, P16, P16, M, N, K, s);
          (void)dg_m_grouped_fp8_gemm_nt_contiguous(P16, P16, P16, P16, P16, P16, M, N, K, 8, NULL, 0, s);
          (void)dg_m_grouped_fp8_gemm_nt_contiguous_ue8m0(P16, P16, P16, P16, P16, P16, M, N, K, 8, NULL, 0, s);
          (void)dg_m_grouped_fp8_gemm_nt_masked(P16, P16, P16, P16, P16, P16, 8, M, N, K, 0, NULL, 0, s);
          (void)dg_m_grouped_fp8_gemm_nt_masked_ue8m0(P16, P16, P16, P16, P16, P16, 8, M, N, K, 0, NULL, 0, s);
          (void)dg_k_grouped_fp8_gemm_nt_contiguous(P16, P16, P16, P16, NULL, P16, P16, 8, M, N, K, NULL, 0, s);
          (void)dg_quant_1x128(P16, P16, P16, 1, M, K, s);
          (void)dg_quant_128x128(P16, P16, P16, 1, N, K, s);
          (void)dg_quant_1x128_ue8m0(P16, P16, P16, 2, M, K, s);
          (void)dg_quant_128x128_ue8m0(P16, P16, P16, 2, N, K, s);
          if (strlen(dg_get_last_error()) > 511) ++failures;
        }
    }
  }
  unsetenv("DG_FORCE_CONFIG");
  dg_set_num_cus(0);
  /* a few exact statuses */
  expect(dg_fp8_gemm_nt(P16, P16, P16, P16, P16, 64, 2112, 7000, NULL, 0, s), DG_ERR_SHAPE, "K % 128");
  expect(dg_fp8_gemm_nt(NULL, P16, P16, P16, P16, 64, 2112, 7168, NULL, 0, s), DG_ERR_INVALID_ARG, "null A");
  expect(dg_fp8_gemm_nt(P16, P16, P16, P16, P16, 64, 2112, 7168, P4, 64, s), DG_ERR_WORKSPACE, "workspace");
  expect(dg_m_grouped_fp8_gemm_nt_masked(P16, P16, P16, P16, P16, P16, 1025, 8, 128, 256, 0, NULL, 0, s),
         DG_ERR_SHAPE, "G > 1024");
  expect(dg_fp8_gemm_nt(NULL, NULL, NULL, NULL, NULL, 0, 2112, 7168, NULL, 0, s), DG_OK, "M = 0");
  if (dg_get_m_alignment_for_contiguous_layout() != 128) ++failures;
  if (strncmp(dg_version(), "dg-mi355x", 9) != 0) ++failures;
  printf("abi driver: %d failures\n", failures);
  return failures ? 1 : 0;
}
