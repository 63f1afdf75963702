/* Host-side sanitizer driver for the C ABI (no GPU): calls every entry point
 * of include/swinattn.h with the argument errors the ABI documents and with
 * calls that reach the HIP runtime, built together with a copy of the
 * library whose host code carries AddressSanitizer and UndefinedBehavior-
 * Sanitizer instrumentation.  Exits 0 when every status is as documented;
 * a sanitizer report aborts it.  Placeholder pointers are aligned and never
 * dereferenced: every call with them fails its argument checks (or, on a
 * machine without a GPU, the runtime's device query) before any device work. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "../../include/swinattn.h"

static int failures = 0;

static void expect(int got, int want, const char* what) {
  if (got != want) {
    printf("FAIL %s: status %d, expected %d\n", what, got, want);
    ++failures;
  }
}

/* the call's status is one of those allowed without a GPU */
static void expect_no_gpu(int got, const char* what) {
  if (got != SWIN_OK && got != SWIN_ERR_HIP) {
    printf("FAIL %s: status %d\n", what, got);
    ++failures;
  }
}

int main(void) {
  void* A = (void*)(uintptr_t)(1u << 20);
  void* Bp = (void*)(uintptr_t)(2u << 20);
  void* C = (void*)(uintptr_t)(3u << 20);
  void* D = (void*)(uintptr_t)(4u << 20);
  void* E = (void*)(uintptr_t)(5u << 20);
  const int I = SWIN_ERR_INVALID_ARG, U = SWIN_ERR_UNSUPPORTED;

  for (int s = -6; s <= 2; ++s) {
    const char* str = swin_wattn_status_string(s);
    if (!str || strlen(str) == 0) {
      printf("FAIL status string %d\n", s);
      ++failures;
    }
  }
  /* forward, bf16 and fp32 */
  expect(swin_wattn_fwd(NULL, C, Bp, 2, 14, 14, 2, 32, 7, 3, NULL), I, "fwd null qkv");
  expect(swin_wattn_fwd((char*)A + 8, C, Bp, 2, 14, 14, 2, 32, 7, 3, NULL), I, "fwd misaligned");
  expect(swin_wattn_fwd(A, C, Bp, 2, 15, 14, 2, 32, 7, 3, NULL), I, "fwd H % window");
  expect(swin_wattn_fwd(A, C, Bp, 2, 14, 14, 2, 32, 7, 7, NULL), I, "fwd shift");
  expect(swin_wattn_fwd(A, C, A, 2, 14, 14, 2, 32, 7, 3, NULL), I, "fwd overlap");
  expect(swin_wattn_fwd(A, C, Bp, 2, 14, 14, 2, 64, 7, 3, NULL), U, "fwd head_dim");
  expect(swin_wattn_fwd(A, C, Bp, 2, 28, 28, 2, 32, 14, 0, NULL), U, "fwd window 14");
  expect(swin_wattn_fwd(A, C, Bp, 0, 14, 14, 2, 32, 7, 3, NULL), SWIN_OK, "fwd B=0");
  expect(swin_wattn_fwd_f32(A, C, Bp, 2, 24, 24, 78, 32, 12, 0, NULL), U, "fwd fp32 tables");
  expect(swin_wattn_fwd_f32(NULL, C, Bp, 2, 14, 14, 2, 32, 7, 3, NULL), I, "fwd fp32 null");
  expect(swin_wattn_fwd_i8(NULL, 0.03f, 0.03f, 0.03f, 0.f, C, Bp, 2, 14, 14, 2, 32, 7, 3, NULL), I,
         "fwd int8 null");
  expect(swin_linear_i8_fwd(A, 0.03f, Bp, NULL, NULL, NULL, NULL, C, 64, 192, 576, NULL), I,
         "linear int8 no weight scales");
  expect(swin_linear_i8_fwd(A, 0.03f, Bp, (const float*)C, NULL, A, (const float*)C, Bp, 64, 192,
                            576, NULL), I, "linear int8 residual with int8 output");
  expect(swin_linear_i8_fwd(A, 0.03f, Bp, (const float*)C, NULL, NULL, NULL, Bp, 64, 800, 576,
                            NULL), U, "linear int8 K");
  expect(swin_linear_i8_pack_weight(A, A, 576, 192, NULL), I, "linear int8 pack overlap");
  expect(swin_wattn_fwd_i8(A, 0.03f, 0.03f, 0.03f, 0.f, C, A, 2, 14, 14, 2, 32, 7, 3, NULL), I,
         "fwd int8 overlap");
  expect(swin_wattn_fwd_i8(A, 0.0f, 0.03f, 0.03f, 0.f, C, Bp, 2, 14, 14, 2, 32, 7, 3, NULL), I,
         "fwd int8 zero scale");
  expect(swin_wattn_fwd_i8(A, 1e-20f, 1e-20f, 1.f, 0.f, C, Bp, 2, 14, 14, 2, 32, 7, 3, NULL), I,
         "fwd int8 score scale");
  expect(swin_wattn_fwd_i8(A, 0.03f, 0.03f, 0.03f, 0.f, C, Bp, 2, 14, 14, 2, 64, 7, 3, NULL), U,
         "fwd int8 head_dim");
  expect(swin_wattn_fwd_i8(A, 0.03f, 0.03f, 0.03f, 0.f, C, Bp, 0, 14, 14, 2, 32, 7, 3, NULL), SWIN_OK,
         "fwd int8 B=0");
  /* backward */
  expect(swin_wattn_bwd(A, C, D, NULL, E, 2, 14, 14, 2, 32, 7, 3, NULL), I, "bwd null dqkv");
  expect(swin_wattn_bwd(A, C, D, A, E, 2, 14, 14, 2, 32, 7, 3, NULL), I, "bwd overlap");
  expect(swin_wattn_bwd(A, C, D, Bp, E, 2, 14, 14, 2, 32, 13, 0, NULL), I, "bwd H % window");
  expect(swin_wattn_bwd(A, C, D, Bp, E, 2, 28, 28, 2, 32, 14, 0, NULL), U, "bwd window 14");
  /* linear layers */
  expect(swin_linear_fwd(NULL, Bp, NULL, NULL, C, 64, 192, 576, NULL), I, "linear null x");
  expect(swin_linear_fwd(A, Bp, NULL, NULL, C, 64, 200, 576, NULL), I, "linear K % 32");
  expect(swin_linear_fwd(A, Bp, NULL, NULL, C, 64, 416, 576, NULL), U, "linear K > 384");
  expect(swin_linear_fwd(A, Bp, NULL, NULL, C, 0, 192, 576, NULL), SWIN_OK, "linear T=0");
  expect(swin_linear_pack_weight(A, A, 576, 192, NULL), I, "pack overlap");
  expect(swin_ln_linear_pack_weight(A, C, D, NULL, Bp, NULL, 576, 192, NULL), I, "ln pack null");
  expect(swin_ln_linear_fwd(A, Bp, NULL, 1e-5f, C, 64, 192, 576, NULL), I, "ln null consts");
  expect(swin_ln_linear_fwd(A, Bp, D, -1.f, C, 64, 192, 576, NULL), I, "ln eps");
  /* fused layer norm + QKV + attention */
  expect(swin_ln_qkv_wattn_fwd(NULL, Bp, C, 1e-5f, D, E, 2, 14, 14, 6, 32, 7, 3, NULL), I,
         "fused null x");
  expect(swin_ln_qkv_wattn_fwd(A, Bp, C, 1e-5f, D, A, 2, 14, 14, 6, 32, 7, 3, NULL), I,
         "fused overlap");
  expect(swin_ln_qkv_wattn_fwd(A, Bp, C, 1e-5f, D, E, 2, 14, 14, 8, 32, 7, 3, NULL), U,
         "fused C > 192");
  expect(swin_ln_qkv_wattn_fwd(A, Bp, C, 1e-5f, D, E, 0, 14, 14, 6, 32, 7, 3, NULL), SWIN_OK,
         "fused B=0");
  /* setup cache and copies */
  expect(swin_wattn_precompute(14, 14, 7, 7, NULL), I, "precompute shift");
  expect(swin_wattn_copy_index(14, 14, 7, 3, NULL, NULL), I, "copy null");
  expect_no_gpu(swin_wattn_precompute(14, 14, 7, 3, NULL), "precompute");
  const int st = swin_wattn_copy_mask(14, 14, 7, 3, (float*)A, NULL);
  if (st != SWIN_ERR_NOT_PREPARED && st != SWIN_ERR_HIP) {
    printf("FAIL copy without a prepared key: %d\n", st);
    ++failures;
  }
  expect_no_gpu(swin_wattn_release(), "release");
  printf("%s (%d failures)\n", failures ? "FAILED" : "clean", failures);
  return failures ? 1 : 0;
}
