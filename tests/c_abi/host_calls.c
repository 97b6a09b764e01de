/* A plain C99 caller of the library's host-only entry points: the header
 * compiles as C, the library links and loads, and the rules the header
 * states hold when called from C (no GPU is touched). Exit status 0 on
 * success; a failed check prints its line. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "mhc_coeff_bwd.h"
#include "mhc_h_aggregate.h"

#define CHECK(cond)                                              \
  do {                                                           \
    if (!(cond)) {                                               \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      return 1;                                                  \
    }                                                            \
  } while (0)

int main(void) {
  const int64_t T = 1024, H = 7168;
  /* Fake, far-apart, 256-byte-aligned device addresses: the host-only calls
   * use pointers only as numbers. */
  const uintptr_t base = (uintptr_t)1 << 34;
  const uint16_t* residual = (const uint16_t*)base;
  const float* pre = (const float*)(base + ((uintptr_t)1 << 30));
  const uint16_t* grad_out = (const uint16_t*)(base + ((uintptr_t)2 << 30));
  uint16_t* grad_residual = (uint16_t*)(base + ((uintptr_t)3 << 30));
  float* grad_pre = (float*)(base + ((uintptr_t)4 << 30));
  uint16_t* out = (uint16_t*)(base + ((uintptr_t)5 << 30));
  mhc_launch plan, ov;
  int64_t blocks = 0;

  CHECK(mhc_abi_version() == MHC_ABI_VERSION);
  CHECK(strcmp(mhc_status_string(MHC_ERROR_ALIASING), "MHC_ERROR_ALIASING") == 0);

  CHECK(mhc_h_aggregate_validate_fwd(residual, pre, out, T, H) == MHC_SUCCESS);
  CHECK(mhc_h_aggregate_validate_fwd(residual, pre, (uint16_t*)residual, T, H) ==
        MHC_ERROR_ALIASING);
  CHECK(strlen(mhc_last_error_message()) > 0);
  CHECK(mhc_h_aggregate_validate_fwd(residual, pre, out, -1, H) == MHC_ERROR_INVALID_VALUE);
  CHECK(mhc_h_aggregate_validate_bwd(residual, pre, grad_out, grad_residual, grad_pre, T, H) ==
        MHC_SUCCESS);

  CHECK(mhc_h_aggregate_plan_fwd(residual, pre, out, T, H, NULL, &plan, &blocks) == MHC_SUCCESS);
  CHECK(plan.block_threads == 64 && plan.vec_width == 8 && blocks == T * (H / 8 / 64));

  CHECK(mhc_h_aggregate_plan_bwd(residual, pre, grad_out, grad_residual, grad_pre, T, H, NULL,
                                 &plan, &blocks) == MHC_SUCCESS);
  CHECK(plan.layout == MHC_BWD_ROWS && plan.block_threads == 256 && blocks == T);

  memset(&ov, 0, sizeof ov);
  ov.layout = MHC_BWD_SPLIT;
  CHECK(mhc_h_aggregate_plan_bwd(residual, pre, grad_out, grad_residual, grad_pre, T, H, &ov,
                                 &plan, &blocks) == MHC_SUCCESS);
  CHECK(plan.layout == MHC_BWD_SPLIT && plan.streams_per_block == 4 && blocks == T);
  CHECK(plan.wave_priority == MHC_PRIO_FLAT);

  /* issue priority: the policy's choice is reported, an override is honoured
     within the row layout and refused outside it */
  memset(&ov, 0, sizeof ov);
  ov.wave_priority = T * MHC_HC <= 16 * 256 ? MHC_PRIO_FLAT : MHC_PRIO_PROGRESS;
  CHECK(mhc_h_aggregate_plan_bwd(residual, pre, grad_out, grad_residual, grad_pre, T, H, &ov,
                                 &plan, &blocks) == MHC_SUCCESS);
  CHECK(plan.layout == MHC_BWD_ROWS && plan.wave_priority == ov.wave_priority);
  ov.wave_priority = 3;
  CHECK(mhc_h_aggregate_plan_bwd(residual, pre, grad_out, grad_residual, grad_pre, T, H, &ov,
                                 &plan, &blocks) == MHC_ERROR_INVALID_VALUE);
  ov.wave_priority = MHC_PRIO_PROGRESS;
  ov.layout = MHC_BWD_SPLIT;
  CHECK(mhc_h_aggregate_plan_bwd(residual, pre, grad_out, grad_residual, grad_pre, T, H, &ov,
                                 &plan, &blocks) == MHC_ERROR_INVALID_VALUE);
  memset(&ov, 0, sizeof ov);
  ov.wave_priority = MHC_PRIO_FLAT;
  CHECK(mhc_h_aggregate_plan_fwd(residual, pre, out, T, H, &ov, &plan, &blocks) ==
        MHC_ERROR_INVALID_VALUE);

  CHECK(mhc_h_aggregate_plan_bwd_n(residual, pre, grad_out, grad_residual, grad_pre, T, 3, H, 0,
                                   NULL, &plan, &blocks) == MHC_ERROR_INVALID_VALUE);
  /* compute entry points reject bad arguments before any HIP call */
  CHECK(mhc_h_aggregate_fwd(residual, pre, (uint16_t*)residual, T, H, NULL) ==
        MHC_ERROR_ALIASING);
  CHECK(mhc_h_aggregate_bwd(NULL, NULL, NULL, NULL, NULL, 0, H, NULL) == MHC_SUCCESS);

  /* the coefficient backward epilogue's library */
  {
    const int64_t R = 8192;
    const int32_t n = 4;
    const uintptr_t cb = (uintptr_t)1 << 40;
    const uintptr_t step = (uintptr_t)1 << 24; /* 16 MiB apart */
    const float* mix = (const float*)cb;
    const float* cpre = (const float*)(cb + 1 * step);
    const float* post = (const float*)(cb + 2 * step);
    const float* gpre = (const float*)(cb + 3 * step);
    const float* gpost = (const float*)(cb + 4 * step);
    const float* gres = (const float*)(cb + 5 * step);
    const float* alpha = (const float*)(cb + 6 * step);
    float* gmix = (float*)(cb + 7 * step);
    float* gb = (float*)(cb + 8 * step);
    float* ga = (float*)(cb + 9 * step);
    void* ws = (void*)(cb + 10 * step);
    const int64_t ws_bytes = mhc_coeff_bwd_workspace_bytes(R, n);
    CHECK(mhc_coeff_abi_version() == MHC_COEFF_ABI_VERSION);
    CHECK(ws_bytes == 256 + 27 * (R / MHC_COEFF_CHUNK) * 4);
    CHECK(mhc_coeff_bwd_workspace_bytes(R, 3) == -1);
    CHECK(mhc_coeff_bwd_plan(2 * R, n, 0) == 1 && mhc_coeff_bwd_plan(2 * R + 1, n, 0) == 2);
    CHECK(mhc_coeff_bwd_validate(mix, cpre, post, gpre, gpost, gres, alpha, 2.0f, gmix, gb, ga,
                                 ws, ws_bytes, R, n) == MHC_SUCCESS);
    CHECK(mhc_coeff_bwd_validate(mix, cpre, post, gpre, gpost, gres, alpha, 2.0f, (float*)mix,
                                 gb, ga, ws, ws_bytes, R, n) == MHC_ERROR_ALIASING);
    CHECK(mhc_coeff_bwd_validate(mix, cpre, post, gpre, gpost, gres, alpha, 0.0f, gmix, gb, ga,
                                 ws, ws_bytes, R, n) == MHC_ERROR_INVALID_VALUE);
    CHECK(strlen(mhc_coeff_last_error_message()) > 0);
    CHECK(mhc_coeff_bwd(mix, cpre, post, gpre, gpost, gres, alpha, 2.0f, gmix, gb, ga, ws,
                        ws_bytes - 4, R, n, 0, NULL, NULL, NULL) == MHC_ERROR_INVALID_VALUE);
    /* 16-bit row tensors need 2-byte alignment only; an unknown format is refused */
    CHECK(mhc_coeff_bwd_validate_ex(mix, (const char*)cpre + 2, post, gpre, gpost, gres, alpha,
                                    2.0f, gmix, gb, ga, ws, ws_bytes, R, n, MHC_COEFF_BF16) ==
          MHC_SUCCESS);
    CHECK(mhc_coeff_bwd_validate_ex(mix, cpre, post, gpre, gpost, gres, alpha, 2.0f, gmix, gb,
                                    ga, ws, ws_bytes, R, n, 7) == MHC_ERROR_INVALID_VALUE);
    /* the entry point that allocates nothing refuses calls past its array */
    CHECK(mhc_coeff_bwd_noalloc(mix, cpre, post, gpre, gpost, gres, alpha, 2.0f, gmix, gb, ga,
                                MHC_COEFF_SCRATCH_BYTES, n, 0, NULL, NULL, NULL) ==
          MHC_ERROR_INVALID_VALUE);
  }
  printf("c abi ok\n");
  return 0;
}
