/* A plain C99 program that runs both libraries on the GPU through their C
 * ABIs, with device memory from the HIP runtime and the null stream: no
 * Python, no torch. Usage: gpu_calls DIR T H R
 *   reads  DIR/residual.bin (bf16 bits, T*4*H), DIR/pre.bin (fp32, T*4),
 *          DIR/grad_out.bin (bf16 bits, T*H) and the coefficient epilogue's
 *          inputs DIR/c_mix.bin, c_pre.bin, c_post.bin, c_grad_pre.bin,
 *          c_grad_post.bin, c_grad_res.bin, c_alpha.bin (fp32, R rows, n = 4);
 *          and the same six row tensors as bf16 bits in DIR/c16_*.bin;
 *   writes DIR/out.bin, grad_residual.bin, grad_pre.bin, c_grad_mix.bin,
 *          c_grad_b.bin, c_grad_alpha.bin (workspace entry point), the same
 *          from the entry point that allocates nothing (c_na_*.bin), and the
 *          bf16 call's c16_grad_mix.bin, c16_grad_b.bin, c16_grad_alpha.bin.
 * Exit status 0 on success; a failure prints what failed. */
#define __HIP_PLATFORM_AMD__
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "mhc_coeff_bwd.h"
#include "mhc_h_aggregate.h"

#define HIP_CHECK(call)                                                        \
  do {                                                                         \
    hipError_t e_ = (call);                                                    \
    if (e_ != hipSuccess) {                                                    \
      fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));        \
      return 1;                                                                \
    }                                                                          \
  } while (0)

static char path_buf[4096];

static const char* path(const char* dir, const char* name) {
  snprintf(path_buf, sizeof path_buf, "%s/%s", dir, name);
  return path_buf;
}

/* Reads `bytes` bytes of DIR/name into a new device buffer. */
static int upload(const char* dir, const char* name, size_t bytes, void** dev) {
  FILE* f = fopen(path(dir, name), "rb");
  void* host = malloc(bytes ? bytes : 1);
  if (!f || !host || fread(host, 1, bytes, f) != bytes) {
    fprintf(stderr, "cannot read %s\n", path(dir, name));
    return 1;
  }
  fclose(f);
  HIP_CHECK(hipMalloc(dev, bytes ? bytes : 1));
  HIP_CHECK(hipMemcpy(*dev, host, bytes, hipMemcpyHostToDevice));
  free(host);
  return 0;
}

/* Writes `bytes` bytes of a device buffer to DIR/name. */
static int download(const char* dir, const char* name, const void* dev, size_t bytes) {
  void* host = malloc(bytes ? bytes : 1);
  if (!host) return 1;
  HIP_CHECK(hipMemcpy(host, dev, bytes, hipMemcpyDeviceToHost));
  FILE* f = fopen(path(dir, name), "wb");
  if (!f || fwrite(host, 1, bytes, f) != bytes) {
    fprintf(stderr, "cannot write %s\n", path(dir, name));
    return 1;
  }
  fclose(f);
  free(host);
  return 0;
}

#define MHC_CHECK(call)                                                        \
  do {                                                                         \
    mhc_status s_ = (call);                                                    \
    if (s_ != MHC_SUCCESS) {                                                   \
      fprintf(stderr, "%s failed: %s\n", #call, mhc_status_string(s_));        \
      return 1;                                                                \
    }                                                                          \
  } while (0)

int main(int argc, char** argv) {
  if (argc != 5) {
    fprintf(stderr, "usage: gpu_calls DIR T H R\n");
    return 2;
  }
  const char* dir = argv[1];
  const int64_t T = atoll(argv[2]), H = atoll(argv[3]), R = atoll(argv[4]);
  const int32_t n = 4;
  const int64_t m = 2 * n + n * n;
  void *residual, *pre, *grad_out, *out, *grad_residual, *grad_pre;
  if (upload(dir, "residual.bin", (size_t)(T * 4 * H * 2), &residual) ||
      upload(dir, "pre.bin", (size_t)(T * 4 * 4), &pre) ||
      upload(dir, "grad_out.bin", (size_t)(T * H * 2), &grad_out))
    return 1;
  HIP_CHECK(hipMalloc(&out, (size_t)(T * H * 2)));
  HIP_CHECK(hipMalloc(&grad_residual, (size_t)(T * 4 * H * 2)));
  HIP_CHECK(hipMalloc(&grad_pre, (size_t)(T * 4 * 4)));
  MHC_CHECK(mhc_h_aggregate_fwd(residual, pre, out, T, H, NULL));
  MHC_CHECK(mhc_h_aggregate_bwd(residual, pre, grad_out, grad_residual, grad_pre, T, H, NULL));
  HIP_CHECK(hipDeviceSynchronize());
  if (download(dir, "out.bin", out, (size_t)(T * H * 2)) ||
      download(dir, "grad_residual.bin", grad_residual, (size_t)(T * 4 * H * 2)) ||
      download(dir, "grad_pre.bin", grad_pre, (size_t)(T * 4 * 4)))
    return 1;

  void *mix, *cpre, *post, *gpre, *gpost, *gres, *alpha, *gmix, *gb, *ga, *ws;
  if (upload(dir, "c_mix.bin", (size_t)(R * m * 4), &mix) ||
      upload(dir, "c_pre.bin", (size_t)(R * n * 4), &cpre) ||
      upload(dir, "c_post.bin", (size_t)(R * n * 4), &post) ||
      upload(dir, "c_grad_pre.bin", (size_t)(R * n * 4), &gpre) ||
      upload(dir, "c_grad_post.bin", (size_t)(R * n * 4), &gpost) ||
      upload(dir, "c_grad_res.bin", (size_t)(R * n * n * 4), &gres) ||
      upload(dir, "c_alpha.bin", 12, &alpha))
    return 1;
  const int64_t ws_bytes = mhc_coeff_bwd_workspace_bytes(R, n);
  HIP_CHECK(hipMalloc(&gmix, (size_t)(R * m * 4)));
  HIP_CHECK(hipMalloc(&gb, (size_t)(m * 4)));
  HIP_CHECK(hipMalloc(&ga, 12));
  HIP_CHECK(hipMalloc(&ws, (size_t)ws_bytes));
  HIP_CHECK(hipMemset(ws, 0, (size_t)ws_bytes));
  /* one launch (the policy at this size), then two, on the same workspace */
  for (int32_t launches = 0; launches <= 2; launches += 2) {
    MHC_CHECK(mhc_coeff_bwd(mix, cpre, post, gpre, gpost, gres, alpha, 2.0f, gmix, gb, ga, ws,
                            ws_bytes, R, n, launches, NULL, NULL, NULL));
    HIP_CHECK(hipDeviceSynchronize());
  }
  if (download(dir, "c_grad_mix.bin", gmix, (size_t)(R * m * 4)) ||
      download(dir, "c_grad_b.bin", gb, (size_t)(m * 4)) ||
      download(dir, "c_grad_alpha.bin", ga, 12))
    return 1;

  /* the entry point that allocates nothing, into fresh outputs */
  void *na_gmix, *na_gb, *na_ga;
  HIP_CHECK(hipMalloc(&na_gmix, (size_t)(R * m * 4)));
  HIP_CHECK(hipMalloc(&na_gb, (size_t)(m * 4)));
  HIP_CHECK(hipMalloc(&na_ga, 12));
  MHC_CHECK(mhc_coeff_bwd_noalloc(mix, cpre, post, gpre, gpost, gres, alpha, 2.0f, na_gmix,
                                  na_gb, na_ga, R, n, 0, NULL, NULL, NULL));
  HIP_CHECK(hipDeviceSynchronize());
  if (download(dir, "c_na_grad_mix.bin", na_gmix, (size_t)(R * m * 4)) ||
      download(dir, "c_na_grad_b.bin", na_gb, (size_t)(m * 4)) ||
      download(dir, "c_na_grad_alpha.bin", na_ga, 12))
    return 1;

  /* bf16 row tensors through mhc_coeff_bwd_ex, on the same workspace */
  void *b_mix, *b_pre, *b_post, *b_gpre, *b_gpost, *b_gres, *b_gmix;
  if (upload(dir, "c16_mix.bin", (size_t)(R * m * 2), &b_mix) ||
      upload(dir, "c16_pre.bin", (size_t)(R * n * 2), &b_pre) ||
      upload(dir, "c16_post.bin", (size_t)(R * n * 2), &b_post) ||
      upload(dir, "c16_grad_pre.bin", (size_t)(R * n * 2), &b_gpre) ||
      upload(dir, "c16_grad_post.bin", (size_t)(R * n * 2), &b_gpost) ||
      upload(dir, "c16_grad_res.bin", (size_t)(R * n * n * 2), &b_gres))
    return 1;
  HIP_CHECK(hipMalloc(&b_gmix, (size_t)(R * m * 2)));
  MHC_CHECK(mhc_coeff_bwd_ex(b_mix, b_pre, b_post, b_gpre, b_gpost, b_gres, alpha, 2.0f, b_gmix,
                             gb, ga, ws, ws_bytes, R, n, MHC_COEFF_BF16, 0, NULL, NULL, NULL));
  HIP_CHECK(hipDeviceSynchronize());
  if (download(dir, "c16_grad_mix.bin", b_gmix, (size_t)(R * m * 2)) ||
      download(dir, "c16_grad_b.bin", gb, (size_t)(m * 4)) ||
      download(dir, "c16_grad_alpha.bin", ga, 12))
    return 1;
  printf("c gpu calls ok\n");
  return 0;
}
