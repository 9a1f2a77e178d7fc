/*
 * A C99 client of libqsa that uses include/qsa.h and the HIP runtime API
 * only: the header compiles as C, the library links, argument errors come
 * back before any device work, and ("gpu") one qsa_quantize call on device
 * memory and a stream returns what a constant block must give.
 *
 * The blocks of the "gpu" case hold one magnitude each, with the sign
 * alternating over channels (one block all zero): per the per-block
 * symmetric quantisation of QuantSparse (gist.science/es/paper/2509.23681,
 * technical summary §1), the scale is fl32(|x| / 127), every code is +-127
 * (0 in the zero block), and each pooled sum is +-127 times the block's row
 * count (the last block of 130 tokens has 2 rows).
 */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "qsa.h"

static int expect(const char* what, int got, int want) {
  if (got == want) return 0;
  fprintf(stderr, "%s: status %d (%s), expected %d; detail: %s\n", what, got,
          qsa_status_string(got), want, qsa_last_error_detail());
  return 1;
}

static int host_checks(void) {
  qsa_dims d = {1, 2, 130, 64, 64};
  int bad = 0;
  /* stand-in device addresses: argument checks reject these calls before any
     pointer is used */
  const uint16_t* x = (const uint16_t*)(uintptr_t)4096;
  int8_t* codes = (int8_t*)(uintptr_t)8192;
  float* scales = (float*)(uintptr_t)12288;
  int32_t* pooled = (int32_t*)(uintptr_t)16384;

  if (qsa_version() != QSA_VERSION) {
    fprintf(stderr, "qsa_version %d, header %d\n", qsa_version(), QSA_VERSION);
    bad = 1;
  }
  bad |= expect("NULL dims", qsa_quantize(NULL, x, codes, scales, pooled, NULL), QSA_ERR_NULL);
  bad |= expect("NULL codes", qsa_quantize(&d, x, NULL, scales, pooled, NULL), QSA_ERR_NULL);
  bad |= expect("misaligned x",
                qsa_quantize(&d, (const uint16_t*)(uintptr_t)4098, codes, scales, pooled, NULL),
                QSA_ERR_ALIGN);
  d.head_dim = 96;
  bad |= expect("head_dim 96", qsa_quantize(&d, x, codes, scales, pooled, NULL), QSA_ERR_SHAPE);
  d.head_dim = 64;
  d.block = 32;
  bad |= expect("block 32", qsa_quantize(&d, x, codes, scales, pooled, NULL), QSA_ERR_SHAPE);
  d.block = 64;
  bad |= expect("work below the l1 scratch size",
                qsa_l1_change(&d, x, x, (double*)(uintptr_t)20480, (void*)(uintptr_t)24576,
                              QSA_L1_WORK_BYTES - 1, NULL),
                QSA_ERR_PARAM);
  if (strlen(qsa_status_string(QSA_ERR_SHAPE)) == 0) {
    fprintf(stderr, "empty status string\n");
    bad = 1;
  }
  return bad;
}

static uint16_t bf16_bits(float f) { /* exact for the values used here */
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  return (uint16_t)(u >> 16);
}

#define HIP_OK(call)                                                      \
  do {                                                                    \
    hipError_t e_ = (call);                                               \
    if (e_ != hipSuccess) {                                               \
      fprintf(stderr, "%s: %s\n", #call, hipGetErrorString(e_));          \
      return 1;                                                           \
    }                                                                     \
  } while (0)

enum { H = 2, L = 130, D = 64, BS = 64, NB = (L + BS - 1) / BS };

static float magnitude(int h, int blk) { /* block (1, 2) is all zero */
  return (h == 1 && blk == NB - 1) ? 0.0f : 0.5f * (float)((h + 1) * (blk + 1));
}

static int gpu_checks(void) {
  const qsa_dims d = {1, H, L, D, BS};
  static uint16_t hx[H * L * D];
  static int8_t hc[H * L * D];
  static float hs[H * NB];
  static int32_t hp[H * NB * D];
  void *dx, *dc, *ds, *dp;
  hipStream_t s;
  int h, t, c, blk, bad = 0;

  for (h = 0; h < H; ++h)
    for (t = 0; t < L; ++t)
      for (c = 0; c < D; ++c) {
        const float v = magnitude(h, t / BS);
        hx[((size_t)h * L + t) * D + c] = bf16_bits(c % 2 ? -v : v);
      }
  HIP_OK(hipMalloc(&dx, sizeof hx));
  HIP_OK(hipMalloc(&dc, sizeof hc));
  HIP_OK(hipMalloc(&ds, sizeof hs));
  HIP_OK(hipMalloc(&dp, sizeof hp));
  HIP_OK(hipStreamCreate(&s));
  HIP_OK(hipMemcpy(dx, hx, sizeof hx, hipMemcpyHostToDevice));
  bad |= expect("qsa_quantize", qsa_quantize(&d, (const uint16_t*)dx, (int8_t*)dc, (float*)ds,
                                             (int32_t*)dp, s),
                QSA_OK);
  HIP_OK(hipStreamSynchronize(s));
  HIP_OK(hipMemcpy(hc, dc, sizeof hc, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(hs, ds, sizeof hs, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(hp, dp, sizeof hp, hipMemcpyDeviceToHost));

  for (h = 0; h < H; ++h)
    for (blk = 0; blk < NB; ++blk) {
      const float v = magnitude(h, blk);
      const float want_s = v / 127.0f; /* IEEE fp32 division, as the kernel's */
      const int rows = (blk + 1) * BS <= L ? BS : L - blk * BS;
      const int mag = v > 0.0f ? 127 : 0;
      if (memcmp(&hs[h * NB + blk], &want_s, sizeof want_s) != 0) {
        fprintf(stderr, "scale (%d,%d): %.9g, expected %.9g\n", h, blk, hs[h * NB + blk], want_s);
        bad = 1;
      }
      for (c = 0; c < D; ++c) {
        const int want_code = c % 2 ? -mag : mag;
        const int32_t got_p = hp[(h * NB + blk) * D + c];
        for (t = blk * BS; t < blk * BS + rows; ++t) {
          if (hc[((size_t)h * L + t) * D + c] != want_code) {
            fprintf(stderr, "code (%d,%d,%d): %d, expected %d\n", h, t, c,
                    hc[((size_t)h * L + t) * D + c], want_code);
            bad = 1;
            break;
          }
        }
        if (got_p != want_code * rows) {
          fprintf(stderr, "pooled (%d,%d,%d): %d, expected %d\n", h, blk, c, got_p,
                  want_code * rows);
          bad = 1;
        }
      }
    }
  HIP_OK(hipStreamDestroy(s));
  HIP_OK(hipFree(dx));
  HIP_OK(hipFree(dc));
  HIP_OK(hipFree(ds));
  HIP_OK(hipFree(dp));
  return bad;
}

int main(int argc, char** argv) {
  int bad = host_checks();
  if (!bad && argc > 1 && strcmp(argv[1], "gpu") == 0) bad = gpu_checks();
  printf(bad ? "FAILED\n" : "OK\n");
  return bad;
}
