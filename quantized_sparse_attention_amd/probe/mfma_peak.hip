// Measured MFMA throughput of the running chip, for the benchmark report.
//
// The attention kernels are priced against the published dense peaks (int8
// 5.0 POP/s, bf16 2.5 PFLOP/s at 2.4 GHz).  Under a sustained MFMA load the
// chip lowers its clock to stay in its power budget, so the rate an MFMA-only
// loop reaches on the same box is the practical ceiling.  These kernels issue
// nothing but the two instructions the attention kernels use, on register
// operands, with four independent accumulator chains per type:
//   kind 0: v_mfma_i32_32x32x32_i8   (65,536 int8 ops each)
//   kind 1: v_mfma_f32_32x32x16_bf16 (32,768 bf16 flops each)
//   kind 2: both, in the attention kernels' ratio (equal op counts: one int8
//           MFMA per two bf16 MFMAs)
// Not part of the attention library: built into libqsa_probe.so.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int kThreads = 256;

template <int KIND>
__global__ __launch_bounds__(kThreads) void mfma_peak_kernel(int iters, float* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const v4i a = {lane, lane + 1, -lane, 3};
  const v4i b = {1, -lane, lane, 7};
  v8bf va, vb;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    va[e] = (__bf16)(0.001f * (float)(lane + e));
    vb[e] = (__bf16)(0.002f * (float)(e - lane));
  }
  v16i ai[4];
  v16f af[4];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      ai[c][r] = 0;
      af[c][r] = 0.0f;
    }
  for (int it = 0; it < iters; ++it) {
    if (KIND == 0) {
#pragma unroll
      for (int c = 0; c < 4; ++c) ai[c] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, ai[c], 0, 0, 0);
    } else if (KIND == 1) {
#pragma unroll
      for (int c = 0; c < 4; ++c) af[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, vb, af[c], 0, 0, 0);
    } else {
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        ai[c] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, ai[c], 0, 0, 0);
        af[2 * c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, vb, af[2 * c], 0, 0, 0);
        af[2 * c + 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, vb, af[2 * c + 1], 0, 0, 0);
      }
    }
  }
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += (float)ai[c][r] + af[c][r];
  out[(size_t)blockIdx.x * kThreads + threadIdx.x] = s;
}

}  // namespace

extern "C" {

// Operations (int8 ops plus bf16 flops) one launch of `kind` performs.
double qsa_probe_mfma_ops(int32_t kind, int32_t iters, int32_t blocks) {
  const double waves = (double)blocks * (kThreads / 64);
  const double per_iter = kind == 0 ? 4.0 * 65536.0 : kind == 1 ? 4.0 * 32768.0
                                                                : 2.0 * 65536.0 + 4.0 * 32768.0;
  return waves * (double)iters * per_iter;
}

// Launches kind (0 int8, 1 bf16, 2 mixed) on `stream` with `blocks`
// workgroups of 256 threads, each wave running `iters` iterations; `out` is
// a device buffer of blocks * 256 floats (written, not read).  Returns 0, or
// -1 for an invalid argument, -2 when the launch fails.
int qsa_probe_mfma(int32_t kind, int32_t iters, int32_t blocks, float* out, void* stream) {
  if (kind < 0 || kind > 2 || iters < 1 || blocks < 1 || out == nullptr) return -1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (kind == 0)
    hipLaunchKernelGGL(mfma_peak_kernel<0>, dim3(blocks), dim3(kThreads), 0, s, iters, out);
  else if (kind == 1)
    hipLaunchKernelGGL(mfma_peak_kernel<1>, dim3(blocks), dim3(kThreads), 0, s, iters, out);
  else
    hipLaunchKernelGGL(mfma_peak_kernel<2>, dim3(blocks), dim3(kThreads), 0, s, iters, out);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

}  // extern "C"
