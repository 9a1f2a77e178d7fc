// Normalised L1 change between a layer's consecutive outputs: the sums
// sum |cur - prev| and sum |prev| over all elements, for an adaptive
// refresh trigger (DVD-Quant, gist.science/es/paper/2505.18663, technical
// summary §2C: the normalised L1 distance of consecutive output features is
// accumulated against a threshold).
//
// HBM-bound: both bf16 tensors are read once with 16-byte loads.  Every
// element's |cur - prev| and |prev| are formed in fp64 (exact for bf16
// operands whose exponents differ by at most 45) and summed in fp64: per
// thread in a grid-stride order, then by a fixed tree, then the per-block
// partials by one wave in a fixed order -- deterministic for a given size.
#include <mutex>

#include "qsa_internal.h"

// The partial sums of qsa_l1_change_noalloc: a fixed QSA_L1_WORK_BYTES per
// GPU, held until the process ends.  Host code reaches it only through the
// per-device address from hipGetSymbolAddress (l1_static_scratch); the name
// itself is a host-side stand-in, not a device address.
static __device__ __align__(256) double scratch[QSA_L1_WORK_BYTES / sizeof(double)];

namespace qsa {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxScratchDevices = 64;

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__global__ __launch_bounds__(kThreads) void l1_partial_kernel(const uint16_t* __restrict__ prev,
                                                              const uint16_t* __restrict__ cur,
                                                              uint64_t n8,
                                                              double* __restrict__ partial) {
  __shared__ double s_red[2][kThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  double num = 0.0, den = 0.0;
  const uint64_t stride = (uint64_t)gridDim.x * kThreads;
  for (uint64_t i = (uint64_t)blockIdx.x * kThreads + tid; i < n8; i += stride) {
    const uint4 a = *reinterpret_cast<const uint4*>(prev + 8 * i);
    const uint4 b = *reinterpret_cast<const uint4*>(cur + 8 * i);
    const uint32_t wa[4] = {a.x, a.y, a.z, a.w}, wb[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const double p0 = bf16_lo(wa[e]), p1 = bf16_hi(wa[e]);
      const double c0 = bf16_lo(wb[e]), c1 = bf16_hi(wb[e]);
      num += fabs(c0 - p0);
      num += fabs(c1 - p1);
      den += fabs(p0);
      den += fabs(p1);
    }
  }
  num = wave_sum(num);
  den = wave_sum(den);
  if (lane == 0) {
    s_red[0][wave] = num;
    s_red[1][wave] = den;
  }
  __syncthreads();
  if (tid == 0) {
    partial[2 * blockIdx.x] = (s_red[0][0] + s_red[0][1]) + (s_red[0][2] + s_red[0][3]);
    partial[2 * blockIdx.x + 1] = (s_red[1][0] + s_red[1][1]) + (s_red[1][2] + s_red[1][3]);
  }
}

__global__ __launch_bounds__(64) void l1_final_kernel(const double* __restrict__ partial,
                                                      int nblocks, double* __restrict__ sums) {
  const int lane = threadIdx.x;
  double num = 0.0, den = 0.0;
  for (int i = lane; i < nblocks; i += 64) {
    num += partial[2 * i];
    den += partial[2 * i + 1];
  }
  num = wave_sum(num);
  den = wave_sum(den);
  if (lane == 0) {
    sums[0] = num;
    sums[1] = den;
  }
}

}  // namespace

int l1_change_blocks(uint64_t n_elements) {
  const uint64_t n8 = n_elements / 8;
  uint64_t b = (n8 + kThreads - 1) / kThreads;
  return (int)(b < 1 ? 1 : (b > kL1MaxBlocks ? kL1MaxBlocks : b));
}

hipError_t l1_static_scratch(double** work) {
  static std::mutex mu;
  static double* addr[kMaxScratchDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = static_cast<double*>(p);
  }
  *work = addr[dev];
  return hipSuccess;
}

hipError_t launch_l1_change(uint64_t n_elements, const uint16_t* prev, const uint16_t* cur,
                            double* sums, double* work, hipStream_t s) {
  const int nb = l1_change_blocks(n_elements);
  hipLaunchKernelGGL(l1_partial_kernel, dim3(nb), dim3(kThreads), 0, s, prev, cur,
                     n_elements / 8, work);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(l1_final_kernel, dim3(1), dim3(64), 0, s, work, nb, sums);
  return hipGetLastError();
}

}  // namespace qsa
