// Standalone sparse-step correction: out = bf16(sparse + r + dr).
//
// QuantSparse (gist.science/es/paper/2509.23681), technical summary §2B: a
// cache of the first- and second-order residuals corrects the sparse
// attention output at small cost.  Elementwise and HBM-bound: 16-byte loads
// and stores (8 bf16 per lane), grid-stride over the whole tensor.
#include "qsa_internal.h"

namespace qsa {
namespace {

__global__ __launch_bounds__(256) void apply_residual_kernel(const uint4* __restrict__ sp,
                                                             const uint4* __restrict__ r,
                                                             const uint4* __restrict__ dr,
                                                             uint4* out, uint64_t n_vec) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t k = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; k < n_vec; k += stride) {
    const uint4 a = sp[k];
    const uint4 b = r[k];
    const uint4 c = dr ? dr[k] : make_uint4(0, 0, 0, 0);
    const uint32_t aw[4] = {a.x, a.y, a.z, a.w};
    const uint32_t bw[4] = {b.x, b.y, b.z, b.w};
    const uint32_t cw[4] = {c.x, c.y, c.z, c.w};
    uint32_t o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float lo = bf16_lo(aw[e]) + bf16_lo(bw[e]) + bf16_lo(cw[e]);
      const float hi = bf16_hi(aw[e]) + bf16_hi(bw[e]) + bf16_hi(cw[e]);
      o[e] = pack_bf16x2(lo, hi);
    }
    out[k] = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

}  // namespace

hipError_t launch_apply_residual(const qsa_dims& d, const uint16_t* sparse_out,
                                 const uint16_t* r, const uint16_t* dr, uint16_t* out,
                                 hipStream_t s) {
  const uint64_t n = (uint64_t)d.batch * d.heads * d.seq_len * d.head_dim;
  const uint64_t n_vec = n / 8;  // head_dim is a multiple of 8
  uint64_t blocks = (n_vec + 255) / 256;
  if (blocks > 256 * 64) blocks = 256 * 64;
  hipLaunchKernelGGL(apply_residual_kernel, dim3((uint32_t)blocks), dim3(256), 0, s,
                     reinterpret_cast<const uint4*>(sparse_out), reinterpret_cast<const uint4*>(r),
                     reinterpret_cast<const uint4*>(dr), reinterpret_cast<uint4*>(out), n_vec);
  return hipGetLastError();
}

}  // namespace qsa
