// Device helpers of the per-block symmetric int8 quantisation (QuantSparse,
// gist.science/es/paper/2509.23681, technical summary §1 and §4: 8-bit
// activations), shared by the quantisation kernels and by the windowed
// attention pass that quantises its own query rows.  Either way a code is
// clamp(rint(fl32(x / s)), -127, 127) with s = fl32(amax / 127), bit for bit.
// Each function keeps FP contraction off in its own body, so the result does
// not depend on the including file's settings; the library is built with
// correctly rounded fp32 division.
#pragma once

#include "qsa_internal.h"

namespace qsa {
namespace {

// code = clamp(rint(fl32(x / s)), -127, 127) for a block scale s > 0 with
// |x| <= 127 s (the clamp only guards the contract), returned as the fp32
// value of that integer.
//
// Without a division per element: with inv = fl32(1 / s), p = fl32(x * inv)
// is within 127 * 2^-23 < 2^-16 of the exact quotient q = x / s, and fl32(q)
// within half an ulp below 128, 2^-18, of q.  c = rint(p) and d = p - c are
// exact (d by Sterbenz's lemma).  If |d| <= 1/2 - 2^-15 then |q - c| <
// 1/2 - 2^-16 and |fl32(q) - c| < 1/2 - 2^-16 + 2^-18 < 1/2, so c is
// rint(fl32(q)); otherwise the element takes the IEEE division.  Needs 1 / s
// finite and normal: the caller takes the division for every element when
// s < 2^-100 (fast = false).
__device__ __forceinline__ bool near_half(float p, float c) {
#pragma clang fp contract(off)
  return !(fabsf(p - c) <= 0.5f - 0x1p-15f);
}

__device__ __forceinline__ void codes8(const float (&x)[8], float s, float inv, bool fast,
                                       float (&q)[8]) {
#pragma clang fp contract(off)
  bool any_div = !fast;  // one flag per lane; the rare branch re-tests each element
  if (fast) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float p = x[e] * inv;
      q[e] = __builtin_rintf(p);
      any_div |= near_half(p, q[e]);
    }
  }
  if (any_div) {
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (!fast || near_half(x[e] * inv, q[e])) q[e] = __builtin_rintf(x[e] / s);
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) q[e] = __builtin_amdgcn_fmed3f(q[e], -127.0f, 127.0f);
}

// Eight integer-valued floats in [-127, 127] to their int8 bytes (lo: e 0-3,
// hi: e 4-7) and to four pairs of int16 (pairs[k] holds elements 2k, 2k+1).
// Adding 1.5 * 2^23 is exact and leaves the integer's two's complement in the
// low mantissa bits; byte permutes then gather them.
__device__ __forceinline__ void pack_codes(const float (&q)[8], uint32_t& lo, uint32_t& hi,
                                           uint32_t (&pairs)[4]) {
#pragma clang fp contract(off)
  uint32_t b[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) b[e] = __float_as_uint(q[e] + 0x1.8p23f);
#pragma unroll
  for (int k = 0; k < 4; ++k) pairs[k] = __builtin_amdgcn_perm(b[2 * k + 1], b[2 * k], 0x05040100u);
  lo = __builtin_amdgcn_perm(pairs[1], pairs[0], 0x06040200u);
  hi = __builtin_amdgcn_perm(pairs[3], pairs[2], 0x06040200u);
}

}  // namespace
}  // namespace qsa
