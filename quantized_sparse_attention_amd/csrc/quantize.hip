// Per-block symmetric int8 quantisation of Q or K plus pooled code sums.
//
// QuantSparse (gist.science/es/paper/2509.23681), technical summary §1 and §4:
// activations are quantised to 8 bits; the pooled sums feed the block
// saliency (average pooling of §2A's global guidance).
//
// One workgroup (4 waves) per (batch, head, token block).  HBM-bound: each
// bf16 element is read once and each code written once, with 16-byte
// coalesced loads (8 bf16 per lane) and 8-byte stores.
//
// Bit-exactness: the scale is an IEEE fp32 division amax / 127 and each code
// the round-half-even of an IEEE fp32 division x / scale, reached through a
// multiplication by 1 / scale and an exact check of the remainder (the
// division itself only for the rare quotients next to a half-integer).  The
// library is compiled with correctly rounded fp32 division, no fast-math and
// no FP contraction in this file, and fp32 denormals preserved.
//
// Rotated variant (Hadamard rotation of the activations before quantisation,
// DVD-Quant gist.science/es/paper/2505.18663, technical summary §2B: it
// spreads extreme channels over all channels): every token row x becomes
// y = x H_D with H_D the Sylvester Hadamard matrix (entries +-1, unscaled),
// computed in fp32 by the fast Walsh-Hadamard transform in a fixed order:
// stages h = 1, 2, 4, ..., D/2, each replacing every pair (j, j+h) of a
// 2h-aligned group by (v_j + v_{j+h}, v_j - v_{j+h}); then y is quantised as
// above.  Since H_D H_D^T = D I, (q H)(k H)^T = D (q k^T): attention on
// rotated codes uses sm_scale / D.  A lane holds 8 consecutive channels, so
// stages h < 8 run in registers and h >= 8 exchange with the lane h/8 away.
#include "qsa_internal.h"

#pragma clang fp contract(off)

namespace qsa {
namespace {

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// code = clamp(rint(fl32(x / s)), -127, 127) for a block scale s > 0 with
// |x| <= 127 s (the clamp only guards the contract).
//
// Without a division per element: with inv = fl32(1 / s), p = fl32(x * inv)
// is within 127 * 2^-23 < 2^-16 of the exact quotient q = x / s, and so is
// fl32(q) (half an ulp below 128 is 2^-18).  Unless q lies within 2^-16 of a
// half-integer, p, q and fl32(q) round to the same integer c = rint(p).  The
// remainder d = fl32(x - c s) (one fused rounding) tells: | |d| - s/2 | >
// 2^-14 s implies | |q - c| - 1/2 | > 2^-16 (the roundings of d and of the
// test move it by less than 2^-23 s), so c is right; otherwise the element
// takes the IEEE division.  Needs 1 / s finite and s 2^-14 normal: the caller
// takes the division for every element when s < 2^-100.
__device__ __forceinline__ void codes8(const float (&x)[8], float s, float inv, bool fast,
                                       int (&c)[8]) {
  float q[8];
  bool any_div = !fast;
  uint32_t div = fast ? 0u : 0xffu;  // elements that take the division
  if (fast) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      q[e] = __builtin_rintf(x[e] * inv);
      const float d = __builtin_fmaf(-q[e], s, x[e]);
      if (!(fabsf(fabsf(d) - 0.5f * s) > s * 0x1p-14f)) div |= 1u << e;
    }
    any_div = div != 0u;
  }
  if (any_div) {
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if ((div >> e) & 1u) q[e] = __builtin_rintf(x[e] / s);
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) c[e] = (int)fminf(fmaxf(q[e], -127.0f), 127.0f);
}

// In-place fast Walsh-Hadamard transform of one token row held 8 channels
// per lane by CPR consecutive lanes (lane l holds channels 8 (l % CPR) + e).
template <int CPR>
__device__ __forceinline__ void fwht_row(float (&v)[8], int lane) {
#pragma unroll
  for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if (e & h) continue;
      const float a = v[e], b = v[e + h];
      v[e] = a + b;
      v[e + h] = a - b;
    }
  }
#pragma unroll
  for (int m = 1; m < CPR; m <<= 1) {  // h = 8 m: the partner lane is lane ^ m
    const bool upper = (lane & m) != 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float o = __shfl_xor(v[e], m, 64);
      v[e] = upper ? o - v[e] : v[e] + o;  // lower: v_j + v_{j+h}; upper: v_j - v_{j+h}
    }
  }
}

// MAP: the rows are quantised in position-major order of windows of w tokens
// (row p*(L/w) + k of the quantised sequence is row k*w + p of x), read
// straight from x.
template <int BS, int D, bool ROT, bool MAP>
__global__ __launch_bounds__(256) void quantize_kernel(const uint16_t* __restrict__ x,
                                                       int8_t* __restrict__ codes,
                                                       float* __restrict__ scales,
                                                       int32_t* __restrict__ pooled, int L,
                                                       int nb, int w) {
  constexpr int CPR = D / 8;        // 16-byte chunks per token row
  constexpr int RPP = 256 / CPR;    // rows covered per pass
  constexpr int PASSES = BS / RPP;  // passes over the block
  static_assert(BS % RPP == 0, "block must be a multiple of rows per pass");

  __shared__ float s_amax[4];
  __shared__ int32_t s_pool[4][D];

  const uint32_t wg = blockIdx.x;
  const uint32_t i = wg % (uint32_t)nb;
  const uint64_t bh = wg / (uint32_t)nb;
  const int t0 = (int)i * BS;
  const int n = min(BS, L - t0);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int cc = tid % CPR;
  const int r0 = tid / CPR;

  const uint16_t* xh = x + bh * (uint64_t)L * D + cc * 8;
  const int m = MAP ? L / w : 1;
  int8_t* cb = codes + (bh * (uint64_t)L + (uint64_t)t0) * D + cc * 8;

  float y[PASSES][8];
  float amax = 0.0f;
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int row = r0 + p * RPP;
    uint4 raw = make_uint4(0, 0, 0, 0);
    if (row < n) {
      const int r = t0 + row;
      const int src = MAP ? (r % m) * w + r / m : r;
      raw = *reinterpret_cast<const uint4*>(xh + (size_t)src * D);
    }
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      y[p][2 * e] = bf16_lo(w[e]);
      y[p][2 * e + 1] = bf16_hi(w[e]);
    }
    if (ROT) fwht_row<CPR>(y[p], lane);  // rows past the end are zero: they stay zero
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(y[p][e]));
  }
  amax = wave_max(amax);
  if (lane == 0) s_amax[wave] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(s_amax[0], s_amax[1]), fmaxf(s_amax[2], s_amax[3]));
  const float s = amax / 127.0f;  // IEEE division; 0 for an all-zero block
  const bool fast = s >= 0x1p-100f;
  const float inv = fast ? 1.0f / s : 0.0f;

  int psum[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) psum[e] = 0;

#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int row = r0 + p * RPP;
    if (row < n) {
      int c[8];
      if (s > 0.0f) {
        codes8(y[p], s, inv, fast, c);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) c[e] = 0;
      }
      uint32_t lo = 0, hi = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        lo |= (uint32_t)(c[e] & 0xff) << (8 * e);
        hi |= (uint32_t)(c[4 + e] & 0xff) << (8 * e);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) psum[e] += c[e];
      *reinterpret_cast<uint2*>(cb + (size_t)row * D) = make_uint2(lo, hi);
    }
  }

  // reduce the per-lane channel sums over lanes holding the same channels
#pragma unroll
  for (int o = CPR; o < 64; o <<= 1) {
#pragma unroll
    for (int e = 0; e < 8; ++e) psum[e] += __shfl_xor(psum[e], o, 64);
  }
  if (lane < CPR) {
#pragma unroll
    for (int e = 0; e < 8; ++e) s_pool[wave][lane * 8 + e] = psum[e];
  }
  __syncthreads();
  const uint64_t blk = bh * (uint64_t)nb + i;
  if (tid < D) {
    pooled[blk * D + tid] = s_pool[0][tid] + s_pool[1][tid] + s_pool[2][tid] + s_pool[3][tid];
  }
  if (tid == 0) scales[blk] = s;
}

template <int BS, int D, bool ROT, bool MAP>
hipError_t launch_t(const qsa_dims& d, const uint16_t* x, int8_t* codes, float* scales,
                    int32_t* pooled, int w, hipStream_t s) {
  const int nb = (d.seq_len + BS - 1) / BS;
  const uint64_t n_wg = (uint64_t)d.batch * d.heads * nb;
  hipLaunchKernelGGL((quantize_kernel<BS, D, ROT, MAP>), dim3((uint32_t)n_wg), dim3(256), 0, s,
                     x, codes, scales, pooled, d.seq_len, nb, w);
  return hipGetLastError();
}

template <bool ROT, bool MAP>
hipError_t dispatch(const qsa_dims& d, const uint16_t* x, int8_t* codes, float* scales,
                    int32_t* pooled, int w, hipStream_t s) {
  if (d.block == 64 && d.head_dim == 128)
    return launch_t<64, 128, ROT, MAP>(d, x, codes, scales, pooled, w, s);
  if (d.block == 64 && d.head_dim == 64)
    return launch_t<64, 64, ROT, MAP>(d, x, codes, scales, pooled, w, s);
  if (d.block == 128 && d.head_dim == 128)
    return launch_t<128, 128, ROT, MAP>(d, x, codes, scales, pooled, w, s);
  return launch_t<128, 64, ROT, MAP>(d, x, codes, scales, pooled, w, s);
}

}  // namespace

hipError_t launch_quantize(const qsa_dims& d, const uint16_t* x, int8_t* codes, float* scales,
                           int32_t* pooled, hipStream_t s) {
  return dispatch<false, false>(d, x, codes, scales, pooled, 1, s);
}

hipError_t launch_quantize_rotated(const qsa_dims& d, const uint16_t* x, int8_t* codes,
                                   float* scales, int32_t* pooled, hipStream_t s) {
  return dispatch<true, false>(d, x, codes, scales, pooled, 1, s);
}

hipError_t launch_quantize_position_major(const qsa_dims& d, const uint16_t* x, int window,
                                          int8_t* codes, float* scales, int32_t* pooled,
                                          hipStream_t s) {
  return dispatch<false, true>(d, x, codes, scales, pooled, window, s);
}

}  // namespace qsa
