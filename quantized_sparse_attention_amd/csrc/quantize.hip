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
// multiplication by 1 / scale and a check of that product's distance to its
// rounding (the division itself only for the rare quotients next to a
// half-integer).  The
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
#include <type_traits>

#include "qsa_internal.h"
#include "quant_codes.h"

#pragma clang fp contract(off)

namespace qsa {
namespace {

typedef short v2s16 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ uint32_t add_i16x2(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_bit_cast(v2s16, a) + __builtin_bit_cast(v2s16, b));
}

// The value of lane (lane ^ M) for M < 16, moved with DPP inside the lane's
// row of 16 (no LDS crossbar): lane distances 1 and 2 by quad permutes, 8 by
// a rotate of the row by 8 (its own inverse), 4 by two moves: a mirror of
// each half-row (lane i takes lane 7 - i) after a reversal of each quad
// (lane i takes i ^ 3), so lane i reads 7 - (i ^ 3) = i ^ 4.
template <int M>
__device__ __forceinline__ float lane_xor(float v) {
  static_assert(M == 1 || M == 2 || M == 4 || M == 8, "partners inside a row of 16 lanes");
  const int x = __float_as_int(v);
  if constexpr (M == 4) {
    const int t = __builtin_amdgcn_update_dpp(0, x, 0x141, 0xF, 0xF, true);  // row_half_mirror
    return __int_as_float(
        __builtin_amdgcn_update_dpp(0, t, 0x1B, 0xF, 0xF, true));  // quad_perm [3,2,1,0]
  } else {
    // quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_ror:8
    constexpr int ctrl = M == 1 ? 0xB1 : M == 2 ? 0x4E : 0x128;
    return __int_as_float(__builtin_amdgcn_update_dpp(0, x, ctrl, 0xF, 0xF, true));
  }
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
  auto stage = [&](auto mc) {  // h = 8 m: the partner lane is lane ^ m
    constexpr int m = decltype(mc)::value;
    // lower lane: v_j + v_{j+h}; upper lane: v_j - v_{j+h}.  One fused
    // multiply-add by +-1 rounds exactly as that sum or difference.
    const float sgn = (lane & m) != 0 ? -1.0f : 1.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = __builtin_fmaf(sgn, v[e], lane_xor<m>(v[e]));
  };
  if constexpr (CPR > 1) stage(std::integral_constant<int, 1>{});
  if constexpr (CPR > 2) stage(std::integral_constant<int, 2>{});
  if constexpr (CPR > 4) stage(std::integral_constant<int, 4>{});
  if constexpr (CPR > 8) stage(std::integral_constant<int, 8>{});
  static_assert(CPR <= 16, "rows of at most 16 lanes");
}

// MAP: the rows are quantised in position-major order of windows of w tokens
// (row p*(L/w) + k of the quantised sequence is row k*w + p of x), read
// straight from x.  POOL: the pooled code sums are computed and written
// (the windowed passes, which select nothing, skip them).  Workgroups
// blockIdx.y = 0 and 1 quantise the two tensors of a pair (x2, codes2 and
// scales2 for the second).
template <int BS, int D, bool ROT, bool MAP, bool POOL = true>
__global__ __launch_bounds__(256) void quantize_kernel(const uint16_t* __restrict__ x,
                                                       int8_t* __restrict__ codes,
                                                       float* __restrict__ scales,
                                                       int32_t* __restrict__ pooled, int L,
                                                       int nb, int w,
                                                       const uint16_t* __restrict__ x2 = nullptr,
                                                       int8_t* __restrict__ codes2 = nullptr,
                                                       float* __restrict__ scales2 = nullptr) {
  if (blockIdx.y) {
    x = x2;
    codes = codes2;
    scales = scales2;
  }
  constexpr int CPR = D / 8;        // 16-byte chunks per token row
  constexpr int RPP = 256 / CPR;    // rows covered per pass
  constexpr int PASSES = BS / RPP;  // passes over the block
  static_assert(BS % RPP == 0, "block must be a multiple of rows per pass");

  __shared__ float s_amax[4];
  __shared__ int32_t s_pool[POOL ? 4 : 1][POOL ? D : 1];

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

  // per-channel code sums as packed int16 pairs: a block sum is at most
  // 127 * BS in magnitude
  static_assert(127 * BS <= 32767, "block code sums must fit int16");
  uint32_t psum[4] = {0u, 0u, 0u, 0u};

#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int row = r0 + p * RPP;
    if (row < n) {
      float q[8];
      if (s > 0.0f) {
        codes8(y[p], s, inv, fast, q);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) q[e] = 0.0f;
      }
      uint32_t lo, hi, pairs[4];
      pack_codes(q, lo, hi, pairs);
      if constexpr (POOL) {
#pragma unroll
        for (int k = 0; k < 4; ++k) psum[k] = add_i16x2(psum[k], pairs[k]);
      }
      *reinterpret_cast<uint2*>(cb + (size_t)row * D) = make_uint2(lo, hi);
    }
  }

  const uint64_t blk = bh * (uint64_t)nb + i;
  if constexpr (!POOL) {
    if (tid == 0) scales[blk] = s;
    return;
  }
  // reduce the per-lane channel sums over lanes holding the same channels
#pragma unroll
  for (int o = CPR; o < 64; o <<= 1) {
#pragma unroll
    for (int k = 0; k < 4; ++k)
      psum[k] = add_i16x2(psum[k], (uint32_t)__shfl_xor((int)psum[k], o, 64));
  }
  if (lane < CPR) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      s_pool[wave][lane * 8 + 2 * k] = (int16_t)(psum[k] & 0xffffu);
      s_pool[wave][lane * 8 + 2 * k + 1] = (int16_t)(psum[k] >> 16);
    }
  }
  __syncthreads();
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

// Codes and scales only, of one tensor or (x2 not NULL) two of the same
// shape in one launch.
template <int BS, int D, bool MAP>
hipError_t launch_pair_t(const qsa_dims& d, const uint16_t* x, const uint16_t* x2, int8_t* codes,
                         int8_t* codes2, float* scales, float* scales2, int w, hipStream_t s) {
  const int nb = (d.seq_len + BS - 1) / BS;
  const uint64_t n_wg = (uint64_t)d.batch * d.heads * nb;
  hipLaunchKernelGGL((quantize_kernel<BS, D, false, MAP, false>),
                     dim3((uint32_t)n_wg, x2 ? 2u : 1u),
                     dim3(256), 0, s, x, codes, scales, nullptr, d.seq_len, nb, w, x2, codes2,
                     scales2);
  return hipGetLastError();
}

template <bool MAP>
hipError_t dispatch_pair(const qsa_dims& d, const uint16_t* x, const uint16_t* x2, int8_t* codes,
                         int8_t* codes2, float* scales, float* scales2, int w, hipStream_t s) {
  if (d.block == 64 && d.head_dim == 128)
    return launch_pair_t<64, 128, MAP>(d, x, x2, codes, codes2, scales, scales2, w, s);
  if (d.block == 64 && d.head_dim == 64)
    return launch_pair_t<64, 64, MAP>(d, x, x2, codes, codes2, scales, scales2, w, s);
  if (d.block == 128 && d.head_dim == 128)
    return launch_pair_t<128, 128, MAP>(d, x, x2, codes, codes2, scales, scales2, w, s);
  return launch_pair_t<128, 64, MAP>(d, x, x2, codes, codes2, scales, scales2, w, s);
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

hipError_t launch_quantize_codes(const qsa_dims& d, const uint16_t* x, const uint16_t* x2,
                                 int window, int8_t* codes, int8_t* codes2, float* scales,
                                 float* scales2, hipStream_t s) {
  if (window > 0)
    return dispatch_pair<true>(d, x, x2, codes, codes2, scales, scales2, window, s);
  return dispatch_pair<false>(d, x, x2, codes, codes2, scales, scales2, 1, s);
}

}  // namespace qsa
