// Block-sparse flash attention on int8 Q/K codes (sparse step) and the
// full-attention refresh step of the second-order residual cache.
//
// QuantSparse (gist.science/es/paper/2509.23681), technical summary §1
// (sparsified attention), §4 (8-bit activations, ~15 % density) and §2B
// (first-order residual = full - sparse attention; second-order residual =
// its change between consecutive refreshes; a cache of both corrects sparse
// steps).  Same content on the Korean page (ko/paper/2509.23681) §2.2.
//
// Layout of the work (gfx950, wave64):
//  * one workgroup per (batch*head, query block i) with BS/32 waves; wave w
//    owns query rows 32w..32w+31 of the block;
//  * per kept key block j: K codes [BS x D] int8 and V [BS x D] bf16 are read
//    from HBM/L2 with 16-byte loads into registers one tile ahead, then stored
//    to LDS (V transposed to [D x BS] so that P.V operands are contiguous);
//  * S^T = K_j . Q^T on v_mfma_i32_32x32x32_i8 (exact int32 dots);
//  * logits z = (sm_scale * sq_i * sk_j * log2 e) * S, online softmax in fp32
//    with exp2; the running max is only moved when a tile's max exceeds it
//    by more than TAU (so P <= 2^TAU, exact in fp32 and bf16 ranges);
//  * P is rounded to bf16 straight from the S^T accumulator registers (its
//    layout is the B operand of the next MFMA, no LDS round trip) and
//    O^T += V^T . P^T on v_mfma_f32_32x32x16_bf16 with fp32 accumulation;
//    the softmax denominator sums the same bf16-rounded P (v_dot2_f32_bf16);
//  * the epilogue normalises, adds the cached residuals (sparse step) or
//    forms the residuals (refresh step), and stores bf16.
// The refresh step keeps two online-softmax states, one over the kept blocks
// and one over the others, so full and sparse attention share every
// exponential and MFMA; it merges them at the end like split-K attention.
#include "qsa_internal.h"

namespace qsa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kTau = 8.0f;
constexpr v2bf kOnes = {(__bf16)1.0f, (__bf16)1.0f};

template <int BS, int D>
struct Cfg {
  static constexpr int WAVES = BS / 32;
  static constexpr int THREADS = WAVES * 64;
  static constexpr int KP = D + 16;  // K tile row pitch in bytes
  static constexpr int VP = BS + 8;  // V^T tile row pitch in bf16 elements
  static constexpr int NT = BS / 32;  // 32-key accumulator tiles per key block
  static constexpr int DT = D / 32;   // 32-channel output tiles
  static constexpr int KS = D / 32;   // 32-channel steps of the QK^T MFMA
  static constexpr int PS = BS / 16;  // 16-key steps of the PV MFMA
  static constexpr int K_CHUNKS = BS * D / 16 / THREADS;
  static constexpr int V_TASKS = (BS / 4) * (D / 8) / THREADS;
  static constexpr int LDS_K = BS * KP;
  static constexpr int LDS_V = D * VP * 2;
};

template <int BS, int D>
struct Stage {
  uint4 k[Cfg<BS, D>::K_CHUNKS];
  uint4 v[Cfg<BS, D>::V_TASKS][4];
};

// Global -> registers for key block j (rows beyond the sequence read as 0).
template <int BS, int D>
__device__ __forceinline__ void load_stage(Stage<BS, D>& st, const int8_t* __restrict__ kc,
                                           const uint16_t* __restrict__ v, int tid, int nvalid) {
  using C = Cfg<BS, D>;
#pragma unroll
  for (int c = 0; c < C::K_CHUNKS; ++c) {
    const int chunk = tid + c * C::THREADS;
    const int row = chunk / (D / 16), col = chunk % (D / 16);
    st.k[c] = row < nvalid ? *reinterpret_cast<const uint4*>(kc + (size_t)row * D + col * 16)
                           : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int t = 0; t < C::V_TASKS; ++t) {
    const int task = tid + t * C::THREADS;
    const int dg = task % (D / 8), kg = task / (D / 8);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int key = 4 * kg + kk;
      st.v[t][kk] = key < nvalid
                        ? *reinterpret_cast<const uint4*>(v + (size_t)key * D + dg * 8)
                        : make_uint4(0, 0, 0, 0);
    }
  }
}

__device__ __forceinline__ uint32_t word_of(const uint4& u, int w) {
  return w == 0 ? u.x : w == 1 ? u.y : w == 2 ? u.z : u.w;
}

// Registers -> LDS: K as [BS][KP] bytes, V transposed as [D][VP] bf16.
template <int BS, int D>
__device__ __forceinline__ void store_stage(const Stage<BS, D>& st, int8_t* lk, uint16_t* lv,
                                            int tid) {
  using C = Cfg<BS, D>;
#pragma unroll
  for (int c = 0; c < C::K_CHUNKS; ++c) {
    const int chunk = tid + c * C::THREADS;
    const int row = chunk / (D / 16), col = chunk % (D / 16);
    *reinterpret_cast<uint4*>(lk + row * C::KP + col * 16) = st.k[c];
  }
#pragma unroll
  for (int t = 0; t < C::V_TASKS; ++t) {
    const int task = tid + t * C::THREADS;
    const int dg = task % (D / 8), kg = task / (D / 8);
#pragma unroll
    for (int dd = 0; dd < 8; ++dd) {
      const int w = dd >> 1;
      uint32_t a0 = word_of(st.v[t][0], w), a1 = word_of(st.v[t][1], w);
      uint32_t a2 = word_of(st.v[t][2], w), a3 = word_of(st.v[t][3], w);
      uint32_t lo, hi;
      if (dd & 1) {
        lo = (a0 >> 16) | (a1 & 0xffff0000u);
        hi = (a2 >> 16) | (a3 & 0xffff0000u);
      } else {
        lo = (a0 & 0xffffu) | (a1 << 16);
        hi = (a2 & 0xffffu) | (a3 << 16);
      }
      *reinterpret_cast<uint2*>(lv + (dg * 8 + dd) * C::VP + 4 * kg) = make_uint2(lo, hi);
    }
  }
}

// Online-softmax state of one query row (held by lanes l and l^32).
template <int BS, int D>
struct Acc {
  v16f o[Cfg<BS, D>::DT];
  float m;
  float l;
  __device__ __forceinline__ void init() {
#pragma unroll
    for (int t = 0; t < Cfg<BS, D>::DT; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[t][r] = 0.0f;
    m = -__builtin_inff();
    l = 0.0f;
  }
};

// One key block against this wave's 32 query rows: QK^T, softmax update, PV.
template <int BS, int D>
__device__ __forceinline__ void process_tile(Acc<BS, D>& acc, const v4i (&qb)[Cfg<BS, D>::KS],
                                             const int8_t* lk, const uint16_t* lv, int lane,
                                             float cs, int nvalid) {
  using C = Cfg<BS, D>;
  const int g = lane >> 5, ql = lane & 31;

  v16i s[C::NT];
#pragma unroll
  for (int t = 0; t < C::NT; ++t) {
#pragma unroll
    for (int r = 0; r < 16; ++r) s[t][r] = 0;
#pragma unroll
    for (int c = 0; c < C::KS; ++c) {
      const v4i a = *reinterpret_cast<const v4i*>(lk + (32 * t + ql) * C::KP + 32 * c + 16 * g);
      s[t] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, qb[c], s[t], 0, 0, 0);
    }
  }
  // s[t][r] = S[query ql][key 32t + 8(r/4) + 4g + r%4]
  const bool tail = nvalid < BS;
  if (tail) {
#pragma unroll
    for (int t = 0; t < C::NT; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 32 * t + 8 * (r >> 2) + 4 * g + (r & 3);
        if (key >= nvalid) s[t][r] = INT32_MIN;
      }
  }
  int imax = INT32_MIN;
#pragma unroll
  for (int t = 0; t < C::NT; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) imax = max(imax, s[t][r]);
  imax = max(imax, __shfl_xor(imax, 32, 64));
  const float mt = cs * (float)imax;
  if (__ballot(mt > acc.m + kTau)) {
    const float mn = fmaxf(acc.m, mt);
    const float alpha = __builtin_amdgcn_exp2f(acc.m - mn);
#pragma unroll
    for (int t = 0; t < C::DT; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc.o[t][r] *= alpha;
    acc.l *= alpha;
    acc.m = mn;
  }
  const float negm = -acc.m;
  uint32_t pk[C::NT][8];
  float rs = 0.0f;
#pragma unroll
  for (int t = 0; t < C::NT; ++t)
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf((float)s[t][r], cs, negm));
      float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf((float)s[t][r + 1], cs, negm));
      if (tail) {
        if (s[t][r] == INT32_MIN) p0 = 0.0f;
        if (s[t][r + 1] == INT32_MIN) p1 = 0.0f;
      }
      pk[t][r >> 1] = pack_bf16x2(p0, p1);
      // the row sum adds the bf16-rounded P that the PV MFMA consumes, so the
      // normalisation matches the numerator exactly (one v_dot2 per pair)
      rs = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(v2bf, pk[t][r >> 1]), kOnes, rs,
                                           false);
    }
  acc.l += rs;

#pragma unroll
  for (int st = 0; st < C::PS; ++st) {
    const int t = st >> 1, h = st & 1;
    const uint4 bu = make_uint4(pk[t][4 * h], pk[t][4 * h + 1], pk[t][4 * h + 2], pk[t][4 * h + 3]);
    const v8bf b = __builtin_bit_cast(v8bf, bu);
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) {
      const uint16_t* base = lv + (32 * dt + ql) * C::VP + 16 * st + 4 * g;
      const uint2 lo = *reinterpret_cast<const uint2*>(base);
      const uint2 hi = *reinterpret_cast<const uint2*>(base + 8);
      const v8bf a = __builtin_bit_cast(v8bf, make_uint4(lo.x, lo.y, hi.x, hi.y));
      acc.o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc.o[dt], 0, 0, 0);
    }
  }
}

__device__ __forceinline__ float4 load_bf16x4(const uint16_t* p) {
  const uint2 u = *reinterpret_cast<const uint2*>(p);
  return make_float4(bf16_lo(u.x), bf16_hi(u.x), bf16_lo(u.y), bf16_hi(u.y));
}

__device__ __forceinline__ void store_bf16x4(uint16_t* p, float a, float b, float c, float d) {
  *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16x2(a, b), pack_bf16x2(c, d));
}

// Next usable position of a kept list at or after `pos` (entries outside
// [0, nb) are skipped); returns kc when none is left.
__device__ __forceinline__ int next_kept(const int32_t* kl, int pos, int kc, int nb) {
  while (pos < kc) {
    const int j = kl[pos];
    if (j >= 0 && j < nb) break;
    ++pos;
  }
  return pos;
}

template <int BS, int D, bool REFRESH>
__global__ __launch_bounds__((Cfg<BS, D>::THREADS)) void attn_kernel(AttnArgs a, int L, int nb,
                                                                  uint32_t n_work) {
  using C = Cfg<BS, D>;
  __shared__ __attribute__((aligned(16))) int8_t s_k[C::LDS_K];
  __shared__ __attribute__((aligned(16))) uint16_t s_v[C::LDS_V / 2];

  const uint32_t work = xcd_contiguous(blockIdx.x, n_work);
  const uint32_t i = work % (uint32_t)nb;
  const uint64_t bh = work / (uint32_t)nb;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, ql = lane & 31;

  const uint64_t head_off = bh * (uint64_t)L * D;
  const int8_t* kc_h = a.k_codes + head_off;
  const uint16_t* v_h = a.v + head_off;
  const float* sk_h = a.k_scales + bh * (uint64_t)nb;

  // this wave's 32 query rows, as the B operand of S^T = K Q^T
  const int qrow = (int)i * BS + 32 * wave + ql;
  const bool qvalid = qrow < L;
  v4i qb[C::KS];
#pragma unroll
  for (int c = 0; c < C::KS; ++c) {
    qb[c] = qvalid ? *reinterpret_cast<const v4i*>(a.q_codes + head_off + (size_t)qrow * D +
                                                   32 * c + 16 * g)
                   : v4i{0, 0, 0, 0};
  }
  const float c0 = a.sm_scale * a.q_scales[bh * (uint64_t)nb + i] * kLog2e;

  const int32_t* kl = a.kept_idx + (bh * (uint64_t)nb + i) * (uint64_t)a.kmax;
  const int kcnt = min(max(a.kept_cnt[bh * (uint64_t)nb + i], 0), a.kmax);

  Acc<BS, D> acc_k;  // kept blocks (the sparse attention)
  acc_k.init();
  Acc<BS, D> acc_n;  // the other blocks (refresh step only)
  if (REFRESH) acc_n.init();

  Stage<BS, D> st;
  // iteration state: sparse step walks the kept list, refresh walks all blocks
  int pos = 0;
  int cur;
  if (REFRESH) {
    cur = 0;
  } else {
    pos = next_kept(kl, 0, kcnt, nb);
    cur = pos < kcnt ? kl[pos] : -1;
  }
  if (cur >= 0) {
    const int nv = min(BS, L - cur * BS);
    load_stage<BS, D>(st, kc_h + (size_t)cur * BS * D, v_h + (size_t)cur * BS * D, tid, nv);
  }
  int kpos = 0;  // refresh: cursor into the kept list
  while (cur >= 0) {
    __syncthreads();
    store_stage<BS, D>(st, s_k, s_v, tid);
    __syncthreads();
    int nxt;
    if (REFRESH) {
      nxt = cur + 1 < nb ? cur + 1 : -1;
    } else {
      pos = next_kept(kl, pos + 1, kcnt, nb);
      nxt = pos < kcnt ? kl[pos] : -1;
    }
    if (nxt >= 0) {
      const int nv = min(BS, L - nxt * BS);
      load_stage<BS, D>(st, kc_h + (size_t)nxt * BS * D, v_h + (size_t)nxt * BS * D, tid, nv);
    }
    const int nvalid = min(BS, L - cur * BS);
    const float cs = c0 * sk_h[cur];
    if (REFRESH) {
      while (kpos < kcnt && kl[kpos] < cur) ++kpos;
      const bool kept = kpos < kcnt && kl[kpos] == cur;
      if (kept) {
        process_tile<BS, D>(acc_k, qb, s_k, s_v, lane, cs, nvalid);
      } else {
        process_tile<BS, D>(acc_n, qb, s_k, s_v, lane, cs, nvalid);
      }
    } else {
      process_tile<BS, D>(acc_k, qb, s_k, s_v, lane, cs, nvalid);
    }
    cur = nxt;
  }

  // ---- epilogue --------------------------------------------------------------
  const float lk = acc_k.l + __shfl_xor(acc_k.l, 32, 64);
  const float inv_k = lk > 0.0f ? 1.0f / lk : 0.0f;
  float wk = 0.0f, wn = 0.0f, inv_f = 0.0f;
  if (REFRESH) {
    const float ln = acc_n.l + __shfl_xor(acc_n.l, 32, 64);
    const float m = fmaxf(acc_k.m, acc_n.m);
    const float ak = __builtin_amdgcn_exp2f(acc_k.m - m);
    const float an = __builtin_amdgcn_exp2f(acc_n.m - m);
    const float lf = lk * ak + ln * an;
    inv_f = lf > 0.0f ? 1.0f / lf : 0.0f;
    wk = ak * inv_f;
    wn = an * inv_f;
  }
  if (!qvalid) return;
  const size_t row_off = head_off + (size_t)qrow * D;
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt) {
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int d0 = 32 * dt + 8 * r4 + 4 * g;
      float os[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) os[e] = acc_k.o[dt][4 * r4 + e] * inv_k;
      if (!REFRESH) {
        if (a.r_in) {
          const float4 rv = load_bf16x4(a.r_in + row_off + d0);
          os[0] += rv.x; os[1] += rv.y; os[2] += rv.z; os[3] += rv.w;
        }
        if (a.dr_in) {
          const float4 dv = load_bf16x4(a.dr_in + row_off + d0);
          os[0] += dv.x; os[1] += dv.y; os[2] += dv.z; os[3] += dv.w;
        }
        store_bf16x4(a.out + row_off + d0, os[0], os[1], os[2], os[3]);
      } else {
        float of[4], rho[4], drv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          of[e] = acc_k.o[dt][4 * r4 + e] * wk + acc_n.o[dt][4 * r4 + e] * wn;
          rho[e] = of[e] - os[e];
          drv[e] = 0.0f;
        }
        if (a.has_prev) {
          const float4 rp = load_bf16x4(a.r_out + row_off + d0);
          drv[0] = rho[0] - rp.x; drv[1] = rho[1] - rp.y;
          drv[2] = rho[2] - rp.z; drv[3] = rho[3] - rp.w;
        }
        store_bf16x4(a.dr_out + row_off + d0, drv[0], drv[1], drv[2], drv[3]);
        store_bf16x4(a.r_out + row_off + d0, rho[0], rho[1], rho[2], rho[3]);
        store_bf16x4(a.out + row_off + d0, of[0], of[1], of[2], of[3]);
      }
    }
  }
}

template <int BS, int D, bool REFRESH>
hipError_t launch_t(const qsa_dims& d, const AttnArgs& a, hipStream_t s) {
  const int nb = (d.seq_len + BS - 1) / BS;
  const uint32_t n_work = (uint32_t)((uint64_t)d.batch * d.heads * nb);
  hipLaunchKernelGGL((attn_kernel<BS, D, REFRESH>), dim3(n_work), dim3(Cfg<BS, D>::THREADS), 0,
                     s, a, d.seq_len, nb, n_work);
  return hipGetLastError();
}

template <bool REFRESH>
hipError_t dispatch(const qsa_dims& d, const AttnArgs& a, hipStream_t s) {
  if (d.block == 64 && d.head_dim == 128) return launch_t<64, 128, REFRESH>(d, a, s);
  if (d.block == 64 && d.head_dim == 64) return launch_t<64, 64, REFRESH>(d, a, s);
  if (d.block == 128 && d.head_dim == 128) return launch_t<128, 128, REFRESH>(d, a, s);
  return launch_t<128, 64, REFRESH>(d, a, s);
}

}  // namespace

hipError_t launch_sparse_attn(const qsa_dims& d, const AttnArgs& a, hipStream_t s) {
  return dispatch<false>(d, a, s);
}

hipError_t launch_full_attn_residual(const qsa_dims& d, const AttnArgs& a, hipStream_t s) {
  return dispatch<true>(d, a, s);
}

}  // namespace qsa
