// Block saliency and top-k + band selection of the block-sparse mask.
//
// QuantSparse (gist.science/es/paper/2509.23681), technical summary §1 and §4
// (attention kept at ~15 % density) and §2A (average-pooled global guidance,
// top-k salient local guidance): every query block keeps the key blocks whose
// mean-pooled dequantised codes score highest, plus a fixed band of offsets.
//
// One workgroup per (batch*head, tile of TR query blocks): TR = 16 with 8
// waves when the tile's keys fit the LDS (up to 1,216 key blocks; one
// workgroup per CU), else TR = 8 with 4 waves (two per CU) or fewer rows.
//  1. Exact integer scores S_ij = sum_d Pq[i,d] Pk[j,d] on the int8 MFMA:
//     each pooled sum P (|P| <= 127*128) is split into int8 digits
//     P = 128*hi + lo with lo in [0,127], hi in [-127,127], and
//       S = 16384*sum(hi*hi') + 128*(sum(hi*lo') + sum(lo*hi')) + sum(lo*lo')
//     where every partial sum fits int32 and the recombination is exact in
//     fp64 (all values are integers below 2^53).
//  2. score = fl64(fl64(S * sq*sk) / (n_i*n_j)) in IEEE fp64, mapped to an
//     order-preserving uint64 key (-0 canonicalised to +0), kept in LDS.
//  3. Per row (one wave), a radix select finds the k-th largest key.  Its
//     sign class comes first from ballot counts (keys of score >= 0 are
//     >= 2^63): if fewer than k keys are in the upper class, all of them are
//     taken and the rest is chosen in the lower one.  Inside the class,
//     t = key - (smallest key of the class) keeps the order, and the digits
//     (8 bits, the last one shorter) start at the top bit of the class's
//     range, so no pass is spent on the sign and exponent bits most keys
//     share.  The passes stop once the bin holding the k-th key is taken
//     whole; the threshold is then known on its decided bits only.
//  4. Ascending compaction with wave ballots: j is kept if its key is in the
//     class above the candidates', or it is a candidate whose decided bits
//     of t exceed the threshold's, or equal them with fewer than `need`
//     lower-indexed equal candidates before it, or j - i is a band offset.
#include "qsa_internal.h"

#pragma clang fp contract(off)

namespace qsa {
namespace {

constexpr int kSelMaxThreads = 512;
constexpr int kHist = 256;

__device__ __forceinline__ uint64_t order_key(double score) {
  uint64_t b = (uint64_t)__double_as_longlong(score);
  if (score == 0.0) b = 0;  // -0 and +0 are equal scores
  return (b >> 63) ? ~b : (b | 0x8000000000000000ull);
}

// Digits of 16 consecutive pooled sums (four int4 loads; all zero for a
// column past the last block), packed 4 per 32-bit word.
__device__ __forceinline__ void split16(const int4 (&raw)[4], bool valid, v4i& hi, v4i& lo) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    uint32_t h = 0, l = 0;
    const int vv[4] = {raw[w].x, raw[w].y, raw[w].z, raw[w].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int hv = vv[e] >> 7;   // floor division by 128
      const int lv = vv[e] & 127;  // remainder in [0, 127]
      h |= (uint32_t)(hv & 0xff) << (8 * e);
      l |= (uint32_t)lv << (8 * e);
    }
    hi[w] = valid ? (int)h : 0;
    lo[w] = valid ? (int)l : 0;
  }
}

template <int KSTEPS>
__device__ __forceinline__ void load16(const int32_t* __restrict__ p, int4 (&raw)[KSTEPS][4]) {
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks)
#pragma unroll
    for (int w = 0; w < 4; ++w) raw[ks][w] = *reinterpret_cast<const int4*>(p + ks * 64 + 4 * w);
}

__device__ __forceinline__ uint64_t lanemask_lt(int lane) {
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// Calls f(j, valid, key) for the keys of one row in ascending chunks of 64
// (lane l takes j = base + l; every lane of the wave takes part in every
// chunk).  NPL > 0: the lane's keys are in registers kr[e] (j = 64e + lane,
// nb <= 64 * NPL); NPL == 0: they are read from the row in LDS.
template <int NPL, typename F>
__device__ __forceinline__ void each_key(const uint64_t* keys, const uint64_t (&kr)[NPL > 0 ? NPL : 1],
                                         int nb, int lane, F&& f) {
  if constexpr (NPL > 0) {
#pragma unroll
    for (int e = 0; e < NPL; ++e)
      if (64 * e < nb) f(64 * e + lane, 64 * e + lane < nb, kr[e]);
  } else {
    for (int base = 0; base < nb; base += 64) {
      const int j = base + lane;
      f(j, j < nb, j < nb ? keys[j] : 0ull);
    }
  }
}

template <int D, int NPL>
__global__ __launch_bounds__(kSelMaxThreads) void select_kernel(
    const int32_t* __restrict__ pq, const float* __restrict__ sq, const int32_t* __restrict__ pk,
    const float* __restrict__ sk, int L, int bs, int nb, int TR, int topk, Band band, int kmax,
    int32_t* __restrict__ kept_idx, int32_t* __restrict__ kept_cnt) {
  // [TR][nb] keys, then one kHist-bin histogram per wave
  extern __shared__ uint64_t s_keys[];
  const int nwaves = blockDim.x >> 6;
  uint32_t* s_hist_all = reinterpret_cast<uint32_t*>(s_keys + (size_t)TR * nb);

  constexpr int KSTEPS = D / 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t* s_hist = s_hist_all + wave * kHist;
  const uint64_t bh = blockIdx.y;
  const int r0 = blockIdx.x * TR;
  const int32_t* pqh = pq + bh * (uint64_t)nb * D;
  const int32_t* pkh = pk + bh * (uint64_t)nb * D;
  const float* sqh = sq + bh * (uint64_t)nb;
  const float* skh = sk + bh * (uint64_t)nb;

  // ---- 1+2: scores of TR query blocks against every key block -------------
  const int g = lane >> 4;  // k-group of the 16x16x64 MFMA operands
  v4i a_hi[KSTEPS], a_lo[KSTEPS];
  {
    const int arow = lane & 15;
    const int i = r0 + arow;
    const bool ok = arow < TR && i < nb;
    int4 raw[KSTEPS][4];
    load16<KSTEPS>(pqh + (uint64_t)(ok ? i : 0) * D + g * 16, raw);
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) split16(raw[ks], ok, a_hi[ks], a_lo[ks]);
  }
  // this lane's accumulator rows 4g + r: their query scale and token count
  double a_sq[4];
  int a_n[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int i = r0 + 4 * g + r;
    const bool ok = 4 * g + r < TR && i < nb;
    a_sq[r] = ok ? (double)sqh[i] : 0.0;
    a_n[r] = ok ? min(bs, L - i * bs) : 0;
  }
  // Column tiles ct = wave, wave + nwaves, ...; the pooled sums and scale of
  // the next tile are loaded while this one is scored.
  const int n_ctiles = (nb + 15) / 16;
  int4 raw[KSTEPS][4];
  float skv = 0.0f;
  auto fetch = [&](int ct) {
    const int j = min(ct * 16 + (lane & 15), nb - 1);
    load16<KSTEPS>(pkh + (uint64_t)j * D + g * 16, raw);
    skv = skh[j];
  };
  if (wave < n_ctiles) fetch(wave);
  for (int ct = wave; ct < n_ctiles; ct += nwaves) {
    const int j = ct * 16 + (lane & 15);
    const bool okj = j < nb;
    v4i b_hi[KSTEPS], b_lo[KSTEPS];
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) split16(raw[ks], okj, b_hi[ks], b_lo[ks]);
    const double skj = (double)skv;
    if (ct + nwaves < n_ctiles) fetch(ct + nwaves);
    v4i hh = {0, 0, 0, 0}, mid = {0, 0, 0, 0}, ll = {0, 0, 0, 0};
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      hh = __builtin_amdgcn_mfma_i32_16x16x64_i8(a_hi[ks], b_hi[ks], hh, 0, 0, 0);
      mid = __builtin_amdgcn_mfma_i32_16x16x64_i8(a_hi[ks], b_lo[ks], mid, 0, 0, 0);
      mid = __builtin_amdgcn_mfma_i32_16x16x64_i8(a_lo[ks], b_hi[ks], mid, 0, 0, 0);
      ll = __builtin_amdgcn_mfma_i32_16x16x64_i8(a_lo[ks], b_lo[ks], ll, 0, 0, 0);
    }
    if (okj) {
      const int nj = min(bs, L - j * bs);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 4 * g + r;  // accumulator row of this lane
        if (row < TR && r0 + row < nb) {
          const double S = (double)hh[r] * 16384.0 + (double)mid[r] * 128.0 + (double)ll[r];
          const double a = a_sq[r] * skj;
          const double b = S * a;
          const int ci = a_n[r] * nj;
          // a power of two (every pair of full blocks) divides exactly by a
          // multiplication with its inverse: the same IEEE result as b / c
          const double q = (ci & (ci - 1)) == 0 ? b * (1.0 / (double)ci) : b / (double)ci;
          s_keys[(uint64_t)row * nb + j] = order_key(q);
        }
      }
    }
  }
  __syncthreads();

  // ---- 3+4: per-row radix select and ascending compaction -----------------
  const int k_eff = min(topk, nb);
  const int rows_per_wave = (TR + nwaves - 1) / nwaves;
  for (int it = 0; it < rows_per_wave; ++it) {
    const int row = it * nwaves + wave;
    const int i = r0 + row;
    const bool active = row < TR && i < nb;
    const uint64_t* keys = s_keys + (uint64_t)(active ? row : 0) * nb;
    uint64_t kr[NPL > 0 ? NPL : 1];
    if constexpr (NPL > 0) {
#pragma unroll
      for (int e = 0; e < NPL; ++e) {
        const int j = 64 * e + lane;
        kr[e] = j < nb ? keys[j] : 0ull;
      }
    }

    // The k-th largest key is found in its sign class first: with npos keys
    // of score >= 0 (keys >= 2^63), it is among them if npos >= k, else all
    // of them are taken and the rest is chosen among the negative keys.
    // Inside the class, t = key - (smallest key of the class) preserves the
    // order and the radix digits start at the top bit of the class's range,
    // so the first histogram already spreads the keys (the top bits of a
    // key are the sign and the exponent, shared by many keys).
    constexpr uint64_t kSign = 0x8000000000000000ull;
    int need = k_eff;  // how many still to take among the candidates
    const bool do_select = active && k_eff > 0 && k_eff < nb;
    bool pos_class = true;     // candidates: keys >= 2^63, else keys < 2^63
    uint64_t lo = 0;           // smallest candidate key
    uint64_t prefix = 0, pmask = 0;  // decided high bits of t and their value
    int lowbit = 0;            // undecided low bits of t
    if (do_select) {
      int npos = 0;
      each_key<NPL>(keys, kr, nb, lane, [&](int, bool v, uint64_t key) {
        npos += __popcll(__ballot(v && key >= kSign));
      });
      pos_class = npos >= need;
      if (!pos_class) need -= npos;
      uint64_t kmin = ~0ull, kmax_ = 0ull;
      each_key<NPL>(keys, kr, nb, lane, [&](int, bool v, uint64_t key) {
        if (v && (key >= kSign) == pos_class) {
          kmin = key < kmin ? key : kmin;
          kmax_ = key > kmax_ ? key : kmax_;
        }
      });
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) {
        const uint64_t a = __shfl_xor(kmin, o, 64), b = __shfl_xor(kmax_, o, 64);
        kmin = a < kmin ? a : kmin;
        kmax_ = b > kmax_ ? b : kmax_;
      }
      lo = kmin;
      const uint64_t range = kmax_ - kmin;
      lowbit = range ? 64 - __clzll((long long)range) : 0;
      pmask = lowbit == 64 ? 0ull : ~0ull << lowbit;  // bits >= lowbit are 0 for every t
    }
    while (lowbit > 0) {
      const int width = min(8, lowbit);
      const int shift = lowbit - width;
      const uint64_t dmask = (1ull << width) - 1;
      // The histogram is this wave's own: LDS operations of one wave are
      // performed in order, so waiting for them (lgkmcnt) orders the zeroing,
      // the counting and the reads without a workgroup barrier.
#pragma unroll
      for (int e = 0; e < 4; ++e) s_hist[lane * 4 + e] = 0;
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
      __builtin_amdgcn_wave_barrier();
      each_key<NPL>(keys, kr, nb, lane, [&](int, bool v, uint64_t key) {
        const uint64_t t = key - lo;
        if (v && (key >= kSign) == pos_class && (t & pmask) == prefix)
          atomicAdd(&s_hist[(t >> shift) & dmask], 1u);
      });
      __builtin_amdgcn_s_waitcnt(0xc07f);
      __builtin_amdgcn_wave_barrier();
      uint32_t c[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) c[e] = s_hist[lane * 4 + e];
      const uint32_t mine = c[0] + c[1] + c[2] + c[3];
      // inclusive suffix sum over lanes (lanes >= this one)
      uint32_t suf = mine;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t v = __shfl_down(suf, o, 64);
        if (lane + o < 64) suf += v;
      }
      const uint32_t above = suf - mine;  // candidates in higher digit bins
      const bool here = above < (uint32_t)need && (uint32_t)need <= suf;
      int digit = 0;
      uint32_t cnt_above = above;
      if (here) {
        for (int e = 3; e >= 0; --e) {
          if (cnt_above + c[e] >= (uint32_t)need) {
            digit = lane * 4 + e;
            break;
          }
          cnt_above += c[e];
        }
      }
      const uint64_t who = __ballot(here);
      const int src = __ffsll((unsigned long long)who) - 1;
      digit = __shfl(digit, src, 64);
      cnt_above = __shfl(cnt_above, src, 64);
      const uint32_t in_bin = s_hist[digit];
      need -= (int)cnt_above;
      prefix |= (uint64_t)digit << shift;
      pmask |= dmask << shift;
      lowbit = shift;
      // every candidate of the chosen bin is taken: no finer digit can matter
      if ((uint32_t)need == in_bin) break;
    }

    if (active) {
      int32_t* out = kept_idx + ((bh * (uint64_t)nb) + i) * (uint64_t)kmax;
      int pos = 0, ties_seen = 0;
      each_key<NPL>(keys, kr, nb, lane, [&](int j, bool valid, uint64_t key) {
        bool in_band = false;
        for (int b = 0; b < band.n; ++b) in_band |= (j - i) == band.off[b];
        bool sel;
        if (k_eff == 0) {
          sel = false;
        } else if (k_eff == nb) {
          sel = true;
        } else {
          // keys of the class above the candidates' are all taken; the
          // candidates compare on the decided digits only (all of them unless
          // the select stopped at a bin taken whole)
          const bool in_cls = (key >= kSign) == pos_class;
          const uint64_t mk = (key - lo) & pmask;
          const bool eq = in_cls && mk == prefix;
          const uint64_t eqb = __ballot(valid && eq);
          const int rank = ties_seen + __popcll(eqb & lanemask_lt(lane));
          sel = (!pos_class && key >= kSign) || (in_cls && mk > prefix) || (eq && rank < need);
          ties_seen += __popcll(eqb);
        }
        sel = valid && (sel || in_band);
        const uint64_t selb = __ballot(sel);
        const int p = pos + __popcll(selb & lanemask_lt(lane));
        if (sel && p < kmax) out[p] = j;
        pos += __popcll(selb);
      });
      for (int p = pos + lane; p < kmax; p += 64) out[p] = -1;
      if (lane == 0) kept_cnt[bh * (uint64_t)nb + i] = min(pos, kmax);
    }
  }
}

}  // namespace

namespace {
template <int D, int NPL>
void launch_select_kernel(dim3 grid, int threads, size_t lds, size_t lds_cap, hipStream_t s,
                          const int32_t* pooled_q, const float* scale_q, const int32_t* pooled_k,
                          const float* scale_k, const qsa_dims& d, int nb, int TR, int topk,
                          const Band& band, int kmax, int32_t* kept_idx, int32_t* kept_cnt) {
  // set once per kernel (a function-local static is initialised exactly once,
  // also when several host threads launch at the same time)
  static const hipError_t attr = hipFuncSetAttribute(
      (const void*)select_kernel<D, NPL>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_cap);
  (void)attr;
  hipLaunchKernelGGL((select_kernel<D, NPL>), grid, dim3(threads), lds, s, pooled_q, scale_q,
                     pooled_k, scale_k, d.seq_len, d.block, nb, TR, topk, band, kmax, kept_idx,
                     kept_cnt);
}

// keys per lane held in registers during the select: the smallest of 16, 24,
// 32 that covers the row; longer rows are read from LDS
template <int D>
void launch_select_d(dim3 grid, int threads, size_t lds, size_t lds_cap, hipStream_t s,
                     const int32_t* pooled_q, const float* scale_q, const int32_t* pooled_k,
                     const float* scale_k, const qsa_dims& d, int nb, int TR, int topk,
                     const Band& band, int kmax, int32_t* kept_idx, int32_t* kept_cnt) {
#define QSA_SEL_LAUNCH(NPL)                                                                   \
  launch_select_kernel<D, NPL>(grid, threads, lds, lds_cap, s, pooled_q, scale_q, pooled_k, scale_k, d, \
                               nb, TR, topk, band, kmax, kept_idx, kept_cnt)
  if (nb <= 64 * 16)
    QSA_SEL_LAUNCH(16);
  else if (nb <= 64 * 24)
    QSA_SEL_LAUNCH(24);
  else if (nb <= 64 * 32)
    QSA_SEL_LAUNCH(32);
  else
    QSA_SEL_LAUNCH(0);
#undef QSA_SEL_LAUNCH
}
}  // namespace

hipError_t launch_select(const qsa_dims& d, const int32_t* pooled_q, const float* scale_q,
                         const int32_t* pooled_k, const float* scale_k, int32_t topk,
                         const Band& band, int32_t kmax, int32_t* kept_idx, int32_t* kept_cnt,
                         hipStream_t s) {
  const int nb = (d.seq_len + d.block - 1) / d.block;
  // 16 query blocks and 8 waves per workgroup when their keys and histograms
  // fit the LDS (one workgroup per CU; the pooled K sums are split once per 16
  // rows), else 8 blocks and 4 waves (two per CU), fewer for long sequences
  const size_t lds_cap = 160 * 1024;
  auto lds_of = [&](int tr, int threads) {
    return (size_t)tr * nb * sizeof(uint64_t) + (size_t)(threads / 64) * kHist * sizeof(uint32_t);
  };
  int TR = 16, threads = kSelMaxThreads;
  if (lds_of(TR, threads) > lds_cap) {
    TR = 8;
    threads = 256;
    while (TR > 1 && lds_of(TR, threads) > lds_cap) TR >>= 1;
  }
  const size_t lds = lds_of(TR, threads);
  if (lds > lds_cap) return hipErrorInvalidValue;
  const dim3 grid((nb + TR - 1) / TR, (uint32_t)(d.batch * d.heads));
  if (d.head_dim == 128)
    launch_select_d<128>(grid, threads, lds, lds_cap, s, pooled_q, scale_q, pooled_k, scale_k, d, nb, TR,
                         topk, band, kmax, kept_idx, kept_cnt);
  else
    launch_select_d<64>(grid, threads, lds, lds_cap, s, pooled_q, scale_q, pooled_k, scale_k, d, nb, TR,
                        topk, band, kmax, kept_idx, kept_cnt);
  return hipGetLastError();
}

}  // namespace qsa
