// Block saliency and top-k + band selection of the block-sparse mask.
//
// QuantSparse (gist.science/es/paper/2509.23681), technical summary §1 and §4
// (attention kept at ~15 % density) and §2A (average-pooled global guidance,
// top-k salient local guidance): every query block keeps the key blocks whose
// mean-pooled dequantised codes score highest, plus a fixed band of offsets.
//
// Two ways to run it, with the same scores, keys and selection code, so the
// same kept lists bit for bit:
//  * qsa_select_blocks: one workgroup per (batch*head, tile of TR query
//    blocks), TR = 16 with 8 waves when the tile's keys fit the LDS (up to
//    1,216 key blocks; one workgroup per CU), else TR = 8 with 4 waves or
//    fewer rows; the keys stay in LDS between scoring and selection.
//  * qsa_select_blocks_work: the keys of whole (batch, head) slices go to a
//    caller workspace (score_keys_kernel, many workgroups per CU), then one
//    wave per query block selects from them (select_rows_kernel).
// The steps:
//  1. Exact integer scores S_ij = sum_d Pq[i,d] Pk[j,d] on the int8 MFMA:
//     each pooled sum P (|P| <= 127*128) is split into int8 digits
//     P = 128*hi + lo with lo in [0,127], hi in [-127,127], and
//       S = 16384*sum(hi*hi') + 128*(sum(hi*lo') + sum(lo*hi')) + sum(lo*lo')
//     where every partial sum fits int32 and the recombination is exact in
//     fp64 (all values are integers below 2^53).
//  2. score = fl64(fl64(S * sq*sk) / (n_i*n_j)) in IEEE fp64 (a power-of-two
//     count as an exact ldexp), mapped to an order-preserving uint64 key (-0
//     canonicalised to +0).
//  3. Per row (one wave), a radix select finds the k-th largest key, on the
//     keys' high 32 bits first (a monotone function of the key); the slots
//     tied there are ordered by their low halves.  The sign class comes first
//     from ballot counts (keys of score >= 0 have the top bit set): if fewer
//     than k keys are in the upper class, all of them are taken and the rest
//     is chosen in the lower one.  Inside the class, t = hi - (smallest high
//     half of the class) keeps the order, and the digits (8 bits, the last
//     one shorter) start at the top bit of the class's range, so no pass is
//     spent on the sign and exponent bits most keys share.  The passes stop
//     once the bin holding the k-th key is taken whole; the threshold is
//     then known on its decided bits only.
//  4. Ascending compaction with wave ballots: j is kept if its key is in the
//     class above the candidates', or it is a candidate whose decided bits
//     exceed the threshold's, or equal them with fewer than `need`
//     lower-indexed equal candidates before it, or j - i is a band offset.
// Rows of more than 2,048 key blocks take the one-pass kernel and the same
// steps on full 64-bit keys read from LDS each pass.
#include "qsa_internal.h"

#pragma clang fp contract(off)

namespace qsa {
namespace {

constexpr int kSelMaxThreads = 512;
// waves per SIMD the row-select kernel is compiled for (its register budget)
#ifndef QSA_SEL_ROWS_WAVES
#define QSA_SEL_ROWS_WAVES 4
#endif
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

// Order keys of one 16-column tile of scores: this lane's accumulator rows
// 4g + r (r = 0..3) of the row block whose pooled-Q digits are a_hi/a_lo,
// against column j (pooled-K digits b_hi/b_lo, scale skj, nj tokens).
// a_sq[r] and a_n[r] are the rows' query scales and token counts.
template <int KSTEPS>
__device__ __forceinline__ void score_tile(const v4i (&a_hi)[KSTEPS], const v4i (&a_lo)[KSTEPS],
                                           const v4i (&b_hi)[KSTEPS], const v4i (&b_lo)[KSTEPS],
                                           double skj, int nj, const double (&a_sq)[4],
                                           const int (&a_n)[4], uint64_t (&key)[4]) {
  v4i hh = {0, 0, 0, 0}, mid = {0, 0, 0, 0}, ll = {0, 0, 0, 0};
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks) {
    hh = __builtin_amdgcn_mfma_i32_16x16x64_i8(a_hi[ks], b_hi[ks], hh, 0, 0, 0);
    mid = __builtin_amdgcn_mfma_i32_16x16x64_i8(a_hi[ks], b_lo[ks], mid, 0, 0, 0);
    mid = __builtin_amdgcn_mfma_i32_16x16x64_i8(a_lo[ks], b_hi[ks], mid, 0, 0, 0);
    ll = __builtin_amdgcn_mfma_i32_16x16x64_i8(a_lo[ks], b_lo[ks], ll, 0, 0, 0);
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const double S = (double)hh[r] * 16384.0 + (double)mid[r] * 128.0 + (double)ll[r];
    const double a = a_sq[r] * skj;
    const double b = S * a;
    const int ci = a_n[r] * nj;
    // a power of two 2^e (every pair of full blocks) divides exactly as a
    // scaling by 2^-e: the same IEEE result as b / c (b's magnitude is far
    // from the subnormal range); other counts (short last blocks) divide
    double q = 0.0;
    if (__builtin_expect(ci > 0 && (ci & (ci - 1)) == 0, 1))
      q = __builtin_ldexp(b, -__builtin_ctz((unsigned)ci));
    else if (ci > 0)
      q = b / (double)ci;
    key[r] = order_key(q);
  }
}

// The pooled-Q digits, scales and token counts of the lane's rows of the row
// block starting at query block r0 (rows past nb or past tr are zero).
template <int KSTEPS>
__device__ __forceinline__ void load_rows(const int32_t* __restrict__ pqh,
                                          const float* __restrict__ sqh, int r0, int tr, int nb,
                                          int L, int bs, int lane, v4i (&a_hi)[KSTEPS],
                                          v4i (&a_lo)[KSTEPS], double (&a_sq)[4], int (&a_n)[4]) {
  constexpr int D = KSTEPS * 64;
  const int g = lane >> 4;
  const int arow = lane & 15;
  const int i = r0 + arow;
  const bool ok = arow < tr && i < nb;
  int4 raw[KSTEPS][4];
  load16<KSTEPS>(pqh + (uint64_t)(ok ? i : 0) * D + g * 16, raw);
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks) split16(raw[ks], ok, a_hi[ks], a_lo[ks]);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int ir = r0 + 4 * g + r;
    const bool okr = 4 * g + r < tr && ir < nb;
    a_sq[r] = okr ? (double)sqh[ir] : 0.0;
    a_n[r] = okr ? min(bs, L - ir * bs) : 0;
  }
}

// Top-k + band selection of query block i from its nb keys (kr in registers
// when NPL > 0, else keys[j]), written ascending to out (kmax entries, -1
// padded) with the count to *cnt.  Every lane of the wave takes part;
// s_hist is this wave's own kHist-bin histogram.
//
// The k-th largest key is found in its sign class first: with npos keys of
// score >= 0 (keys >= 2^63), it is among them if npos >= k, else all of them
// are taken and the rest is chosen among the negative keys.  Inside the
// class, t = key - (smallest key of the class) preserves the order and the
// radix digits start at the top bit of the class's range, so the first
// histogram already spreads the keys (the top bits of a key are the sign and
// the exponent, shared by many keys).
template <int NPL>
__device__ __forceinline__ void select_row_lds(const uint64_t* keys,
                                           const uint64_t (&kr)[NPL > 0 ? NPL : 1], int nb,
                                           int lane, uint32_t* s_hist, int i, int topk,
                                           const Band& band, int kmax, int32_t* out,
                                           int32_t* cnt) {
  const int k_eff = min(topk, nb);
  constexpr uint64_t kSign = 0x8000000000000000ull;
  int need = k_eff;  // how many still to take among the candidates
  const bool do_select = k_eff > 0 && k_eff < nb;
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
  if (lane == 0) *cnt = min(pos, kmax);
}

// Radix select among the slots of a bitmask (bit e: slot e) over 32-bit
// values t[e] < 2^lowbit: narrows (prefix, pmask), the decided high bits,
// to the bin that holds the need-th largest value, with 8-bit digits from
// the top.  On return `need` counts what is still to take from the slots
// equal to prefix on pmask, and `whole` says that all of them are taken.
// SENTINEL: slots outside `cand` hold t = ~0, which never matches a prefix
// (lowbit < 32: pmask keeps bit 31 and prefix leaves it 0), so the mask need
// not be tested.  The histogram is this wave's own: its LDS operations are
// performed in order, so waits (lgkmcnt) order them without barriers.
template <int NPL, bool SENTINEL>
__device__ __forceinline__ void radix32(const uint32_t (&t)[NPL], uint32_t cand, int n_cand,
                                        int nb, int lane, uint32_t* s_hist, int lowbit,
                                        int& need, uint32_t& prefix, uint32_t& pmask,
                                        bool& whole) {
  prefix = 0;
  pmask = lowbit >= 32 ? 0u : ~0u << lowbit;
  int in_set = n_cand;  // slots equal to prefix on pmask
  while (lowbit > 0) {
    const int width = min(8, lowbit);
    const int shift = lowbit - width;
    const uint32_t dmask = (1u << width) - 1u;
#pragma unroll
    for (int e = 0; e < 4; ++e) s_hist[lane * 4 + e] = 0;
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int e = 0; e < NPL; ++e)
      if (64 * e < nb && (SENTINEL || ((cand >> e) & 1u)) && (t[e] & pmask) == prefix)
        atomicAdd(&s_hist[(t[e] >> shift) & dmask], 1u);
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_wave_barrier();
    uint32_t c[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) c[e] = s_hist[lane * 4 + e];
    const uint32_t mine = c[0] + c[1] + c[2] + c[3];
    uint32_t suf = mine;  // inclusive suffix sum over lanes
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t v = __shfl_down(suf, o, 64);
      if (lane + o < 64) suf += v;
    }
    const uint32_t above = suf - mine;
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
    in_set = (int)s_hist[digit];
    need -= (int)cnt_above;
    prefix |= (uint32_t)digit << shift;
    pmask |= dmask << shift;
    lowbit = shift;
    if (need == in_set) break;  // every slot of the chosen bin is taken
  }
  whole = need == in_set;
}

// The smallest and largest of t[e] over the slots of `cand`, across the wave.
template <int NPL>
__device__ __forceinline__ void range32(const uint32_t (&t)[NPL], uint32_t cand, uint32_t& mn,
                                        uint32_t& mx) {
  mn = ~0u;
  mx = 0u;
#pragma unroll
  for (int e = 0; e < NPL; ++e)
    if ((cand >> e) & 1u) {
      mn = min(mn, t[e]);
      mx = max(mx, t[e]);
    }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    mn = min(mn, (uint32_t)__shfl_xor((int)mn, o, 64));
    mx = max(mx, (uint32_t)__shfl_xor((int)mx, o, 64));
  }
}

__device__ __forceinline__ int popc_wave(uint32_t bits, int e) {
  return __popcll(__ballot((bits >> e) & 1u));
}

// The selection of select_row_lds with the keys split in halves: hi[e] in
// registers, the high 32 bits of slot e's order key (0 for j >= nb; hi is
// overwritten), and lo_of(e), its low 32 bits, read only for the slots whose
// high halves tie at the k-th place.  The high half is a monotone function
// of the key, so every slot whose high half is above the k-th largest high
// half is kept and every slot below it is not; the slots equal to it are
// ordered by their low halves (equal full keys by index).  All arithmetic is
// 32-bit.  Per-slot conditions are per-lane bitmasks (bit e: slot e).
template <int NPL, typename LoOf>
__device__ __forceinline__ void select_row_split(uint32_t (&hi)[NPL], LoOf&& lo_of, int nb,
                                                 int lane, uint32_t* s_hist, int i, int topk,
                                                 const Band& band, int kmax, int32_t* out,
                                                 int32_t* cnt) {
  static_assert(NPL > 0 && NPL <= 32, "one bit per slot");
  constexpr uint32_t kSign = 0x80000000u;
  const int k_eff = min(topk, nb);
  uint32_t vbits = 0;  // slots j < nb
#pragma unroll
  for (int e = 0; e < NPL; ++e)
    if (64 * e + lane < nb) vbits |= 1u << e;
  const bool do_select = k_eff > 0 && k_eff < nb;
  int need = k_eff;
  uint32_t cbits = 0, abits = 0;     // candidate class / the class above it
  uint32_t prefix = 0, pmask = 0;    // stage A: decided bits of t = hi - min
  bool whole = true;
  uint32_t ebits = 0;                // stage B: slots tied on all 32 high bits
  uint32_t lo[NPL];
  uint32_t prefix2 = 0, pmask2 = 0;  // stage B: decided bits of t2 = lo - min
  bool stage_b = false;
  if (do_select) {
    int npos = 0;
#pragma unroll
    for (int e = 0; e < NPL; ++e)
      if (64 * e < nb) npos += __popcll(__ballot(hi[e] >= kSign));  // hi 0: not counted
    const bool pos_class = npos >= need;
    if (!pos_class) need -= npos;
    int n_cls = 0;
#pragma unroll
    for (int e = 0; e < NPL; ++e) {
      const bool up = hi[e] >= kSign;
      cbits |= (uint32_t)(((vbits >> e) & 1u) && up == pos_class) << e;
      abits |= (uint32_t)(!pos_class && up) << e;
    }
#pragma unroll
    for (int e = 0; e < NPL; ++e)
      if (64 * e < nb) n_cls += popc_wave(cbits, e);
    uint32_t mn, mx;
    range32<NPL>(hi, cbits, mn, mx);
    const uint32_t range = mx - mn;  // < 2^31: one sign class
    const int lowbit = range ? 32 - __clz((int)range) : 0;
#pragma unroll
    for (int e = 0; e < NPL; ++e) hi[e] = ((cbits >> e) & 1u) ? hi[e] - mn : ~0u;
    radix32<NPL, true>(hi, cbits, n_cls, nb, lane, s_hist, lowbit, need, prefix, pmask, whole);
    if (!whole) {
      // every high bit is decided: the tied slots, ordered by their low halves
      stage_b = true;
      int n_e = 0;
#pragma unroll
      for (int e = 0; e < NPL; ++e) {
        const bool tied = ((cbits >> e) & 1u) && hi[e] == prefix;
        ebits |= (uint32_t)tied << e;
        lo[e] = tied ? lo_of(e) : 0u;
      }
#pragma unroll
      for (int e = 0; e < NPL; ++e)
        if (64 * e < nb) n_e += popc_wave(ebits, e);
      uint32_t mn2, mx2;
      range32<NPL>(lo, ebits, mn2, mx2);
      const uint32_t range2 = mx2 - mn2;
      const int lowbit2 = range2 ? 32 - __clz((int)range2) : 0;
#pragma unroll
      for (int e = 0; e < NPL; ++e) lo[e] = lo[e] - mn2;
      bool whole2;
      radix32<NPL, false>(lo, ebits, n_e, nb, lane, s_hist, lowbit2, need, prefix2, pmask2,
                          whole2);
    }
  }

  uint32_t bbits = 0;  // band slots of this lane
  for (int b = 0; b < band.n; ++b) {
    const int jb = i + band.off[b];
    if (jb >= 0 && jb < nb && (jb & 63) == lane) bbits |= 1u << (jb >> 6);
  }
  int pos = 0, ties_seen = 0;
#pragma unroll
  for (int e = 0; e < NPL; ++e) {
    if (64 * e >= nb) break;  // wave-uniform
    const int j = 64 * e + lane;
    bool sel;
    if (k_eff == 0) {
      sel = false;
    } else if (k_eff == nb) {
      sel = true;
    } else {
      const bool in_cls = (cbits >> e) & 1u;
      const uint32_t mk = hi[e] & pmask;
      bool eq;
      if (!stage_b) {
        sel = ((abits >> e) & 1u) || (in_cls && mk > prefix);
        eq = in_cls && mk == prefix;
      } else {
        const bool tied = (ebits >> e) & 1u;
        const uint32_t mk2 = lo[e] & pmask2;
        sel = ((abits >> e) & 1u) || (in_cls && mk > prefix) || (tied && mk2 > prefix2);
        eq = tied && mk2 == prefix2;
      }
      const uint64_t eqb = __ballot(eq);
      const int rank = ties_seen + __popcll(eqb & lanemask_lt(lane));
      sel = sel || (eq && rank < need);
      ties_seen += __popcll(eqb);
    }
    sel = ((vbits >> e) & 1u) && (sel || ((bbits >> e) & 1u));
    const uint64_t selb = __ballot(sel);
    const int p = pos + __popcll(selb & lanemask_lt(lane));
    if (sel && p < kmax) out[p] = j;
    pos += __popcll(selb);
  }
  for (int p = pos + lane; p < kmax; p += 64) out[p] = -1;
  if (lane == 0) *cnt = min(pos, kmax);
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
  double a_sq[4];  // this lane's accumulator rows 4g + r: query scale, tokens
  int a_n[4];
  load_rows<KSTEPS>(pqh, sqh, r0, TR, nb, L, bs, lane, a_hi, a_lo, a_sq, a_n);
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
    uint64_t key[4];
    score_tile<KSTEPS>(a_hi, a_lo, b_hi, b_lo, skj, okj ? min(bs, L - j * bs) : 0, a_sq, a_n,
                       key);
    if (okj) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 4 * g + r;  // accumulator row of this lane
        if (row < TR && r0 + row < nb) s_keys[(uint64_t)row * nb + j] = key[r];
      }
    }
  }
  __syncthreads();

  // ---- 3+4: per-row radix select and ascending compaction -----------------
  const int rows_per_wave = (TR + nwaves - 1) / nwaves;
  for (int it = 0; it < rows_per_wave; ++it) {
    const int row = it * nwaves + wave;
    const int i = r0 + row;
    if (!(row < TR && i < nb)) continue;  // wave-uniform
    const uint64_t* keys = s_keys + (uint64_t)row * nb;
    const uint64_t rowi = bh * (uint64_t)nb + i;
    if constexpr (NPL > 0) {
      uint32_t hi[NPL];
#pragma unroll
      for (int e = 0; e < NPL; ++e) {
        const int j = 64 * e + lane;
        hi[e] = j < nb ? (uint32_t)(keys[j] >> 32) : 0u;
      }
      select_row_split<NPL>(
          hi, [&](int e) { return (uint32_t)keys[64 * e + lane]; }, nb, lane, s_hist, i, topk,
          band, kmax, kept_idx + rowi * (uint64_t)kmax, kept_cnt + rowi);
    } else {
      uint64_t kr[1];
      select_row_lds<NPL>(keys, kr, nb, lane, s_hist, i, topk, band, kmax,
                          kept_idx + rowi * (uint64_t)kmax, kept_cnt + rowi);
    }
  }
}

// Keys per row of the workspace: nb rounded up to 16, so that the 16 keys a
// column tile writes to a row fill one aligned 128-byte line.
__host__ __device__ inline int key_stride(int nb) { return (nb + 15) & ~15; }

// Scores of whole (b, h) slices as order keys in `keys` ([slice][nb][stride],
// slice = bh - bh0).  A workgroup takes 64 query blocks (16 per wave) and the
// column tiles [ct0, ct1) of its share (blockIdx.z of n_split); each pooled-K
// tile of 16 key blocks is read once per workgroup with 16-byte loads that
// cover whole rows, staged in LDS (rows padded by 16 bytes, two buffers, one
// barrier per tile) and read from there in the MFMA operand layout.
template <int D>
__global__ __launch_bounds__(256) void score_keys_kernel(
    const int32_t* __restrict__ pq, const float* __restrict__ sq, const int32_t* __restrict__ pk,
    const float* __restrict__ sk, int L, int bs, int nb, uint64_t bh0, int n_split,
    uint64_t* __restrict__ keys) {
  constexpr int KSTEPS = D / 64;
  constexpr int ROWB = D + 16;                   // bytes per padded LDS digit row
  constexpr int CHUNKS = 16 * D / 4;             // int4 pieces of a tile
  constexpr int PER_T = CHUNKS / 256;            // pieces per thread
  static_assert(CHUNKS % 256 == 0, "whole pieces per thread");
  // the tile's pooled-K sums as their two int8 digits (split16's), one plane each
  __shared__ __attribute__((aligned(16))) int8_t s_hi[2][16 * ROWB];
  __shared__ __attribute__((aligned(16))) int8_t s_lo[2][16 * ROWB];
  __shared__ float s_sk[2][16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint64_t bh = bh0 + blockIdx.y;
  const int32_t* pkh = pk + bh * (uint64_t)nb * D;
  const float* skh = sk + bh * (uint64_t)nb;
  const int ks_row = key_stride(nb);
  uint64_t* kh = keys + (uint64_t)blockIdx.y * nb * ks_row;
  const int r0 = blockIdx.x * 64 + wave * 16;
  const int g = lane >> 4, jj = lane & 15;
  const int n_ct = (nb + 15) / 16;
  const int per = (n_ct + n_split - 1) / n_split;
  const int ct0 = blockIdx.z * per, ct1 = min(n_ct, ct0 + per);
  if (ct0 >= ct1) return;  // workgroup-uniform, before any barrier

  v4i a_hi[KSTEPS], a_lo[KSTEPS];
  double a_sq[4];
  int a_n[4];
  load_rows<KSTEPS>(pq + bh * (uint64_t)nb * D, sq + bh * (uint64_t)nb, r0, 16, nb, L, bs, lane,
                    a_hi, a_lo, a_sq, a_n);

  int4 stage[PER_T];
  float sk_stage = 0.0f;
  auto fetch = [&](int ct) {  // this thread's pieces of tile ct (columns past nb: row nb - 1)
#pragma unroll
    for (int m = 0; m < PER_T; ++m) {
      const int q = tid + 256 * m;
      const int j = min(ct * 16 + q / (D / 4), nb - 1);
      stage[m] = *reinterpret_cast<const int4*>(pkh + (uint64_t)j * D + 4 * (q % (D / 4)));
    }
    if (tid < 16) sk_stage = skh[min(ct * 16 + tid, nb - 1)];
  };
  auto put = [&](int buf) {  // split once per workgroup: P = 128 hi + lo, lo in [0, 127]
#pragma unroll
    for (int m = 0; m < PER_T; ++m) {
      const int q = tid + 256 * m;
      const int off = (q / (D / 4)) * ROWB + 4 * (q % (D / 4));
      const int vv[4] = {stage[m].x, stage[m].y, stage[m].z, stage[m].w};
      uint32_t h = 0, l = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        h |= (uint32_t)((vv[e] >> 7) & 0xff) << (8 * e);
        l |= (uint32_t)(vv[e] & 127) << (8 * e);
      }
      *reinterpret_cast<uint32_t*>(&s_hi[buf][off]) = h;
      *reinterpret_cast<uint32_t*>(&s_lo[buf][off]) = l;
    }
    if (tid < 16) s_sk[buf][tid] = sk_stage;
  };
  fetch(ct0);
  put(0);
  __syncthreads();
  int buf = 0;
  for (int ct = ct0; ct < ct1; ++ct) {
    if (ct + 1 < ct1) fetch(ct + 1);  // lands while this tile is scored
    const int j = ct * 16 + jj;
    const bool okj = j < nb;
    v4i b_hi[KSTEPS], b_lo[KSTEPS];
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      const int off = jj * ROWB + ks * 64 + g * 16;
      b_hi[ks] = *reinterpret_cast<const v4i*>(&s_hi[buf][off]);
      b_lo[ks] = *reinterpret_cast<const v4i*>(&s_lo[buf][off]);
    }
    const double skj = (double)s_sk[buf][jj];
    uint64_t key[4];
    score_tile<KSTEPS>(a_hi, a_lo, b_hi, b_lo, skj, okj ? min(bs, L - j * bs) : 0, a_sq, a_n,
                       key);
    if (okj) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = r0 + 4 * g + r;
        if (i < nb) kh[(uint64_t)i * ks_row + j] = key[r];
      }
    }
    if (ct + 1 < ct1) put(buf ^ 1);  // that buffer was last read before the previous barrier
    __syncthreads();
    buf ^= 1;
  }
}

// Selection from the keys of score_keys_kernel: one wave per query block,
// the high halves of its keys kept in registers (nb <= 64 * NPL), the low
// halves read again (from L2) only for ties, one histogram per wave.
template <int NPL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(QSA_SEL_ROWS_WAVES))) void select_rows_kernel(
    const uint64_t* __restrict__ keys, int nb, uint64_t bh0, int topk, Band band, int kmax,
    int32_t* __restrict__ kept_idx, int32_t* __restrict__ kept_cnt) {
  static_assert(NPL > 0, "keys in registers");
  __shared__ uint32_t s_hist_all[4 * kHist];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i = blockIdx.x * 4 + wave;
  if (i >= nb) return;  // wave-uniform; no workgroup barrier follows
  const uint64_t* row = keys + ((uint64_t)blockIdx.y * nb + i) * key_stride(nb);
  uint32_t hi[NPL];
#pragma unroll
  for (int e = 0; e < NPL; ++e) {
    const int j = 64 * e + lane;
    hi[e] = j < nb ? (uint32_t)(row[j] >> 32) : 0u;
  }
  const uint64_t rowi = (bh0 + blockIdx.y) * (uint64_t)nb + i;
  select_row_split<NPL>(
      hi, [&](int e) { return (uint32_t)row[64 * e + lane]; }, nb, lane, s_hist_all + wave * kHist, i,
      topk, band, kmax, kept_idx + rowi * (uint64_t)kmax, kept_cnt + rowi);
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

uint64_t select_slice_bytes(const qsa_dims& d) {
  const uint64_t nb = (uint64_t)((d.seq_len + d.block - 1) / d.block);
  return nb * (uint64_t)key_stride((int)nb) * sizeof(uint64_t);
}

namespace {
template <int D, int NPL>
void launch_two_pass(const qsa_dims& d, int nb, uint64_t bh0, uint32_t n, const int32_t* pooled_q,
                     const float* scale_q, const int32_t* pooled_k, const float* scale_k,
                     int32_t topk, const Band& band, int32_t kmax, int32_t* kept_idx,
                     int32_t* kept_cnt, uint64_t* keys, hipStream_t s) {
  // column shares per row block: about 4096 workgroups per pass
  const int rb = (nb + 63) / 64, n_ct = (nb + 15) / 16;
  const uint64_t want = (4096 + (uint64_t)rb * n - 1) / ((uint64_t)rb * n);
  const int n_split = (int)(want < 1 ? 1 : want > (uint64_t)n_ct ? n_ct : want);
  hipLaunchKernelGGL((score_keys_kernel<D>), dim3((uint32_t)rb, n, (uint32_t)n_split), dim3(256),
                     0, s, pooled_q, scale_q, pooled_k, scale_k, d.seq_len, d.block, nb, bh0,
                     n_split, keys);
  hipLaunchKernelGGL((select_rows_kernel<NPL>), dim3((uint32_t)((nb + 3) / 4), n), dim3(256), 0, s,
                     (const uint64_t*)keys, nb, bh0, topk, band, kmax, kept_idx, kept_cnt);
}
}  // namespace

hipError_t launch_select_work(const qsa_dims& d, const int32_t* pooled_q, const float* scale_q,
                              const int32_t* pooled_k, const float* scale_k, int32_t topk,
                              const Band& band, int32_t kmax, int32_t* kept_idx,
                              int32_t* kept_cnt, void* work, uint64_t work_bytes,
                              hipStream_t s) {
  const int nb = (d.seq_len + d.block - 1) / d.block;
  const uint64_t slice = select_slice_bytes(d);
  const uint64_t n_bh = (uint64_t)d.batch * d.heads;
  const uint64_t per = work ? work_bytes / slice : 0;
  if (nb > 64 * 32 || per == 0)
    return launch_select(d, pooled_q, scale_q, pooled_k, scale_k, topk, band, kmax, kept_idx,
                         kept_cnt, s);
  const uint64_t chunk = per < n_bh ? (per < 65535 ? per : 65535) : (n_bh < 65535 ? n_bh : 65535);
  uint64_t* keys = static_cast<uint64_t*>(work);
  for (uint64_t bh0 = 0; bh0 < n_bh; bh0 += chunk) {
    const uint32_t n = (uint32_t)(n_bh - bh0 < chunk ? n_bh - bh0 : chunk);
#define QSA_TWO_PASS(DD, NPL)                                                                    \
  launch_two_pass<DD, NPL>(d, nb, bh0, n, pooled_q, scale_q, pooled_k, scale_k, topk, band, kmax, \
                           kept_idx, kept_cnt, keys, s)
    if (d.head_dim == 128) {
      if (nb <= 64 * 16) QSA_TWO_PASS(128, 16);
      else if (nb <= 64 * 24) QSA_TWO_PASS(128, 24);
      else QSA_TWO_PASS(128, 32);
    } else {
      if (nb <= 64 * 16) QSA_TWO_PASS(64, 16);
      else if (nb <= 64 * 24) QSA_TWO_PASS(64, 24);
      else QSA_TWO_PASS(64, 32);
    }
#undef QSA_TWO_PASS
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace qsa
