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
//  * one workgroup per (batch*head, group of QB consecutive query blocks),
//    BS/32 waves per query block; a wave owns 32 query rows and keeps their
//    Q codes in registers.  The kept sets of the group's blocks are turned
//    into bitmaps over the key blocks in LDS and the group walks their union
//    once, in ascending order: a key tile kept by several blocks of the group
//    is loaded once (neighbouring query blocks keep overlapping key sets), and
//    a wave computes only the tiles its own block keeps;
//  * key blocks are walked as 64-key tiles (a 128-token block is two tiles).
//    Per tile the K codes [64 x D] int8 and V [64 x D] bf16 go HBM/L2 -> LDS
//    with 16-byte direct-to-LDS loads (no register staging), rows
//    XOR-swizzled at 16-byte granularity so the operand reads are free of
//    bank conflicts.  Either each wave copies its MFMA operands of the tile
//    into registers right away, so the single LDS tile is refilled with the
//    next tile while this one is computed, or (64-token blocks, D = 128) the
//    tile has two LDS buffers and the operands are read where they are used,
//    which frees the registers for a third wave per SIMD.  That walk takes
//    its tiles from a list built once per phase from the bitmaps (one LDS
//    read per tile) and loads them through buffer descriptors of the head's
//    K and V (the tile is a scalar offset; no vector address arithmetic);
//  * S^T = K_j . Q^T on v_mfma_i32_32x32x32_i8 (exact int32 dots);
//  * logits z = (sm_scale * sq_i * sk_j * log2 e) * S and softmax in fp32
//    with exp2.  The running max is computed on the first tile only; later
//    tiles exponentiate against it directly and the per-lane sum of the tile
//    (which bounds every P) tells whether the max must move (sum > 2^64):
//    only then is the tile max taken and the state rescaled.  Online
//    softmax is exact in real arithmetic for any max used, so this only
//    removes per-element max work;
//  * P is rounded to bf16 straight from the S^T accumulator registers (their
//    layout is the B operand of the next MFMA, no LDS round trip); the
//    denominator sums the same bf16-rounded P (v_dot2_f32_bf16), and
//    O^T += V^T . P^T on v_mfma_f32_32x32x16_bf16 with fp32 accumulation,
//    the V^T operand read from the row-major V tile with ds_read_b64_tr_b16;
//  * the epilogue normalises, adds the cached residuals (sparse step) or
//    forms the residuals (refresh step), and stores bf16.
// The refresh step runs one online-softmax state over the kept blocks (the
// sparse attention), parks that normalised output in its own output rows,
// then continues the same state over every other block (the full
// attention): the two share every exponential and MFMA of the kept tiles.
#include "qsa_internal.h"
#include "quant_codes.h"

#ifndef QSA_ATTN_QB
#define QSA_ATTN_QB 2
#endif
// the kernels of 64-token blocks and D = 128 walk with two LDS tile buffers
// at three waves per SIMD (0: one buffer, operands copied to registers, two
// waves per SIMD)
#ifndef QSA_ATTN_JIT
#define QSA_ATTN_JIT 1
#endif
#ifndef QSA_ATTN_JIT_WAVES
#define QSA_ATTN_JIT_WAVES 3
#endif

namespace qsa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRsLimit = 18446744073709551616.0f;  // 2^64: bound on any P of a tile
constexpr v2bf kOnes = {(__bf16)1.0f, (__bf16)1.0f};
constexpr int KT = 64;  // keys per tile

// A read-only fp32 array read at a wave-uniform index through the constant
// address space, so it becomes a scalar load: it then waits on the scalar
// counter only, not on the vector-memory counter that also tracks the tile
// loads in flight.
__device__ __forceinline__ float load_uniform(const float* p, int i) {
  typedef __attribute__((address_space(4))) const float cf32;
  return ((cf32*)p)[__builtin_amdgcn_readfirstlane(i)];
}

template <int BS, int D>
struct Cfg {
  static constexpr int WPB = BS / 32;  // waves per query block (32 rows each)
  static constexpr int SUB = BS / KT;  // tiles per key block
  static constexpr int NT = KT / 32;   // 32-key accumulator tiles per tile
  static constexpr int DT = D / 32;    // 32-channel output tiles
  static constexpr int KS = D / 32;    // 32-channel steps of the QK^T MFMA
  static constexpr int PS = KT / 16;   // 16-key steps of the PV MFMA
  static constexpr int K_BYTES = KT * D;
  static constexpr int V_BYTES = KT * D * 2;
  static constexpr int K_CPR = D / 16;  // 16-byte chunks per K row
  static constexpr int V_CPR = D / 8;   // 16-byte chunks per V row
  static constexpr int K_ROWS_PER_KB = 1024 / D;
  static constexpr int V_ROWS_PER_KB = 512 / D;
};

// Each of the NWV waves of a workgroup issues an equal share of a tile's 1 KB
// direct-to-LDS loads.
template <int D, int NWV>
struct Dma {
  static constexpr int K = KT * D / 1024 / NWV;
  static constexpr int V = KT * D * 2 / 1024 / NWV;
  static_assert(K >= 1 && V >= 1 && K * NWV * 1024 == KT * D && V * NWV * 1024 == KT * D * 2,
                "tile loads must split evenly over the waves");
};

// Chunk swizzles: 16-byte chunk p of tile row r holds logical chunk p ^ swz(r).
// K rows are D bytes (256/D rows share one 256-byte bank line); V rows 2D bytes.
template <int D>
__device__ __forceinline__ int kswz(int r) {
  return (r / (256 / D)) & (D / 16 - 1);
}
// A transpose read of the V^T operand touches, per 32 lanes, 4 consecutive
// rows x 4 consecutive chunks; XOR-ing the chunk quad with the row (D = 128:
// one row per 256-byte bank line) or with the bank-line index (D = 64: two
// rows per line) puts the 16 chunks on distinct banks.
template <int D>
__device__ __forceinline__ int vswz(int r) {
  return D == 128 ? ((r & 3) << 2) : (((r >> 1) & 1) << 2);
}

// Enqueue the direct-to-LDS loads of one tile (rows past the sequence end
// re-read the last valid row: finite values that the softmax masks).
template <int BS, int D, int NWV>
__device__ __forceinline__ void dma_tile(const int8_t* __restrict__ kt,
                                         const uint16_t* __restrict__ vt, int8_t* lk,
                                         uint16_t* lv, int wave, int lane, int nvalid) {
  using C = Cfg<BS, D>;
  using M = Dma<D, NWV>;
#pragma unroll
  for (int n = 0; n < M::K; ++n) {
    const int kb = wave * M::K + n;
    const int row = kb * C::K_ROWS_PER_KB + lane / C::K_CPR;
    const int p = lane % C::K_CPR;
    const int src = min(row, nvalid - 1);
    const int8_t* g = kt + (size_t)src * D + ((p ^ kswz<D>(row)) << 4);
    __builtin_amdgcn_global_load_lds(g, (lds_void_t*)(lk + kb * 1024), 16, 0, 0);
  }
#pragma unroll
  for (int n = 0; n < M::V; ++n) {
    const int kb = wave * M::V + n;
    const int row = kb * C::V_ROWS_PER_KB + lane / C::V_CPR;
    const int p = lane % C::V_CPR;
    const int src = min(row, nvalid - 1);
    const uint16_t* g = vt + (size_t)src * D + ((p ^ vswz<D>(row)) << 3);
    __builtin_amdgcn_global_load_lds(g, (lds_void_t*)(lv + kb * 512), 16, 0, 0);
  }
}

// The same loads for whole tiles through buffer descriptors of the head's K
// codes and V: each lane's byte offset inside a tile does not depend on the
// tile, so it is computed once, and the tile enters as a scalar offset; the
// tile loop then spends no vector instructions on addresses.
template <int BS, int D, int NWV>
struct BufDma {
  using C = Cfg<BS, D>;
  using M = Dma<D, NWV>;
  __amdgpu_buffer_rsrc_t rk, rv;
  uint32_t ok[M::K], ov[M::V];
  __device__ __forceinline__ void init(const int8_t* kc_h, const uint16_t* v_h, int L, int wave,
                                       int lane) {
    // raw buffers (stride 0) of L rows; a descriptor word 3 of 0x00020000
    // selects 32-bit untyped access on this architecture
    rk = __builtin_amdgcn_make_buffer_rsrc((void*)kc_h, 0, L * D, 0x00020000);
    rv = __builtin_amdgcn_make_buffer_rsrc((void*)v_h, 0, L * D * 2, 0x00020000);
#pragma unroll
    for (int n = 0; n < M::K; ++n) {
      const int kb = wave * M::K + n;
      const int row = kb * C::K_ROWS_PER_KB + lane / C::K_CPR;
      ok[n] = (uint32_t)(row * D + (((lane % C::K_CPR) ^ kswz<D>(row)) << 4));
    }
#pragma unroll
    for (int n = 0; n < M::V; ++n) {
      const int kb = wave * M::V + n;
      const int row = kb * C::V_ROWS_PER_KB + lane / C::V_CPR;
      ov[n] = (uint32_t)(2 * (row * D + (((lane % C::V_CPR) ^ vswz<D>(row)) << 3)));
    }
  }
  // all KT rows of tile t (t * KT + KT <= L)
  __device__ __forceinline__ void tile(int t, int8_t* lk, uint16_t* lv, int wave) const {
#pragma unroll
    for (int n = 0; n < M::K; ++n)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void_t*)(lk + (wave * M::K + n) * 1024),
                                               16, ok[n], t * (KT * D), 0, 0);
#pragma unroll
    for (int n = 0; n < M::V; ++n)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void_t*)(lv + (wave * M::V + n) * 512),
                                               16, ov[n], t * (KT * D * 2), 0, 0);
  }
};

// Per-lane LDS byte offsets of the MFMA operands (the swizzle of a lane's rows
// does not depend on the tile, so these are computed once).
template <int BS, int D>
struct LaneOffs {
  int k[Cfg<BS, D>::KS];  // K operand of K-step c, key rows 0..31
  int v[Cfg<BS, D>::DT];  // V^T operand of channel tile dt, key step 0, half 0
  __device__ __forceinline__ void init(int lane) {
    using C = Cfg<BS, D>;
    const int g = lane >> 5, r = lane & 31;
#pragma unroll
    for (int c = 0; c < C::KS; ++c) k[c] = r * D + (((g * C::KS + c) ^ kswz<D>(r)) << 4);
    // ds_read_b64_tr_b16 in 16-lane groups: out lane i element e comes from
    // source lane (i>>2) + 4e, element i&3.  Source lane 16G+j points at
    // V[key 4(G>>1) + (j>>2)][d 32dt + 16(G&1) + 4(j&3)], so out lane l holds
    // V[keys 4g + 0..3][d = 32dt + l%32]: the A operand of the PV MFMA.
    const int G = lane >> 4, j = lane & 15;
    const int r0 = 4 * (G >> 1) + (j >> 2);
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) {
      const int chunk = 4 * dt + 2 * (G & 1) + ((j & 3) >> 1);
      v[dt] = r0 * (2 * D) + ((chunk ^ vswz<D>(r0)) << 4) + 8 * (j & 1);
    }
  }
};

// Online-softmax state of one query row (held by lanes l and l^32).
template <int BS, int D>
struct Acc {
  v16f o[Cfg<BS, D>::DT];
  float m;
  float l;
  bool started;
  __device__ __forceinline__ void init() {
#pragma unroll
    for (int t = 0; t < Cfg<BS, D>::DT; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[t][r] = 0.0f;
    m = -__builtin_inff();
    l = 0.0f;
    started = false;
  }
};

__device__ __forceinline__ bool key_valid(int t, int r, int g, int nvalid) {
  return 32 * t + 8 * (r >> 2) + 4 * g + (r & 3) < nvalid;
}

// P = exp2(S * cs - m) as packed bf16 pairs; returns the lane's sum of the
// rounded P.
template <int BS, int D, bool TAIL>
__device__ __forceinline__ float exp_pack(const v16i (&s)[Cfg<BS, D>::NT],
                                          uint32_t (&pk)[Cfg<BS, D>::NT][8], float cs,
                                          float negm, int g, int nvalid) {
  using C = Cfg<BS, D>;
  float rs = 0.0f;
#pragma unroll
  for (int t = 0; t < C::NT; ++t)
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf((float)s[t][r], cs, negm));
      float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf((float)s[t][r + 1], cs, negm));
      if (TAIL) {
        if (!key_valid(t, r, g, nvalid)) p0 = 0.0f;
        if (!key_valid(t, r + 1, g, nvalid)) p1 = 0.0f;
      }
      pk[t][r >> 1] = pack_bf16x2(p0, p1);
      rs = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(v2bf, pk[t][r >> 1]), kOnes, rs,
                                           false);
    }
  return rs;
}

template <int BS, int D, bool TAIL>
__device__ __forceinline__ float tile_max(const v16i (&s)[Cfg<BS, D>::NT], float cs, int g,
                                          int nvalid) {
  using C = Cfg<BS, D>;
  int imax = INT32_MIN;
#pragma unroll
  for (int t = 0; t < C::NT; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (!TAIL || key_valid(t, r, g, nvalid)) imax = max(imax, s[t][r]);
  imax = max(imax, __shfl_xor(imax, 32, 64));
  return cs * (float)imax;
}

// The V^T operand of 16-key step st and channel tile dt from the LDS tile.
template <int BS, int D>
__device__ __forceinline__ v8bf v_operand(const LaneOffs<BS, D>& lo, const uint16_t* lv, int st,
                                          int dt) {
  const char* base = reinterpret_cast<const char*>(lv) + 16 * st * (2 * D) + lo.v[dt];
  const v4s lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_t*)(base));
  const v4s hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_t*)(base + 8 * (2 * D)));
  const uint2 ul = __builtin_bit_cast(uint2, lo4), uh = __builtin_bit_cast(uint2, hi4);
  return __builtin_bit_cast(v8bf, make_uint4(ul.x, ul.y, uh.x, uh.y));
}

// MFMA operands of one tile held in registers, so the LDS tile can be
// refilled with the next tile while this one is computed.
template <int BS, int D>
struct Ops {
  v4i k[Cfg<BS, D>::NT][Cfg<BS, D>::KS];   // A operands of S^T = K Q^T
  v8bf v[Cfg<BS, D>::PS][Cfg<BS, D>::DT];  // A operands of O^T += V^T P^T
};

template <int BS, int D>
__device__ __forceinline__ void load_ops(Ops<BS, D>& op, const LaneOffs<BS, D>& lo,
                                         const int8_t* lk, const uint16_t* lv) {
  using C = Cfg<BS, D>;
#pragma unroll
  for (int t = 0; t < C::NT; ++t)
#pragma unroll
    for (int c = 0; c < C::KS; ++c)
      op.k[t][c] = *reinterpret_cast<const v4i*>(lk + 32 * t * D + lo.k[c]);
#pragma unroll
  for (int st = 0; st < C::PS; ++st)
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) op.v[st][dt] = v_operand<BS, D>(lo, lv, st, dt);
}

// S^T = K . Q^T for this wave's 32 query rows: s[t][r] holds
// S[query lane%32][key 32t + 8(r/4) + 4g + r%4] (exact int32).
template <int BS, int D>
__device__ __forceinline__ void qk(const v4i (&kop)[Cfg<BS, D>::NT][Cfg<BS, D>::KS],
                                   const v4i (&qb)[Cfg<BS, D>::KS], v16i (&s)[Cfg<BS, D>::NT]) {
  using C = Cfg<BS, D>;
#pragma unroll
  for (int t = 0; t < C::NT; ++t) {
#pragma unroll
    for (int r = 0; r < 16; ++r) s[t][r] = 0;
#pragma unroll
    for (int c = 0; c < C::KS; ++c)
      s[t] = __builtin_amdgcn_mfma_i32_32x32x32_i8(kop[t][c], qb[c], s[t], 0, 0, 0);
  }
}

// Softmax update for one tile whose scores s are in registers: P = exp2(S cs
// - m) packed to bf16 in pk, running sum and (rarely) max updated.  TAIL: the
// tile is the short last one of the sequence (keys >= nvalid are masked);
// every other tile runs without masking work.  kglob: the tile's K codes in
// global memory, used only to recompute the scores when the running max has
// to move up (rare).
template <int BS, int D, bool TAIL>
__device__ __forceinline__ void softmax_update(Acc<BS, D>& acc, const v16i (&s)[Cfg<BS, D>::NT],
                                               uint32_t (&pk)[Cfg<BS, D>::NT][8],
                                               const v4i (&qb)[Cfg<BS, D>::KS],
                                               const int8_t* __restrict__ kglob, int lane,
                                               float cs, int nvalid) {
  using C = Cfg<BS, D>;
  const int g = lane >> 5;
  if (!acc.started) {
    acc.m = tile_max<BS, D, TAIL>(s, cs, g, nvalid);
    acc.started = true;
  }
  float rs = exp_pack<BS, D, TAIL>(s, pk, cs, -acc.m, g, nvalid);
  if (__ballot(!(rs <= kRsLimit))) {
    // The running max moved up by a lot: rescale the state to the new max and
    // redo the tile, with the K operand reloaded from global memory (this
    // lane's rows of K in the channel order of qb; rows past the end clamp).
    v16i s2[C::NT];
#pragma unroll
    for (int t = 0; t < C::NT; ++t) {
      const int row = min(32 * t + (lane & 31), nvalid - 1);
#pragma unroll
      for (int r = 0; r < 16; ++r) s2[t][r] = 0;
#pragma unroll
      for (int c = 0; c < C::KS; ++c) {
        // one operand at a time: this path must not raise register pressure
        const v4i ka =
            *reinterpret_cast<const v4i*>(kglob + (size_t)row * D + g * (D / 2) + 16 * c);
        s2[t] = __builtin_amdgcn_mfma_i32_32x32x32_i8(ka, qb[c], s2[t], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    const float mn = fmaxf(acc.m, tile_max<BS, D, TAIL>(s2, cs, g, nvalid));
    const float alpha = __builtin_amdgcn_exp2f(acc.m - mn);
#pragma unroll
    for (int t = 0; t < C::DT; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc.o[t][r] *= alpha;
    acc.l *= alpha;
    acc.m = mn;
    rs = exp_pack<BS, D, TAIL>(s2, pk, cs, -acc.m, g, nvalid);
  }
  acc.l += rs;
}

template <int BS, int D>
__device__ __forceinline__ v8bf pk_operand(const uint32_t (&pk)[Cfg<BS, D>::NT][8], int st) {
  const int t = st >> 1, h = st & 1;
  const uint4 bu = make_uint4(pk[t][4 * h], pk[t][4 * h + 1], pk[t][4 * h + 2], pk[t][4 * h + 3]);
  return __builtin_bit_cast(v8bf, bu);
}

// O^T += V^T P^T with the V operands already in registers.
template <int BS, int D>
__device__ __forceinline__ void pv_regs(Acc<BS, D>& acc,
                                        const v8bf (&vop)[Cfg<BS, D>::PS][Cfg<BS, D>::DT],
                                        const uint32_t (&pk)[Cfg<BS, D>::NT][8]) {
  using C = Cfg<BS, D>;
#pragma unroll
  for (int st = 0; st < C::PS; ++st) {
    const v8bf b = pk_operand<BS, D>(pk, st);
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt)
      acc.o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop[st][dt], b, acc.o[dt], 0, 0, 0);
  }
}

// O^T += V^T P^T reading the V operands from the LDS tile, one 16-key step
// ahead of the MFMAs that consume them (the reads of step st+1 are in
// flight while the MFMAs of step st run).
template <int BS, int D>
__device__ __forceinline__ void pv_lds(Acc<BS, D>& acc, const LaneOffs<BS, D>& lo,
                                       const uint16_t* lv,
                                       const uint32_t (&pk)[Cfg<BS, D>::NT][8]) {
  using C = Cfg<BS, D>;
  v8bf va[C::DT], vb[C::DT];
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt) va[dt] = v_operand<BS, D>(lo, lv, 0, dt);
#pragma unroll
  for (int st = 0; st < C::PS; ++st) {
    if (st + 1 < C::PS) {
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt) vb[dt] = v_operand<BS, D>(lo, lv, st + 1, dt);
    }
    const v8bf b = pk_operand<BS, D>(pk, st);
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt)
      acc.o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[dt], b, acc.o[dt], 0, 0, 0);
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) va[dt] = vb[dt];
  }
}

template <int BS, int D, bool TAIL>
__device__ __forceinline__ void softmax_pv(Acc<BS, D>& acc, const v16i (&s)[Cfg<BS, D>::NT],
                                           const v8bf (&vop)[Cfg<BS, D>::PS][Cfg<BS, D>::DT],
                                           const v4i (&qb)[Cfg<BS, D>::KS],
                                           const int8_t* __restrict__ kglob, int lane, float cs,
                                           int nvalid) {
  uint32_t pk[Cfg<BS, D>::NT][8];
  softmax_update<BS, D, TAIL>(acc, s, pk, qb, kglob, lane, cs, nvalid);
  pv_regs<BS, D>(acc, vop, pk);
}

__device__ __forceinline__ float4 load_bf16x4(const uint16_t* p) {
  const uint2 u = *reinterpret_cast<const uint2*>(p);
  return make_float4(bf16_lo(u.x), bf16_hi(u.x), bf16_lo(u.y), bf16_hi(u.y));
}

__device__ __forceinline__ void store_bf16x4(uint16_t* p, float a, float b, float c, float d) {
  *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16x2(a, b), pack_bf16x2(c, d));
}

// Windowed mode with bf16 Q: the codes of this wave's 32 query rows (the B
// operand layout of S^T = K Q^T) formed here as qsa_quantize forms them: the
// block's amax over its rows (the BS/32 waves of a block exchange theirs
// through LDS, one barrier for the workgroup), s = fl32(amax / 127), each
// code rounded by codes8.  Row qrow of the sequence is token qrow, or with
// a.q_pm_w > 0 the position-major row of windows of a.q_pm_w tokens (token
// (qrow % m) * q_pm_w + qrow / m, m = L / q_pm_w).  Rows past L are zero.
// Returns s.
template <int BS, int D>
__device__ __forceinline__ float quantize_q_rows(const AttnArgs& a, v4i (&qb)[Cfg<BS, D>::KS],
                                                 uint64_t head_off, int qrow, bool qvalid, int L,
                                                 int lane, int wave, float* s_qmax) {
  using C = Cfg<BS, D>;
  const int g = lane >> 5;
  int tok = qrow;
  if (a.q_pm_w > 0) {
    const int m = L / a.q_pm_w;
    tok = (qrow % m) * a.q_pm_w + qrow / m;
  }
  const uint16_t* src = a.q_x + head_off + (size_t)tok * D + g * (D / 2);
  float y[C::KS][2][8];
  float amax = 0.0f;
#pragma unroll
  for (int c = 0; c < C::KS; ++c)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint4 r = qvalid ? *reinterpret_cast<const uint4*>(src + 16 * c + 8 * h)
                             : make_uint4(0u, 0u, 0u, 0u);
      const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        y[c][h][2 * e] = bf16_lo(w[e]);
        y[c][h][2 * e + 1] = bf16_hi(w[e]);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(y[c][h][e]));
    }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
  if (lane == 0) s_qmax[wave] = amax;
  __syncthreads();
  const int w0 = (wave / C::WPB) * C::WPB;
  amax = 0.0f;
#pragma unroll
  for (int w = 0; w < C::WPB; ++w) amax = fmaxf(amax, s_qmax[w0 + w]);
  const float s = amax / 127.0f;  // IEEE division; 0 for an all-zero block
  const bool fast = s >= 0x1p-100f;
  const float inv = fast ? 1.0f / s : 0.0f;
#pragma unroll
  for (int c = 0; c < C::KS; ++c) {
    uint32_t lo[2], hi[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float q[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
      if (s > 0.0f) codes8(y[c][h], s, inv, fast, q);
      uint32_t pairs[4];
      pack_codes(q, lo[h], hi[h], pairs);
    }
    qb[c] = v4i{(int)lo[0], (int)hi[0], (int)lo[1], (int)hi[1]};
  }
  return s;
}

// Kept sets of the query blocks of a workgroup as bitmaps over the key blocks,
// in LDS: bit j of row b is set when key block j is in kept(i) of the group's
// b-th query block i.  Row b holds words [b*nw, (b+1)*nw) of one array sized
// for the largest block count (nw = words per row).  The tile walks below read
// them a 32-bit word at a time.
constexpr int kMaxWords = QSA_MAX_BLOCKS / 32;

template <int QB, int THREADS, typename BlockAt>
__device__ __forceinline__ void build_kept_bits(uint32_t* bits, const AttnArgs& a,
                                                uint64_t row0, BlockAt&& block_at, int nq,
                                                int nb, int tid) {
  const int nw = (nb + 31) >> 5;
  for (int k = tid; k < QB * nw; k += THREADS) bits[k] = 0u;
  __syncthreads();
  for (int b = 0; b < nq; ++b) {
    const int blk = block_at(b);
    if (blk < 0) continue;
    const uint64_t row = row0 + blk;
    const int32_t* kl = a.kept_idx + row * (uint64_t)a.kmax;
    // the count and the entries are read together (one memory round trip);
    // entries past the count are ignored
    const int cnt_raw = a.kept_cnt[row];
    for (int p = tid; p < a.kmax; p += THREADS) {
      const int j = kl[p];
      const int cnt = min(max(cnt_raw, 0), a.kmax);
      if (p < cnt && j >= 0 && j < nb) atomicOr(&bits[b * nw + (j >> 5)], 1u << (j & 31));
    }
  }
  __syncthreads();
}

// The group's tiles of one phase as one ascending list in LDS, for groups of
// two query blocks of 64 tokens: the kept tiles (rest = false) or the tiles
// outside the kept sets (rest = true), each present when at least one block
// needs it; entry = tile | needed(block 0) << 14 | needed(block 1) << 15
// (tiles < 16384).  The short last tile is left out; its presence and need
// bits go to info[1] (bit 0: present; bits 1, 2: needed by block 0, 1).
// info[0] = the list length, also when it exceeds cap (then the list is
// incomplete and the bitmap walk is used).  Built by wave 0 from the bitmaps.
// Walking the list costs one LDS read and a few scalar instructions per tile,
// where the bitmap walk scans and refills words with branches and waits.
__device__ __forceinline__ void build_seq(const uint32_t* bits, int nb, int nq, int tail_t,
                                          bool rest, uint16_t* seq, int cap, int* info,
                                          int tid) {
  if (tid >= 64) return;
  const int lane = tid;
  const int nw = (nb + 31) >> 5;
  const int last_bits = nb - 32 * (nw - 1);
  int base = 0, tl = 0;
  for (int w0 = 0; w0 < nw; w0 += 64) {
    const int w = w0 + lane;
    uint32_t b0 = 0u, b1 = 0u;
    if (w < nw) {
      b0 = bits[w];
      if (nq > 1) b1 = bits[nw + w];
      if (rest) {
        const uint32_t valid = w == nw - 1 && last_bits < 32 ? (1u << last_bits) - 1u : ~0u;
        b0 = ~b0 & valid;
        b1 = nq > 1 ? ~b1 & valid : 0u;
      }
    }
    uint32_t u = b0 | b1;
    if (tail_t >= 0 && (tail_t >> 5) == w) {
      const int tb = tail_t & 31;
      tl = (int)((u >> tb) & 1u) | (int)(((b0 >> tb) & 1u) << 1) | (int)(((b1 >> tb) & 1u) << 2);
      u &= ~(1u << tb);
    }
    const int c = __popc(u);
    int incl = c;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(incl, o, 64);
      if (lane >= o) incl += v;
    }
    int pos = base + incl - c;
    while (u) {
      const int bit = __builtin_ctz(u);
      u &= u - 1u;
      if (pos < cap)
        seq[pos] = (uint16_t)((w << 5) + bit) | (uint16_t)(((b0 >> bit) & 1u) << 14) |
                   (uint16_t)(((b1 >> bit) & 1u) << 15);
      ++pos;
    }
    base += __shfl(incl, 63, 64);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) tl |= __shfl_xor(tl, o, 64);
  if (lane == 0) {
    info[0] = base;
    info[1] = tl;
  }
}

// Walk, in ascending order, over the 64-key tiles of the key blocks that at
// least one query block of the group needs: the kept blocks (rest = false) or
// the blocks outside the kept set (rest = true, the refresh step's other
// half).  Every wave of the workgroup produces the same tile sequence; `keep`
// tells a wave whether its own query block needs the tile.  The short last
// tile of the sequence is not returned: tail_hit / tail_keep record it.
template <int QB, int SUB>
struct BitWalk {
  const uint32_t* bits;
  int nw, nq, myb, n_tiles, tail_t, last_bits;
  int wi, base, j, sub;
  uint32_t u, mine;
  bool rest, kj, tail_hit, tail_keep;

  __device__ __forceinline__ void init(const uint32_t* b, int nb, int nq_, int myb_,
                                       int n_tiles_, int tail_t_, bool rest_) {
    bits = b;
    rest = rest_;
    nw = (nb + 31) >> 5;
    nq = nq_;
    myb = myb_;
    n_tiles = n_tiles_;
    tail_t = tail_t_;
    last_bits = nb - 32 * (nw - 1);
    wi = 0;
    base = 0;
    j = 0;
    sub = 0;
    u = 0u;
    mine = 0u;
    kj = false;
    tail_hit = false;
    tail_keep = false;
  }
  __device__ __forceinline__ uint32_t row_word(int b, int w) const {
    uint32_t v = bits[b * nw + w];
    if (rest) {
      const uint32_t valid = w == nw - 1 && last_bits < 32 ? (1u << last_bits) - 1u : ~0u;
      v = ~v & valid;
    }
    return v;
  }
  __device__ __forceinline__ void load_word() {
    uint32_t un = 0u;
#pragma unroll
    for (int b = 0; b < QB; ++b)
      if (b < nq) un |= row_word(b, wi);
    u = __builtin_amdgcn_readfirstlane(un);
    mine = myb >= 0 ? __builtin_amdgcn_readfirstlane(row_word(myb, wi)) : 0u;
    base = wi << 5;
    ++wi;
  }
  // next tile index (wave-uniform), -1 at the end
  __device__ __forceinline__ int next(bool& keep) {
    while (true) {
      if (sub == 0) {
        while (u == 0u) {
          if (wi >= nw) return -1;
          load_word();
        }
        const int bit = __builtin_ctz(u);
        u &= u - 1u;
        j = base + bit;
        kj = (mine >> bit) & 1u;
      }
      const int t = j * SUB + sub;
      if (++sub == SUB) sub = 0;
      if (t >= n_tiles) continue;  // empty second half of a short last block
      if (t == tail_t) {
        tail_hit = true;
        tail_keep = kj;
        continue;
      }
      keep = kj;
      return t;
    }
  }
};

// Shared per-workgroup context of the tile loop.
template <int BS, int D>
struct Ctx {
  const int8_t* kc_h;
  const uint16_t* v_h;
  const float* sk_h;
  int8_t* s_k;   // LDS tile buffer 0
  uint16_t* s_v;
  int L;
  int wave, lane;
  float c0;
};

// Run the online softmax of `acc` over the tiles produced by next() (64-key
// tile indices, -1 at the end), with the next tile's loads in flight while
// the current one is computed.  Every wave loads its share of each tile; a
// wave computes only the tiles its query block keeps.  next() never returns
// the short last tile.
template <int BS, int D, int NWV, typename Next>
__device__ __forceinline__ void walk(const Ctx<BS, D>& x, const v4i (&qb)[Cfg<BS, D>::KS],
                                     const LaneOffs<BS, D>& lo, Acc<BS, D>& acc, Next&& next) {
  using C = Cfg<BS, D>;
  auto dma = [&](int t) {
    dma_tile<BS, D, NWV>(x.kc_h + (size_t)t * KT * D, x.v_h + (size_t)t * KT * D, x.s_k, x.s_v,
                         x.wave, x.lane, KT);
  };
  bool keep = false;
  int cur = next(keep);
  if (cur < 0) return;
  __syncthreads();  // the LDS tile is free
  dma(cur);
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): this wave's loads landed in LDS
  __syncthreads();                     // and every other wave's
  while (cur >= 0) {
    cur = __builtin_amdgcn_readfirstlane(cur);  // wave-uniform: scalar loads
    Ops<BS, D> op;
    v16i s[C::NT];
    float cs = 0.0f;
    if (keep) {
      cs = x.c0 * load_uniform(x.sk_h, cur / C::SUB);
      load_ops<BS, D>(op, lo, x.s_k, x.s_v);
      qk<BS, D>(op.k, qb, s);
    }
    __syncthreads();  // every wave holds its operands: the LDS tile is free
    bool knext = false;
    const int nxt = next(knext);
    if (nxt >= 0) dma(nxt);  // lands while this tile is computed
    if (keep)
      softmax_pv<BS, D, false>(acc, s, op.v, qb, x.kc_h + (size_t)cur * KT * D, x.lane, cs, KT);
    __builtin_amdgcn_s_waitcnt(0x0f70);  // the next tile landed in LDS
    __syncthreads();
    cur = nxt;
    keep = knext;
  }
}

#if QSA_ATTN_JIT
// The walk with two LDS tile buffers and the MFMA operands read from LDS
// right where they are used (no register copy of the tile): the registers
// freed let three waves share a SIMD, which hides more of the gather and
// dependency latency.  Tile n is computed from buffer n % 2 while tile n+1
// loads into the other; one barrier per tile.
template <int BS, int D, int NWV, typename Next>
__device__ __forceinline__ void walk_jit(const Ctx<BS, D>& x, const v4i (&qb)[Cfg<BS, D>::KS],
                                         const LaneOffs<BS, D>& lo, Acc<BS, D>& acc,
                                         Next&& next) {
  using C = Cfg<BS, D>;
  BufDma<BS, D, NWV> bd;
  bd.init(x.kc_h, x.v_h, x.L, x.wave, x.lane);
  auto dma = [&](int t, int buf) {
    bd.tile(t, x.s_k + buf * C::K_BYTES, x.s_v + buf * (C::V_BYTES / 2), x.wave);
  };
  bool keep = false;
  int cur = next(keep);
  if (cur < 0) return;
  __syncthreads();  // both buffers are free
  dma(cur, 0);
  __builtin_amdgcn_s_waitcnt(0x0f70);
  __syncthreads();
  int buf = 0;
  while (cur >= 0) {
    cur = __builtin_amdgcn_readfirstlane(cur);
    bool knext = false;
    const int nxt = next(knext);
    if (nxt >= 0) dma(nxt, buf ^ 1);  // every wave is done with that buffer
    if (keep) {
      const float cs = x.c0 * load_uniform(x.sk_h, cur / C::SUB);
      const int8_t* lk = x.s_k + buf * C::K_BYTES;
      const uint16_t* lv = x.s_v + buf * (C::V_BYTES / 2);
      v16i s[C::NT];
#pragma unroll
      for (int t = 0; t < C::NT; ++t) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[t][r] = 0;
#pragma unroll
        for (int c = 0; c < C::KS; ++c)
          s[t] = __builtin_amdgcn_mfma_i32_32x32x32_i8(
              *reinterpret_cast<const v4i*>(lk + 32 * t * D + lo.k[c]), qb[c], s[t], 0, 0, 0);
      }
      uint32_t pk[C::NT][8];
      softmax_update<BS, D, false>(acc, s, pk, qb, x.kc_h + (size_t)cur * KT * D, x.lane, cs,
                                   KT);
#pragma unroll
      for (int st = 0; st < C::PS; ++st) {
        const v8bf b = pk_operand<BS, D>(pk, st);
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt)
          acc.o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v_operand<BS, D>(lo, lv, st, dt),
                                                              b, acc.o[dt], 0, 0, 0);
      }
    }
    __builtin_amdgcn_s_waitcnt(0x0f70);  // the next tile landed
    __syncthreads();
    cur = nxt;
    keep = knext;
    buf ^= 1;
  }
}
#endif

// The short last tile of the sequence (keys >= nvalid masked); every wave
// loads its share, the waves whose query block keeps it compute it.
template <int BS, int D, int NWV>
__device__ __forceinline__ void tail_tile(const Ctx<BS, D>& x, const v4i (&qb)[Cfg<BS, D>::KS],
                                          const LaneOffs<BS, D>& lo, Acc<BS, D>& acc, int t,
                                          bool keep) {
  using C = Cfg<BS, D>;
  const int nvalid = x.L - t * KT;
  __syncthreads();
  dma_tile<BS, D, NWV>(x.kc_h + (size_t)t * KT * D, x.v_h + (size_t)t * KT * D, x.s_k, x.s_v,
                       x.wave, x.lane, nvalid);
  __builtin_amdgcn_s_waitcnt(0x0f70);
  __syncthreads();
  if (!keep) return;
  const float cs = x.c0 * load_uniform(x.sk_h, t / C::SUB);
  Ops<BS, D> op;
  load_ops<BS, D>(op, lo, x.s_k, x.s_v);
  v16i s[C::NT];
  qk<BS, D>(op.k, qb, s);
  softmax_pv<BS, D, true>(acc, s, op.v, qb, x.kc_h + (size_t)t * KT * D, x.lane, cs, nvalid);
}

// One workgroup per (batch*head, group of QB consecutive query blocks), with
// BS/32 waves per query block.  The group walks the union of its blocks' kept
// sets once, so a key tile kept by several of them is loaded once.
// Register budget: two waves per SIMD (256 VGPRs, all accumulators in
// architectural VGPRs, no AGPR round trips), except the kernels of 64-token
// blocks and D = 128, which take the walk with two tile buffers and three
// waves per SIMD (168 VGPRs) when QSA_ATTN_JIT is set: they wait on latency
// more than on any unit, and the third wave covers more of it.
template <int BS, int D, bool REFRESH>
struct JitWalk {
  static constexpr bool on = QSA_ATTN_JIT && BS == 64 && D == 128;
};

// WIN: each query block keeps the blocks of its own window of a.win_blocks
// blocks (the local and global passes of windowed attention); the group walks
// the union of its blocks' windows in ascending order without kept lists.
template <int BS, int D, int QB, bool REFRESH, bool WIN = false>
__global__ __launch_bounds__((QB * BS / 32 * 64))
__attribute__((amdgpu_waves_per_eu(JitWalk<BS, D, REFRESH>::on ? QSA_ATTN_JIT_WAVES : 2, 8))) void attn_kernel(
    AttnArgs a, int L, int nb, uint32_t n_work) {
  static_assert(!(WIN && REFRESH), "windowed kept sets in the sparse kernel only");
  using C = Cfg<BS, D>;
  constexpr int NWV = QB * C::WPB;  // waves in the workgroup
  constexpr int THREADS = 64 * NWV;
  constexpr int NBUF = JitWalk<BS, D, REFRESH>::on ? 2 : 1;
  __shared__ __attribute__((aligned(1024))) int8_t s_k[NBUF * C::K_BYTES];
  __shared__ __attribute__((aligned(1024))) uint16_t s_v[NBUF * C::V_BYTES / 2];
  __shared__ uint32_t s_bits[QB * kMaxWords];
  __shared__ float s_qmax[WIN ? NWV : 1];  // windowed mode with bf16 Q: per-wave amax
  // The tile list of the two-buffer walk and its length/tail words live in
  // the bitmap array past the words the bitmaps use (it is sized for the
  // largest block count), so the workgroup's LDS footprint, and with it the
  // occupancy, is the same with or without the list.
  constexpr bool kSeq = JitWalk<BS, D, REFRESH>::on && QB == 2;
  const int nw_used = QB * ((nb + 31) >> 5);
  int* s_seq_info = reinterpret_cast<int*>(&s_bits[nw_used]);
  uint16_t* s_seq = reinterpret_cast<uint16_t*>(&s_bits[nw_used + 2]);
  const int seq_cap = 2 * (QB * kMaxWords - nw_used - 2);

  const uint32_t ng = (uint32_t)((nb + QB - 1) / QB);
  const uint32_t work = xcd_contiguous(blockIdx.x, n_work);
  const uint32_t grp = work % ng;
  const uint64_t bh = work / ng;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, ql = lane & 31;
  const int qsub = wave / C::WPB;  // this wave's query block within the group
  const int nq = min(QB, nb - (int)grp * QB);
  const uint64_t row0 = bh * (uint64_t)nb;
  // the group's query blocks: positions grp*QB .. grp*QB+nq-1 of the
  // processing order (ascending unless an order is given)
  // (an order entry outside [0, nb) names no block: -1)
  auto block_at = [&](int b) -> int {
    const int pos = (int)grp * QB + b;
    if (!a.order) return pos;
    const int v = a.order[row0 + pos];
    return v >= 0 && v < nb ? v : -1;
  };
  int i = qsub < nq ? __builtin_amdgcn_readfirstlane(block_at(qsub)) : nb;
  if (i < 0) i = nb;

  const uint64_t head_off = bh * (uint64_t)L * D;

  // this wave's 32 query rows, as the B operand of S^T = K Q^T (same channel
  // order as the K operand: lane group g holds channels g*D/2 + 16c + 0..15)
  const int qrow = i * BS + 32 * (wave % C::WPB) + ql;
  const bool qvalid = qrow < L;
  v4i qb[C::KS];
  bool q_here = false;  // windowed mode: Q codes formed here from bf16 Q
  float sq_here = 0.0f;
  if constexpr (WIN) q_here = a.q_x != nullptr;
  if (q_here) {
    sq_here = quantize_q_rows<BS, D>(a, qb, head_off, qrow, qvalid && i < nb, L, lane, wave,
                                     s_qmax);
  } else {
#pragma unroll
    for (int c = 0; c < C::KS; ++c) {
      qb[c] = qvalid ? *reinterpret_cast<const v4i*>(a.q_codes + head_off + (size_t)qrow * D +
                                                     g * (D / 2) + 16 * c)
                     : v4i{0, 0, 0, 0};
    }
  }
  // the Q loads stay in flight while the kept sets are read (their waits
  // cover them: loads complete in order); in the windowed mode the first
  // tile's wait does
  LaneOffs<BS, D> lo;
  lo.init(lane);
  Ctx<BS, D> x;
  x.kc_h = a.k_codes + head_off;
  x.v_h = a.v + head_off;
  x.sk_h = a.k_scales + bh * (uint64_t)nb;
  x.s_k = s_k;
  x.s_v = s_v;
  x.L = L;
  x.wave = wave;
  x.lane = lane;
  x.c0 = i < nb ? a.sm_scale * (q_here ? sq_here : a.q_scales[bh * (uint64_t)nb + i]) * kLog2e
               : 0.0f;

  if constexpr (!WIN)
    build_kept_bits<QB, THREADS>(s_bits, a, row0, [&](int b) { return block_at(b); }, nq, nb,
                                 tid);
  const int n_tiles = (L + KT - 1) / KT;
  const int tail_t = (L % KT) ? n_tiles - 1 : -1;
  const int myb = i < nb ? qsub : -1;

  // One online-softmax state.  It first runs over the kept blocks: that is
  // the sparse attention.  The refresh step parks the sparse output and then
  // continues the same state over every other block: the full attention.
  Acc<BS, D> acc;
  acc.init();
  const size_t row_off = head_off + (size_t)qrow * D;
  float inv_k = 0.0f;
  if constexpr (WIN) {
    // tiles of the group's windows [t0, t1) and of this block's own [k0, k1)
    const int per = a.win_blocks;
    const int g0 = (int)grp * QB;
    const int w0 = (g0 / per) * per, w1 = min(nb, ((g0 + nq - 1) / per + 1) * per);
    const int m0 = myb >= 0 ? (i / per) * per : 0;
    const int m1 = myb >= 0 ? min(nb, m0 + per) : 0;
    const int t0 = w0 * C::SUB, t1 = min(n_tiles, w1 * C::SUB);
    const int k0 = m0 * C::SUB, k1 = min(n_tiles, m1 * C::SUB);
    int t = t0;
    auto next = [&](bool& keep) {
      if (t == tail_t) ++t;  // the short last tile is walked apart
      if (t >= t1) return -1;
      keep = t >= k0 && t < k1;
      return t++;
    };
#if QSA_ATTN_JIT
    if constexpr (JitWalk<BS, D, REFRESH>::on)
      walk_jit<BS, D, NWV>(x, qb, lo, acc, next);
    else
#endif
      walk<BS, D, NWV>(x, qb, lo, acc, next);
    if (tail_t >= t0 && tail_t < t1)
      tail_tile<BS, D, NWV>(x, qb, lo, acc, tail_t, tail_t >= k0 && tail_t < k1);
    const float lk = acc.l + __shfl_xor(acc.l, 32, 64);
    inv_k = lk > 0.0f ? 1.0f / lk : 0.0f;
  }
#pragma unroll 1
  for (int phase = 0; phase < (WIN ? 0 : REFRESH ? 2 : 1); ++phase) {
    BitWalk<QB, C::SUB> w;
    w.init(s_bits, nb, nq, myb, n_tiles, tail_t, phase == 1);
#if QSA_ATTN_JIT
    if constexpr (JitWalk<BS, D, REFRESH>::on) {
      // the phase's tiles from the list when they all fit (else the bitmap
      // walk); each entry is read one call ahead, so its LDS latency hides
      // behind a whole tile
      int seq_n = seq_cap + 1;
      if (kSeq && seq_cap > 0) {
        if (phase > 0) __syncthreads();  // every wave is done with the last list
        build_seq(s_bits, nb, nq, tail_t, phase == 1, s_seq, seq_cap, s_seq_info, tid);
        __syncthreads();
        seq_n = __builtin_amdgcn_readfirstlane(s_seq_info[0]);
      }
      const bool use_seq = seq_n <= seq_cap;
      int n = 0;
      uint32_t pre = use_seq && seq_n > 0 ? s_seq[0] : 0u;
      const int kshift = 14 + (myb >= 0 ? myb : 0);
      walk_jit<BS, D, NWV>(x, qb, lo, acc, [&](bool& keep) {
        if (!use_seq) return w.next(keep);
        if (n >= seq_n) return -1;
        const uint32_t e = __builtin_amdgcn_readfirstlane(pre);
        ++n;
        pre = s_seq[n < seq_n ? n : 0];
        keep = myb >= 0 && ((e >> kshift) & 1u);
        return (int)(e & 0x3fffu);
      });
      bool th = w.tail_hit, tk = w.tail_keep;
      if (use_seq) {
        const int tb = __builtin_amdgcn_readfirstlane(s_seq_info[1]);
        th = tb & 1;
        tk = myb >= 0 && ((tb >> (1 + myb)) & 1);
      }
      if (th) tail_tile<BS, D, NWV>(x, qb, lo, acc, tail_t, tk);
    } else
#endif
    {
      walk<BS, D, NWV>(x, qb, lo, acc, [&](bool& keep) { return w.next(keep); });
      if (w.tail_hit) tail_tile<BS, D, NWV>(x, qb, lo, acc, tail_t, w.tail_keep);
    }
    if (phase == 0) {
      const float lk = acc.l + __shfl_xor(acc.l, 32, 64);
      inv_k = lk > 0.0f ? 1.0f / lk : 0.0f;
    }
    if (REFRESH && phase == 0 && qvalid) {
      // Park the sparse output in fp32 in this row's own output slots (upper
      // halves in dr, lower halves in out, both written for good in the
      // epilogue), so the state can go on to the full attention.
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt) {
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int d0 = 32 * dt + 8 * r4 + 4 * g;
          uint32_t u[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) u[e] = __float_as_uint(acc.o[dt][4 * r4 + e] * inv_k);
          *reinterpret_cast<uint2*>(a.dr_out + row_off + d0) = make_uint2(
              (u[0] >> 16) | (u[1] & 0xffff0000u), (u[2] >> 16) | (u[3] & 0xffff0000u));
          *reinterpret_cast<uint2*>(a.out + row_off + d0) =
              make_uint2((u[0] & 0xffffu) | (u[1] << 16), (u[2] & 0xffffu) | (u[3] << 16));
        }
      }
    }
  }

  if (!REFRESH) {
    if (!qvalid) return;
    size_t orow_off = row_off;
    if (a.out_map) {
      const int w = a.out_w, m = L / a.out_w;
      const int orow = a.out_map == 1 ? (qrow % w) * m + qrow / w : (qrow % m) * w + qrow / m;
      orow_off = head_off + (size_t)orow * D;
    }
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d0 = 32 * dt + 8 * r4 + 4 * g;
        float os[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) os[e] = acc.o[dt][4 * r4 + e] * inv_k;
        if (a.r_in) {
          const float4 rv = load_bf16x4(a.r_in + orow_off + d0);
          os[0] += rv.x; os[1] += rv.y; os[2] += rv.z; os[3] += rv.w;
        }
        if (a.dr_in) {
          const float4 dv = load_bf16x4(a.dr_in + orow_off + d0);
          os[0] += dv.x; os[1] += dv.y; os[2] += dv.z; os[3] += dv.w;
        }
        store_bf16x4(a.out + orow_off + d0, os[0], os[1], os[2], os[3]);
      }
    }
    return;
  }

  const float lf = acc.l + __shfl_xor(acc.l, 32, 64);
  const float inv_f = lf > 0.0f ? 1.0f / lf : 0.0f;
  if (!qvalid) return;
  {
    // r = full - sparse from the two rounded fp32 outputs: no fused
    // multiply-subtract, so equal outputs (every block kept) give r = 0 exactly
#pragma clang fp contract(off)
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d0 = 32 * dt + 8 * r4 + 4 * g;
        const uint2 hi = *reinterpret_cast<const uint2*>(a.dr_out + row_off + d0);
        const uint2 lw = *reinterpret_cast<const uint2*>(a.out + row_off + d0);
        float os[4];
        os[0] = __uint_as_float((hi.x << 16) | (lw.x & 0xffffu));
        os[1] = __uint_as_float((hi.x & 0xffff0000u) | (lw.x >> 16));
        os[2] = __uint_as_float((hi.y << 16) | (lw.y & 0xffffu));
        os[3] = __uint_as_float((hi.y & 0xffff0000u) | (lw.y >> 16));
        float of[4], rho[4], drv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          of[e] = acc.o[dt][4 * r4 + e] * inv_f;
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

template <int BS, int D, int QB, bool REFRESH, bool WIN = false>
hipError_t launch_t(const qsa_dims& d, const AttnArgs& a, hipStream_t s) {
  const int nb = (d.seq_len + BS - 1) / BS;
  const uint32_t ng = (uint32_t)((nb + QB - 1) / QB);
  const uint32_t n_work = (uint32_t)((uint64_t)d.batch * d.heads * ng);
  hipLaunchKernelGGL((attn_kernel<BS, D, QB, REFRESH, WIN>), dim3(n_work),
                     dim3(QB * BS / 32 * 64), 0, s, a, d.seq_len, nb, n_work);
  return hipGetLastError();
}

// Query blocks per workgroup, the same for the sparse and the refresh kernel:
// a group's blocks share every key tile that more than one of them needs
// (kept tiles in the sparse walk; in the refresh, also the tiles outside
// their kept sets), and the waves of a group split each tile's loads evenly,
// which bounds the group size.  Two 64-token blocks for the 64-token kernels
// and for 128-token blocks with D = 128, one for 128-token blocks with D = 64.
template <bool REFRESH, bool WIN = false>
hipError_t dispatch(const qsa_dims& d, const AttnArgs& a, hipStream_t s) {
  constexpr int Q64 = QSA_ATTN_QB;
  constexpr int Q64s = QSA_ATTN_QB < 2 ? QSA_ATTN_QB : 2;
  if (d.block == 64 && d.head_dim == 128) return launch_t<64, 128, Q64, REFRESH, WIN>(d, a, s);
  if (d.block == 64 && d.head_dim == 64) return launch_t<64, 64, Q64s, REFRESH, WIN>(d, a, s);
  if (d.block == 128 && d.head_dim == 128)
    return launch_t<128, 128, Q64s, REFRESH, WIN>(d, a, s);
  return launch_t<128, 64, 1, REFRESH, WIN>(d, a, s);
}

}  // namespace

hipError_t launch_sparse_attn(const qsa_dims& d, const AttnArgs& a, hipStream_t s) {
  return dispatch<false>(d, a, s);
}

hipError_t launch_full_attn_residual(const qsa_dims& d, const AttnArgs& a, hipStream_t s) {
  return dispatch<true>(d, a, s);
}

hipError_t launch_sparse_attn_window(const qsa_dims& d, const AttnArgs& a, hipStream_t s) {
  if (a.win_blocks < 1 || a.order != nullptr) return hipErrorInvalidValue;
  return dispatch<false, true>(d, a, s);
}

}  // namespace qsa
