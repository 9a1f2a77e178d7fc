// Processing order of the query blocks for the block-sparse attention.
//
// Sparse attention gathers, for every query block, the K/V tiles of its kept
// key blocks (sparsified attention, QuantSparse gist.science/es/paper/
// 2509.23681, technical summary §1).  Query blocks whose kept sets overlap
// can share those loads: inside one workgroup (which walks the union of its
// blocks' kept sets) and in the L2 of one XCD (which runs neighbouring work
// items together).  How much two blocks' sets overlap depends on the data,
// not on how far apart the blocks are.  This kernel orders the query blocks
// of each (batch, head) so that neighbours in the order keep similar sets.
// The order changes no attention output (each block is computed from its
// own kept set), only the reuse.
//
// The blocks are cut into chunks of kChunk consecutive blocks, each ordered
// by one workgroup on its own.  The attention gives positions (2k, 2k+1) of
// the order to one workgroup, whose walk covers the union of the two kept
// sets, so the blocks are first paired: kept sets are compared through a
// 256-bit signature (key block j sets bit j mod 256); the workgroup fills a
// table of the signature overlaps of every two blocks of the chunk (a byte
// each, saturating), and rounds of mutual best partners -- each single block
// picks the single block of largest overlap, ties to the lower index; two
// blocks that pick each other pair up -- give the greedy maximum-overlap
// matching (blocks still single after the rounds pair in block order).  The
// pairs are then ordered by a greedy chain over the signatures of their
// unions, from the pair of the lowest block, always to the unused pair that
// shares the most bits with the current one (ties: the lower pair index,
// pairs indexed by their lower block), so that neighbouring workgroups, which
// run together on one XCD, keep similar sets too.  An odd chunk's single
// block goes last.
#include "qsa_internal.h"

namespace qsa {
namespace {

constexpr int kChunk = 256;        // blocks per chain
constexpr int kPer = kChunk / 64;  // candidates per lane
constexpr int kSigW = 8;           // 32-bit words per signature

constexpr int kBuildThreads = 256;
constexpr int kOvLd = kChunk + 16;  // overlap table row (bytes), padded

// Maximum over the 64 lanes of a wave with DPP moves (row-local butterflies,
// then the row broadcasts of lane 15 and lane 31); every lane gets the result.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));  // row_half_mirror
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));  // row_mirror
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false));  // row_bcast:15
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false));  // row_bcast:31
  return __builtin_amdgcn_readlane(v, 63);
}

// The greedy chain over m <= 64 * PER items (blocks or pairs) with 256-bit
// signatures sig[w][c] (row stride STRIDE), run by one wave: chain[step] =
// the item at that step.  Lane l holds the signatures of items l, l+64, ...
// in registers, so a step is a few register reads, ANDs and bit counts, and
// a wave-wide argmax, with no barrier.
template <int PER, int STRIDE>
__device__ __forceinline__ void run_chain(const uint32_t* sigs, int m, int lane,
                                          int16_t* chain) {
  uint32_t sig[PER][kSigW];
  bool live[PER];
#pragma unroll
  for (int t = 0; t < PER; ++t) {
    const int c = lane + 64 * t;
    live[t] = c < m;
#pragma unroll
    for (int w = 0; w < kSigW; ++w) sig[t][w] = live[t] ? sigs[w * STRIDE + c] : 0u;
  }
  int cur = 0;
  live[0] = lane != 0 && live[0];
  if (lane == 0) chain[0] = 0;
  for (int step = 1; step < m; ++step) {
    // the current item's signature, from the lane that holds it
    const int ol = cur & 63, ot = cur >> 6;
    uint32_t cs[kSigW];
#pragma unroll
    for (int w = 0; w < kSigW; ++w) {
      uint32_t v = 0u;
#pragma unroll
      for (int t = 0; t < PER; ++t)
        if (t == ot) v = sig[t][w];
      cs[w] = __builtin_amdgcn_readlane(v, ol);
    }
    // best live candidate: the largest key (score + 1) << 8 | (255 - index)
    // (highest score, then lowest index); a lane with none left keys 0
    uint32_t key = 0u;
#pragma unroll
    for (int t = 0; t < PER; ++t) {
      uint32_t sc = 0u;
#pragma unroll
      for (int w = 0; w < kSigW; ++w) sc += __popc(cs[w] & sig[t][w]);
      const uint32_t kt = ((sc + 1u) << 8) | (uint32_t)(255 - (lane + 64 * t));
      if (live[t]) key = max(key, kt);
    }
    cur = 255 - (int)(wave_max_u32(key) & 255u);
#pragma unroll
    for (int t = 0; t < PER; ++t)
      if (cur == lane + 64 * t) live[t] = false;
    if (lane == 0) chain[step] = (int16_t)cur;
  }
}

// Pair the chunk's blocks by rounds of mutual best partners (see the
// header): s_partner[b] = the block paired with b, -1 for the single block
// of an odd chunk.  Thread t stands for block t.  The set of single blocks
// only shrinks, so a block's best candidate stays its best while that
// candidate is single: a block rescans only when its pick has been paired.
__device__ __forceinline__ void match(const uint8_t* s_ov, int16_t* s_best, int16_t* s_partner,
                                      uint32_t* s_alive, int n, int tid) {
  constexpr int kMaxRounds = 48;
  constexpr int kWords = kChunk / 32;
  const int lane = tid & 63, wave = tid >> 6;
  // this block's overlaps with every block, kept in registers for the rounds
  uint32_t row[kChunk / 4];
#pragma unroll
  for (int q = 0; q < kChunk / 16; ++q) {
    const uint4 v = tid < n ? *reinterpret_cast<const uint4*>(s_ov + tid * kOvLd + 16 * q)
                            : make_uint4(0u, 0u, 0u, 0u);
    row[4 * q] = v.x;
    row[4 * q + 1] = v.y;
    row[4 * q + 2] = v.z;
    row[4 * q + 3] = v.w;
  }
  bool single = tid < n;
  int best = -1;
  for (int round = 0; round < kMaxRounds; ++round) {
    // single blocks as a bit mask, one ballot per wave
    const uint64_t m = __ballot(single);
    if (lane == 0) {
      s_alive[2 * wave] = (uint32_t)m;
      s_alive[2 * wave + 1] = (uint32_t)(m >> 32);
    }
    __syncthreads();
    const bool stale = best < 0 || !((s_alive[best >> 5] >> (best & 31)) & 1u);
    if (single && stale) {
      // best single partner: the largest key (overlap + 1) << 8 | (255 - u)
      uint32_t key = 0u;
#pragma unroll
      for (int w = 0; w < kWords; ++w) {
        uint32_t am = s_alive[w];
        if (tid >> 5 == w) am &= ~(1u << (tid & 31));
#pragma unroll
        for (int b = 0; b < 32; ++b) {
          const int u = 32 * w + b;
          const uint32_t ov = (row[u >> 2] >> (8 * (u & 3))) & 0xffu;
          const uint32_t k = ((ov + 1u) << 8) | (uint32_t)(255 - u);
          key = ((am >> b) & 1u) ? max(key, k) : key;
        }
      }
      best = key ? 255 - (int)(key & 255u) : -1;
    }
    if (tid < n) s_best[tid] = single ? (int16_t)best : (int16_t)-1;
    __syncthreads();
    // t pairs with u > t when they picked each other; only t writes either
    bool paired = false;
    if (single) {
      const int u = best;
      if (u > tid && s_best[u] == tid) {
        s_partner[tid] = (int16_t)u;
        s_partner[u] = (int16_t)tid;
        paired = true;
      }
    }
    const int made = __syncthreads_or(paired);
    if (single) single = s_partner[tid] < 0;
    if (!made) break;  // fewer than two blocks left single
  }
  // blocks still single pair in block order (more than one only if the
  // rounds ran out), by one thread
  if (__syncthreads_count(single) > 1) {
    if (tid == 0) {
      int pending = -1;
      for (int b = 0; b < n; ++b) {
        if (s_partner[b] >= 0) continue;
        if (pending < 0) {
          pending = b;
        } else {
          s_partner[pending] = (int16_t)b;
          s_partner[b] = (int16_t)pending;
          pending = -1;
        }
      }
    }
    __syncthreads();
  }
}

__global__ __launch_bounds__(kBuildThreads) void order_kernel(const int32_t* __restrict__ kept_idx,
                                                              const int32_t* __restrict__ kept_cnt,
                                                              int kmax, int nb, int n_chunks,
                                                              int vec16,
                                                              int32_t* __restrict__ order) {
  __shared__ uint32_t s_sig[kSigW][kChunk];
  __shared__ int s_cnt[kChunk];
  __shared__ __attribute__((aligned(16))) uint8_t s_ov[kChunk * kOvLd];
  __shared__ int16_t s_best[kChunk], s_partner[kChunk];
  __shared__ int16_t s_pb[kChunk / 2], s_pu[kChunk / 2], s_pchain[kChunk / 2];
  __shared__ uint32_t s_psig[kSigW * (kChunk / 2)];
  __shared__ uint32_t s_alive[kChunk / 32];
  __shared__ int s_wcnt[kBuildThreads / 64];
  const uint64_t bh = blockIdx.x / (uint32_t)n_chunks;
  const int c0 = (int)(blockIdx.x % (uint32_t)n_chunks) * kChunk;
  const int n = min(kChunk, nb - c0);  // blocks in this chunk
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int32_t* kl = kept_idx + (bh * (uint64_t)nb + c0) * (uint64_t)kmax;
  const int32_t* kc = kept_cnt + bh * (uint64_t)nb + c0;
  int32_t* out = order + bh * (uint64_t)nb + c0;
  // signatures, built by the whole workgroup: entry k of the chunk's rows is
  // (block k / kmax, position k % kmax); the loads are independent
  for (int k = tid; k < kSigW * kChunk; k += kBuildThreads) (&s_sig[0][0])[k] = 0u;
  for (int i = tid; i < n; i += kBuildThreads) {
    s_cnt[i] = min(max(kc[i], 0), kmax);
    s_partner[i] = -1;
  }
  __syncthreads();
  // the chunk's kept lists are one run of n * kmax ints; with a 16-byte
  // aligned array the pieces wholly inside the run are read as int4, eight in
  // flight per thread, and the up to three elements at each end one by one
  {
    const uint64_t first = (bh * (uint64_t)nb + c0) * (uint64_t)kmax;  // element index
    const int total = n * kmax;
    const float inv_kmax = 1.0f / (float)kmax;
    auto add = [&](int k, int j) {  // element k of the run holds key block j
      if (j < 0 || j >= nb) return;
      int i = (int)((float)k * inv_kmax);  // row k / kmax, corrected below
      i -= i * kmax > k;
      i += (i + 1) * kmax <= k;
      if (k - i * kmax < s_cnt[i]) {
        const int b = j & (32 * kSigW - 1);
        atomicOr(&s_sig[b >> 5][i], 1u << (b & 31));
      }
    };
    const uint64_t qa = (first + 3) >> 2, qb = (first + total) >> 2;  // whole pieces
    if (vec16 && qb > qa) {
      const int nq = (int)(qb - qa), head = (int)(4 * qa - first);
      const int4* base = reinterpret_cast<const int4*>(kept_idx) + qa;
      for (int q = tid; q < nq; q += 8 * kBuildThreads) {
        int4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int qq = q + u * kBuildThreads;
          v[u] = qq < nq ? base[qq] : make_int4(-1, -1, -1, -1);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int k0 = head + 4 * (q + u * kBuildThreads);
          add(k0, v[u].x);
          add(k0 + 1, v[u].y);
          add(k0 + 2, v[u].z);
          add(k0 + 3, v[u].w);
        }
      }
      const int tail0 = head + 4 * nq;  // elements [0, head) and [tail0, total)
      if (tid < head) add(tid, kl[tid]);
      if (tid < total - tail0) add(tail0 + tid, kl[tail0 + tid]);
    } else {
#pragma unroll 4
      for (int k = tid; k < total; k += kBuildThreads) add(k, kl[k]);
    }
  }
  __syncthreads();
  if (n <= 2) {  // nothing to choose
    if (tid < n) out[tid] = c0 + tid;
    return;
  }
  // signature overlaps of every two blocks (a byte each, saturating)
  if (tid < n) {
    uint32_t sr[kSigW];
#pragma unroll
    for (int w = 0; w < kSigW; ++w) sr[w] = s_sig[w][tid];
    for (int u = 0; u < n; ++u) {
      uint32_t c = 0u;
#pragma unroll
      for (int w = 0; w < kSigW; ++w) c += __popc(sr[w] & s_sig[w][u]);
      s_ov[tid * kOvLd + u] = (uint8_t)min(c, 255u);
    }
  }
  __syncthreads();
  match(s_ov, s_best, s_partner, s_alive, n, tid);
  // the pairs, indexed by their lower block in block order, with the
  // signature of their union; the single block (odd chunks) goes last
  const int u = tid < n ? s_partner[tid] : -1;
  const bool lead = tid < n && u > tid;
  const uint64_t lm = __ballot(lead);
  if (lane == 0) s_wcnt[wave] = __popcll(lm);
  if (tid < n && u < 0) out[n - 1] = c0 + tid;
  __syncthreads();
  const int npairs = n >> 1;
  if (lead) {
    int k = __popcll(lm & ((1ull << lane) - 1ull));
    for (int w = 0; w < wave; ++w) k += s_wcnt[w];
    s_pb[k] = (int16_t)tid;
    s_pu[k] = (int16_t)u;
#pragma unroll
    for (int w = 0; w < kSigW; ++w) s_psig[w * (kChunk / 2) + k] = s_sig[w][tid] | s_sig[w][u];
  }
  __syncthreads();
  // the pairs in a greedy chain of their union signatures, so neighbouring
  // workgroups share tiles too
  if (tid < 64) run_chain<kPer / 2, kChunk / 2>(s_psig, npairs, lane, s_pchain);
  __syncthreads();
  if (tid < npairs) {
    const int k = s_pchain[tid];
    out[2 * tid] = c0 + s_pb[k];
    out[2 * tid + 1] = c0 + s_pu[k];
  }
}

}  // namespace

hipError_t launch_order(const qsa_dims& d, const int32_t* kept_idx, const int32_t* kept_cnt,
                        int32_t kmax, int32_t* order, hipStream_t s) {
  const int nb = (d.seq_len + d.block - 1) / d.block;
  const int n_chunks = (nb + kChunk - 1) / kChunk;
  const uint64_t grid = (uint64_t)d.batch * d.heads * n_chunks;
  const int vec16 = ((uintptr_t)kept_idx & 15u) == 0;
  hipLaunchKernelGGL(order_kernel, dim3((uint32_t)grid), dim3(kBuildThreads), 0, s, kept_idx, kept_cnt,
                     kmax, nb, n_chunks, vec16, order);
  return hipGetLastError();
}

}  // namespace qsa
