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
// by one wave on its own: a greedy chain from the chunk's first block that
// always continues with the unused block of the chunk whose kept set shares
// the most bits with the current one (ties: lowest index).  Kept sets are
// compared through a 256-bit signature (key block j sets bit j mod 256).
// The workgroup builds the signatures in LDS; then one wave runs the chain:
// lane l holds the signatures of the chunk's blocks l, l+64, l+128, l+192 in
// registers, so a step is a few register reads, ANDs and bit counts, and a
// wave-wide argmax, with no barrier.
#include "qsa_internal.h"

namespace qsa {
namespace {

constexpr int kChunk = 256;        // blocks per chain
constexpr int kPer = kChunk / 64;  // candidates per lane
constexpr int kSigW = 8;           // 32-bit words per signature

constexpr int kBuildThreads = 256;

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

__global__ __launch_bounds__(kBuildThreads) void order_kernel(const int32_t* __restrict__ kept_idx,
                                                              const int32_t* __restrict__ kept_cnt,
                                                              int kmax, int nb, int n_chunks,
                                                              int32_t* __restrict__ order) {
  __shared__ uint32_t s_sig[kSigW][kChunk];
  __shared__ int s_cnt[kChunk];
  const uint64_t bh = blockIdx.x / (uint32_t)n_chunks;
  const int c0 = (int)(blockIdx.x % (uint32_t)n_chunks) * kChunk;
  const int n = min(kChunk, nb - c0);  // blocks in this chunk
  const int tid = threadIdx.x, lane = tid & 63;
  const int32_t* kl = kept_idx + (bh * (uint64_t)nb + c0) * (uint64_t)kmax;
  const int32_t* kc = kept_cnt + bh * (uint64_t)nb + c0;
  int32_t* out = order + bh * (uint64_t)nb + c0;

  // signatures, built by the whole workgroup: entry k of the chunk's rows is
  // (block k / kmax, position k % kmax); the loads are independent
  for (int k = tid; k < kSigW * kChunk; k += kBuildThreads) (&s_sig[0][0])[k] = 0u;
  for (int i = tid; i < n; i += kBuildThreads) s_cnt[i] = min(max(kc[i], 0), kmax);
  __syncthreads();
  const int total = n * kmax;
#pragma unroll 4
  for (int k = tid; k < total; k += kBuildThreads) {
    const int j = kl[k];
    const int i = k / kmax;
    if (k - i * kmax < s_cnt[i] && j >= 0 && j < nb) {
      const int b = j & (32 * kSigW - 1);
      atomicOr(&s_sig[b >> 5][i], 1u << (b & 31));
    }
  }
  __syncthreads();
  if (tid >= 64) return;  // one wave runs the chain

  // this lane's candidates (chunk-local index lane + 64 t) and their signatures
  uint32_t sig[kPer][kSigW];
  bool live[kPer];
#pragma unroll
  for (int t = 0; t < kPer; ++t) {
    const int c = lane + 64 * t;
    live[t] = c < n;
#pragma unroll
    for (int w = 0; w < kSigW; ++w) sig[t][w] = live[t] ? s_sig[w][c] : 0u;
  }
  int cur = 0;  // chunk-local
  live[0] = lane != 0 && live[0];
  if (lane == 0) out[0] = c0;
  for (int step = 1; step < n; ++step) {
    // the current block's signature, from the lane that holds it
    const int ol = cur & 63, ot = cur >> 6;
    uint32_t cs[kSigW];
#pragma unroll
    for (int w = 0; w < kSigW; ++w) {
      uint32_t v = 0u;
#pragma unroll
      for (int t = 0; t < kPer; ++t)
        if (t == ot) v = sig[t][w];
      cs[w] = __builtin_amdgcn_readlane(v, ol);
    }
    // best live candidate: the largest key (score + 1) << 8 | (255 - index)
    // (highest score, then lowest index); a lane with none left keys 0
    uint32_t key = 0u;
#pragma unroll
    for (int t = 0; t < kPer; ++t) {
      uint32_t sc = 0u;
#pragma unroll
      for (int w = 0; w < kSigW; ++w) sc += __popc(cs[w] & sig[t][w]);
      const uint32_t kt = ((sc + 1u) << 8) | (uint32_t)(255 - (lane + 64 * t));
      if (live[t]) key = max(key, kt);
    }
    const int bidx = 255 - (int)(wave_max_u32(key) & 255u);
    cur = bidx;
#pragma unroll
    for (int t = 0; t < kPer; ++t)
      if (cur == lane + 64 * t) live[t] = false;
    if (lane == 0) out[step] = c0 + cur;
  }
}

}  // namespace

hipError_t launch_order(const qsa_dims& d, const int32_t* kept_idx, const int32_t* kept_cnt,
                        int32_t kmax, int32_t* order, hipStream_t s) {
  const int nb = (d.seq_len + d.block - 1) / d.block;
  const int n_chunks = (nb + kChunk - 1) / kChunk;
  const uint64_t grid = (uint64_t)d.batch * d.heads * n_chunks;
  hipLaunchKernelGGL(order_kernel, dim3((uint32_t)grid), dim3(kBuildThreads), 0, s, kept_idx, kept_cnt,
                     kmax, nb, n_chunks, order);
  return hipGetLastError();
}

}  // namespace qsa
