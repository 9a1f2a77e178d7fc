// Rank-r projection of the second-order residual onto its dominant principal
// components.
//
// QuantSparse (gist.science/es/paper/2509.23681, technical summary §2B;
// gist.science/ko/paper/2509.23681, §2.2): the second-order residual is
// projected by an SVD onto its dominant, temporally stable components, with
// no storage beyond the residual cache.  For every (batch, head) slice
// X [L, D] of the bf16 residual the result is X V_r V_r^T, V_r the r
// eigenvectors of largest eigenvalue of the Gram matrix G = X^T X (the right
// singular vectors of X of largest singular value), written back in place.
//
// Three kernels:
//  1. gram_kernel: partial Gram matrices over token chunks with the bf16
//     MFMA (v_mfma_f32_32x32x16_bf16; bf16 products are exact in fp32, sums
//     in fp32).  The X tile sits row-major in LDS; the transposing LDS read
//     ds_read_b64_tr_b16 yields, per lane, 8 tokens of one channel -- the
//     A operand for a 32-channel row tile of G and, unchanged, the B operand
//     for a 32-channel column tile (both use the same token order).
//  2. jacobi_kernel: one 1024-thread workgroup per slice sums the partials
//     in a fixed order (deterministic), then diagonalises G by the cyclic
//     Jacobi method (Golub and Van Loan, Matrix Computations, §8.5:
//     symmetric Schur rotations; parallel round-robin ordering, D/2 disjoint
//     rotations per round, D-1 rounds per sweep) in fp32 with the upper
//     triangle of G and the eigenvector matrix in LDS.  A round computes its
//     D/2 rotations, then updates A one 2x2 block (rows of one pair x columns
//     of another) at a time -- the row and the column rotation of a block in
//     one step, since the block's new values depend on its own old ones only;
//     A stays symmetric, so of two mirrored blocks only one is rotated -- and
//     V by columns: two barriers per round.  Each thread issues all LDS reads
//     of its items before any write, so LDS latency overlaps across items.
//     Eigenvalues are ranked descending (ties: lower index).
//  3. project_kernel: 32 token rows per wave on the bf16 MFMA: C^T = V_r^T X^T,
//     then X V_r V_r^T = V_r C^T, with three-term bf16 splits of the basis and
//     of the coefficients (fp32-level error), rounded to bf16 in place.
#include "qsa_internal.h"

namespace qsa {
namespace {

constexpr int kThreads = 256;
constexpr int kJacobiThreads = 1024;
constexpr int kMaxSweeps = 16;

// ---------------------------------------------------------------------------
// 1. partial Gram matrices
// ---------------------------------------------------------------------------

// Chunk swizzle of the row-major bf16 X tile (16-byte chunks): the transposing
// read touches 4 consecutive rows x 4 consecutive chunks per 32 lanes; XOR-ing
// the chunk quad with the row spreads them over distinct banks.
template <int D>
__device__ __forceinline__ int xswz(int r) {
  return D == 128 ? ((r & 3) << 2) : (((r >> 1) & 1) << 2);
}

template <int D>
__global__ __launch_bounds__(kThreads) void gram_kernel(const uint16_t* __restrict__ x,
                                                        float* __restrict__ partial, int L,
                                                        int chunk) {
  constexpr int DT = D / 32;          // 32-channel tiles
  constexpr int CPR = D / 8;          // 16-byte chunks per row
  constexpr int ROWS = 64;            // tokens per LDS tile
  constexpr int NLD = ROWS * CPR / kThreads;
  constexpr int TPW = DT * DT / 4;    // output tiles per wave
  static_assert(NLD >= 1 && TPW >= 1, "tile shape");
  __shared__ __attribute__((aligned(16))) uint16_t s_x[ROWS * D];

  const int s = blockIdx.x, S = gridDim.x;
  const uint64_t bh = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t_begin = s * chunk, t_end = min(L, t_begin + chunk);
  const uint16_t* xb = x + bh * (uint64_t)L * D;

  // output tiles of this wave: row tile ti, column tiles tj0 + u (D = 128:
  // one row of 4 tiles; D = 64: one tile)
  const int ti = (wave * TPW) / DT, tj0 = (wave * TPW) % DT;
  v16f acc[TPW];
#pragma unroll
  for (int u = 0; u < TPW; ++u)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[u][r] = 0.0f;

  // per-lane byte offsets of the transposing reads (see the operand layout
  // above): 16-lane group G, lane j in it; out lane l then holds tokens
  // {4g + e, 8 + 4g + e : e < 4} (g = l / 32) of channel 32 dt + l % 32
  const int G = lane >> 4, j = lane & 15;
  const int r0 = 4 * (G >> 1) + (j >> 2);
  auto lane_off = [&](int dt) {
    const int c = 4 * dt + 2 * (G & 1) + ((j & 3) >> 1);
    return r0 * (2 * D) + ((c ^ xswz<D>(r0)) << 4) + 8 * (j & 1);
  };
  const int off_a = lane_off(ti);
  int off_b[TPW];
#pragma unroll
  for (int u = 0; u < TPW; ++u) off_b[u] = lane_off(tj0 + u);
  auto operand = [&](int st, int off) {
    const char* base = reinterpret_cast<const char*>(s_x) + 16 * st * (2 * D) + off;
    const v4s lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_t*)(base));
    const v4s hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_t*)(base + 8 * (2 * D)));
    const uint2 ul = __builtin_bit_cast(uint2, lo4), uh = __builtin_bit_cast(uint2, hi4);
    return __builtin_bit_cast(v8bf, make_uint4(ul.x, ul.y, uh.x, uh.y));
  };

  uint4 nxt[NLD];
  auto load = [&](int t0) {
#pragma unroll
    for (int n = 0; n < NLD; ++n) {
      const int q = tid + kThreads * n;
      const int row = q / CPR, c = q % CPR;
      const int t = t0 + row;
      nxt[n] = t < t_end ? *reinterpret_cast<const uint4*>(xb + (size_t)t * D + c * 8)
                         : make_uint4(0, 0, 0, 0);
    }
  };
  auto store = [&]() {
#pragma unroll
    for (int n = 0; n < NLD; ++n) {
      const int q = tid + kThreads * n;
      const int row = q / CPR, c = q % CPR;
      *reinterpret_cast<uint4*>(reinterpret_cast<char*>(s_x) + row * (2 * D) +
                                ((c ^ xswz<D>(row)) << 4)) = nxt[n];
    }
  };

  if (t_begin < t_end) load(t_begin);
  for (int t0 = t_begin; t0 < t_end; t0 += ROWS) {
    __syncthreads();  // the previous tile's reads are done
    store();
    __syncthreads();
    if (t0 + ROWS < t_end) load(t0 + ROWS);  // in flight during the MFMAs
#pragma unroll
    for (int st = 0; st < ROWS / 16; ++st) {
      const v8bf a_op = operand(st, off_a);
#pragma unroll
      for (int u = 0; u < TPW; ++u)
        acc[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_op, operand(st, off_b[u]), acc[u],
                                                         0, 0, 0);
    }
  }

  // accumulator element r of lane l is G[32 ti + 8 (r/4) + 4 (l/32) + r%4][32 tj + l%32]
  float* pb = partial + (bh * (uint64_t)S + s) * (uint64_t)(D * D);
#pragma unroll
  for (int u = 0; u < TPW; ++u)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = 32 * ti + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      const int n = 32 * (tj0 + u) + (lane & 31);
      pb[m * D + n] = acc[u][r];
    }
}

// ---------------------------------------------------------------------------
// 2. cyclic Jacobi eigensolver, one workgroup per slice
// ---------------------------------------------------------------------------

// One rotation of a round: rows/columns p < q, J = [[c, s], [-s, c]].
struct Rot {
  float c, s;
  int p, q;
};

template <int D>
__global__ __launch_bounds__(kJacobiThreads) void jacobi_kernel(
    const float* __restrict__ partial, int S, int rank, int rp, float* __restrict__ eigvals,
    float* __restrict__ basis, float* __restrict__ wbasis) {
  constexpr int T = kJacobiThreads;
  constexpr int LD = D + 1;        // padded rows: column walks hit distinct banks
  constexpr int NP = D / 2;        // disjoint rotations per round
  constexpr int IT = NP * D / T;   // (pair, row-or-column) items per thread
  constexpr int KS = T / D;        // pair stride between a thread's items
  // 2x2 blocks of A per round, one of each mirrored pair: block (P, (P + d)
  // mod NP) for d = 0 .. NP/2 - 1 and every P (index P * NP/2 + d), then for
  // d = NP/2 the P < NP/2.  The NP/2 lanes that share a P read one row pair
  // against distinct columns: a[i][j] and a[j][i] fall in one LDS bank (the
  // row stride is 1 modulo the bank count), so those reads hit distinct banks
  // whichever of the two places an entry has.
  constexpr int NBLK = NP * (NP / 2) + NP / 2;
  constexpr int BI = (NBLK + T - 1) / T;  // blocks per thread (the last round partial)
  static_assert(IT * T == NP * D && KS * D == T, "item split");
  __shared__ float a[D * LD];
  __shared__ float v[D * LD];
  __shared__ Rot rot[2][NP];  // this round's rotations and the next round's
  __shared__ float red[T / 64];
  __shared__ int done;

  const uint64_t bh = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  // G = sum of the partials in chunk order (A holds the upper triangle; the
  // lower one is written here but not used)
  const float* pb = partial + bh * (uint64_t)S * (D * D);
  float fro = 0.0f;
  for (int e = tid; e < D * D; e += T) {
    const int i = e / D, k = e % D;
    if (k < i) continue;
    float g = 0.0f;
    for (int s = 0; s < S; ++s) g += pb[(size_t)s * (D * D) + e];
    a[i * LD + k] = g;
    a[k * LD + i] = g;
    fro += (i == k ? 1.0f : 2.0f) * g * g;
    v[i * LD + k] = i == k ? 1.0f : 0.0f;
    v[k * LD + i] = i == k ? 1.0f : 0.0f;
  }
  for (int o = 32; o >= 1; o >>= 1) fro += __shfl_xor(fro, o, 64);
  if (lane == 0) red[wave] = fro;
  __syncthreads();
  float tot = 0.0f;
#pragma unroll
  for (int w = 0; w < T / 64; ++w) tot += red[w];
  // rotations stop once every off-diagonal entry is below 2^-22 ||G||_F, a
  // few fp32 roundings of the largest entries
  const float tol = sqrtf(tot) * 0x1p-22f;

  // this thread's items: pair k = k0 + KS n, row or column index = idx
  const int k0 = tid / D, idx = tid % D;

  // Rotation tid (< NP) of round t from the current A, into dst; returns
  // |a_pq| before the rotation.
  auto make_rot = [&](int t, Rot* dst) {
    int p, q;
    if (tid == 0) {
      p = t;
      q = D - 1;
    } else {
      const int u = (t + tid) % (D - 1), w = (t - tid + (D - 1)) % (D - 1);
      p = min(u, w);
      q = max(u, w);
    }
    const float apq = a[p * LD + q];
    float c = 1.0f, sn = 0.0f;
    if (fabsf(apq) > tol) {
      // symmetric Schur rotation: J = [[c, s], [-s, c]] zeroes a_pq
      const float tau = (a[q * LD + q] - a[p * LD + p]) / (2.0f * apq);
      const float tt = (tau >= 0.0f ? 1.0f : -1.0f) /
                       (fabsf(tau) + sqrtf(__builtin_fmaf(tau, tau, 1.0f)));
      c = 1.0f / sqrtf(__builtin_fmaf(tt, tt, 1.0f));
      sn = tt * c;
    }
    dst[tid] = Rot{c, sn, p, q};
    return fabsf(apq);
  };

  // A round's rotations depend on A only, so the next round's are computed
  // (by the first wave) while this round's V update runs, between the A
  // update and the round's last barrier.
  int cur = 0;
  float big_next = 0.0f;  // |a_pq| of round 0 of the next sweep (threads < NP)
  if (tid < NP) big_next = make_rot(0, rot[0]);
  __syncthreads();
  for (int sweep = 0; sweep < kMaxSweeps; ++sweep) {
    float big = big_next;  // largest |a_pq| met in this sweep (threads < NP)
    for (int t = 0; t < D - 1; ++t) {
      const Rot* rt = rot[cur];
      // A <- J^T A J one 2x2 block at a time: block (P, Q) holds rows p, q of
      // pair P and columns r, s of pair Q, and its new values depend on its
      // four old ones only (the round's pairs are disjoint), so the row and
      // the column rotation of a block are one step with no barrier between.
      // Block (Q, P) is its transpose: only one of the two is rotated, its
      // entries read and written at their upper-triangle places.  The rotated
      // pair's off-diagonal entry is set to 0.
      {
        float b4[BI][4];
        Rot rp[BI], rq[BI];
        int e4[BI][4];  // LDS places of the block's entries
#pragma unroll
        for (int n = 0; n < BI; ++n) {
          const int blk = min(tid + T * n, NBLK - 1);
          const int P = blk < NP * (NP / 2) ? blk / (NP / 2) : blk - NP * (NP / 2);
          const int Q = (P + (blk < NP * (NP / 2) ? blk % (NP / 2) : NP / 2)) % NP;
          rp[n] = rt[P];
          rq[n] = rt[Q];
          const int r0 = rp[n].p, r1 = rp[n].q, c0 = rq[n].p, c1 = rq[n].q;
          e4[n][0] = min(r0, c0) * LD + max(r0, c0);
          e4[n][1] = min(r0, c1) * LD + max(r0, c1);
          e4[n][2] = min(r1, c0) * LD + max(r1, c0);
          e4[n][3] = min(r1, c1) * LD + max(r1, c1);
#pragma unroll
          for (int e = 0; e < 4; ++e) b4[n][e] = a[e4[n][e]];
        }
#pragma unroll
        for (int n = 0; n < BI; ++n) {
          if (tid + T * n >= NBLK) continue;
          if (rp[n].s == 0.0f && rq[n].s == 0.0f) continue;
          const float cp = rp[n].c, sp = rp[n].s, cq = rq[n].c, sq = rq[n].s;
          // rows: J_P^T
          const float xpr = cp * b4[n][0] - sp * b4[n][2], xps = cp * b4[n][1] - sp * b4[n][3];
          const float xqr = sp * b4[n][0] + cp * b4[n][2], xqs = sp * b4[n][1] + cp * b4[n][3];
          // columns: J_Q
          float ypr = cq * xpr - sq * xps, yps = sq * xpr + cq * xps;
          float yqr = cq * xqr - sq * xqs, yqs = sq * xqr + cq * xqs;
          if (rp[n].p == rq[n].p) {  // diagonal block: a_pq = 0 (one place)
            a[e4[n][0]] = ypr;
            a[e4[n][1]] = 0.0f;
            a[e4[n][3]] = yqs;
            continue;
          }
          a[e4[n][0]] = ypr;
          a[e4[n][1]] = yps;
          a[e4[n][2]] = yqr;
          a[e4[n][3]] = yqs;
        }
      }
      __syncthreads();  // A is updated
      // the next round's rotations: round t + 1, or round 0 of the next sweep
      if (tid < NP) {
        const float m = make_rot(t + 1 < D - 1 ? t + 1 : 0, rot[cur ^ 1]);
        if (t + 1 < D - 1)
          big = fmaxf(big, m);
        else
          big_next = m;
      }
      // V <- V J
      {
        Rot r[IT];
        float vp[IT], vq[IT];
#pragma unroll
        for (int n = 0; n < IT; ++n) {
          r[n] = rt[k0 + KS * n];
          vp[n] = v[idx * LD + r[n].p];
          vq[n] = v[idx * LD + r[n].q];
        }
#pragma unroll
        for (int n = 0; n < IT; ++n) {
          if (r[n].s == 0.0f) continue;
          v[idx * LD + r[n].p] = r[n].c * vp[n] - r[n].s * vq[n];
          v[idx * LD + r[n].q] = r[n].s * vp[n] + r[n].c * vq[n];
        }
      }
      __syncthreads();
      cur ^= 1;
    }
    if (wave == 0) {
      for (int o = 32; o >= 1; o >>= 1) big = fmaxf(big, __shfl_xor(big, o, 64));
      if (lane == 0) done = big <= tol;
    }
    __syncthreads();
    const bool stop = done;
    __syncthreads();  // every thread has read the flag before wave 0 rewrites it
    if (stop) break;
  }

  // rank eigenvalues descending, ties to the lower index; write the top ones
  for (int i = tid; i < D; i += T) {
    const float di = a[i * LD + i];
    int rk = 0;
    for (int k = 0; k < D; ++k) {
      const float dk = a[k * LD + k];
      rk += (dk > di) || (dk == di && k < i);
    }
    float* wb = wbasis + bh * (uint64_t)(D * rp);
    if (rk < rank) {
      eigvals[bh * (uint64_t)rank + rk] = di;
      float* ub = basis + bh * (uint64_t)(D * rank);
      for (int d = 0; d < D; ++d) {
        ub[d * rank + rk] = v[d * LD + i];
        wb[d * rp + rk] = v[d * LD + i];
      }
    } else if (rk < rp) {
      for (int d = 0; d < D; ++d) wb[d * rp + rk] = 0.0f;
    }
  }
}

// ---------------------------------------------------------------------------
// 3. projection of every row onto the kept directions, in place
// ---------------------------------------------------------------------------

// On the bf16 MFMA, 32 token rows per wave:
//   C^T [ranks x rows] = V_r^T . X^T   (A: basis rows from LDS; B: the rows of
//                                       X, one 16-byte load per k-step)
//   Xhat^T [D x rows]  = V_r . C^T     (A: basis from LDS; B: the C^T
//                                       accumulator, in registers)
// with fp32 accumulation.  The basis and the coefficients are each split into
// three bf16 terms (hi + mid + lo: the residual of each rounding is exact in
// fp32, so together they carry the fp32 value to ~2^-24 relative) and the six
// products of the second stage above that size are summed, so the result
// carries fp32-level error before its bf16 rounding.  The C^T accumulator
// holds, in lane l, row l % 32 and ranks 8(r/4) + 4(l/32) + r%4 of register
// r: read 8 registers at a time it is the B operand of a 16-rank k-step
// whose rank slots are {4g + e, 8 + 4g + e} (g = l/32, e < 4), and the basis
// operand takes its rank slots in that same order.
constexpr int kProjWaves = 4;

__device__ __forceinline__ void split3(float v, uint16_t (&t)[3]) {
#pragma unroll
  for (int s3 = 0; s3 < 3; ++s3) {
    const uint32_t h = pack_bf16x2(v, 0.0f);
    t[s3] = (uint16_t)(h & 0xffffu);
    v -= bf16_lo(h);
  }
}

// A workgroup splits the basis into LDS once, then projects `tiles`
// consecutive tiles of 32 * kProjWaves rows (the split costs more than one
// tile's rows).
template <int D, int RP>
__global__ __launch_bounds__(64 * kProjWaves) void project_kernel(uint16_t* __restrict__ x,
                                                                  const float* __restrict__ wbasis,
                                                                  int L, int tiles) {
  constexpr int RPAD = RP < 32 ? 32 : RP;     // ranks of the first stage's tiles
  constexpr int RT = RPAD / 32;               // first-stage rank tiles
  constexpr int KS1 = D / 16;                 // first-stage k-steps (channels)
  constexpr int KS2 = RP < 16 ? 1 : RP / 16;  // second-stage k-steps (ranks)
  constexpr int DT = D / 32;                  // second-stage channel tiles
  constexpr int VT_LD = D + 8;                // V^T rows in LDS (bf16), padded
  constexpr int V_LD = RPAD + 4;              // V rows in LDS (bf16), padded
  __shared__ __attribute__((aligned(16))) uint16_t s_vt[3][RPAD * VT_LD];
  __shared__ __attribute__((aligned(16))) uint16_t s_v[3][D * V_LD];

  const uint64_t bh = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  const float* wb = wbasis + bh * (uint64_t)(D * RP);
  for (int e = tid; e < D * RPAD; e += 64 * kProjWaves) {
    const int d = e / RPAD, k = e % RPAD;
    uint16_t t[3];
    split3(k < RP ? wb[d * RP + k] : 0.0f, t);
#pragma unroll
    for (int s3 = 0; s3 < 3; ++s3) {
      s_vt[s3][k * VT_LD + d] = t[s3];
      s_v[s3][d * V_LD + k] = t[s3];
    }
  }
  __syncthreads();

  uint16_t* xb = x + bh * (uint64_t)L * D;
  // this wave's rows of tile tt; rows past the end re-read the last row and
  // are not stored (that row belongs to this wave, whose reads all precede
  // its stores)
  auto row_of = [&](int tt) { return ((blockIdx.x * tiles + tt) * kProjWaves + wave) * 32; };
  auto load_rows = [&](v4i(&dst)[KS1], int row0) {
    const int row = min(row0 + l32, L - 1);
#pragma unroll
    for (int ks = 0; ks < KS1; ++ks)
      dst[ks] = *reinterpret_cast<const v4i*>(xb + (size_t)row * D + 16 * ks + 8 * g);
  };
  v4i xo[KS1];
  if (row_of(0) < L) load_rows(xo, row_of(0));
  for (int tt = 0; tt < tiles; ++tt) {
    const int row0 = row_of(tt);
    if (row0 >= L) break;  // past the only barrier
    // the next tile's rows load while this one is computed
    v4i xn[KS1];
    const bool more = tt + 1 < tiles && row_of(tt + 1) < L;
    if (more) load_rows(xn, row_of(tt + 1));
    v16f ct[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int r = 0; r < 16; ++r) ct[rt][r] = 0.0f;
#pragma unroll
    for (int ks = 0; ks < KS1; ++ks) {
      const v8bf b = __builtin_bit_cast(v8bf, xo[ks]);
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int s3 = 0; s3 < 3; ++s3) {
          const v8bf a = *reinterpret_cast<const v8bf*>(
              &s_vt[s3][(32 * rt + l32) * VT_LD + 16 * ks + 8 * g]);
          ct[rt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, ct[rt], 0, 0, 0);
        }
    }

    // coefficient splits as second-stage B operands: k-step ks2 takes
    // registers 8 (ks2 % 2) .. +7 of rank tile ks2 / 2
    uint32_t cb[3][KS2][4];
#pragma unroll
    for (int ks2 = 0; ks2 < KS2; ++ks2)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = 8 * (ks2 & 1) + 2 * j;
        float c0 = ct[ks2 >> 1][r], c1 = ct[ks2 >> 1][r + 1];
#pragma unroll
        for (int s3 = 0; s3 < 3; ++s3) {
          const uint32_t h = pack_bf16x2(c0, c1);
          cb[s3][ks2][j] = h;
          c0 -= bf16_lo(h);
          c1 -= bf16_hi(h);
        }
      }

    const bool store = row0 + l32 < L;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      v16f o;
#pragma unroll
      for (int r = 0; r < 16; ++r) o[r] = 0.0f;
#pragma unroll
      for (int ks2 = 0; ks2 < KS2; ++ks2) {
        v8bf a[3], b[3];
#pragma unroll
        for (int s3 = 0; s3 < 3; ++s3) {
          const uint16_t* base = &s_v[s3][(32 * dt + l32) * V_LD + 16 * ks2 + 4 * g];
          const uint2 lo4 = *reinterpret_cast<const uint2*>(base);
          const uint2 hi4 = *reinterpret_cast<const uint2*>(base + 8);
          a[s3] = __builtin_bit_cast(v8bf, make_uint4(lo4.x, lo4.y, hi4.x, hi4.y));
          b[s3] = __builtin_bit_cast(v8bf, make_uint4(cb[s3][ks2][0], cb[s3][ks2][1],
                                                      cb[s3][ks2][2], cb[s3][ks2][3]));
        }
        // smallest products first
        o = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[1], b[1], o, 0, 0, 0);
        o = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[2], b[0], o, 0, 0, 0);
        o = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0], b[2], o, 0, 0, 0);
        o = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[1], b[0], o, 0, 0, 0);
        o = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0], b[1], o, 0, 0, 0);
        o = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0], b[0], o, 0, 0, 0);
      }
      if (store) {
        uint16_t* xr = xb + (size_t)(row0 + l32) * D + 32 * dt + 4 * g;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          *reinterpret_cast<uint2*>(xr + 8 * q) = make_uint2(
              pack_bf16x2(o[4 * q], o[4 * q + 1]), pack_bf16x2(o[4 * q + 2], o[4 * q + 3]));
      }
    }
    if (more) {
#pragma unroll
      for (int ks = 0; ks < KS1; ++ks) xo[ks] = xn[ks];
    }
  }
}

template <int D>
hipError_t launch_d(const qsa_dims& d, uint16_t* dr, int rank, float* basis, float* eigvals,
                    float* partial, float* wbasis, hipStream_t st) {
  const ProjectPlan pl = project_plan(d, rank);
  const uint32_t bh = (uint32_t)(d.batch * d.heads);
  hipLaunchKernelGGL((gram_kernel<D>), dim3((uint32_t)pl.chunks, bh), dim3(kThreads), 0, st, dr,
                     partial, d.seq_len, pl.chunk);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((jacobi_kernel<D>), dim3(bh), dim3(kJacobiThreads), 0, st, partial, pl.chunks,
                     rank, pl.rank_pad, eigvals, basis, wbasis);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // about 2048 workgroups in all, each over `tiles` row tiles
  const int64_t n_tiles = (d.seq_len + 32 * kProjWaves - 1) / (32 * kProjWaves);
  const int64_t want = (n_tiles * (int64_t)bh + 2047) / 2048;
  const int tiles = (int)(want < 1 ? 1 : want > n_tiles ? n_tiles : want);
  const dim3 grid((uint32_t)((n_tiles + tiles - 1) / tiles), bh);
  const dim3 block(64 * kProjWaves);
  switch (pl.rank_pad) {
    case 8:
      hipLaunchKernelGGL((project_kernel<D, 8>), grid, block, 0, st, dr, wbasis,
                         d.seq_len, tiles);
      break;
    case 16:
      hipLaunchKernelGGL((project_kernel<D, 16>), grid, block, 0, st, dr, wbasis,
                         d.seq_len, tiles);
      break;
    case 32:
      hipLaunchKernelGGL((project_kernel<D, 32>), grid, block, 0, st, dr, wbasis,
                         d.seq_len, tiles);
      break;
    default:
      hipLaunchKernelGGL((project_kernel<D, 64>), grid, block, 0, st, dr, wbasis,
                         d.seq_len, tiles);
      break;
  }
  return hipGetLastError();
}

}  // namespace

ProjectPlan project_plan(const qsa_dims& d, int rank) {
  ProjectPlan p;
  const int64_t L = d.seq_len;
  int chunks = (int)((L + 2047) / 2048);
  chunks = chunks < 1 ? 1 : (chunks > 32 ? 32 : chunks);
  int64_t chunk = (L + chunks - 1) / chunks;
  chunk = (chunk + 63) / 64 * 64;
  p.chunk = (int)chunk;
  p.chunks = (int)((L + chunk - 1) / chunk);
  if (p.chunks < 1) p.chunks = 1;
  p.rank_pad = rank <= 8 ? 8 : rank <= 16 ? 16 : rank <= 32 ? 32 : 64;
  const uint64_t bh = (uint64_t)d.batch * d.heads;
  p.partial_floats = bh * p.chunks * (uint64_t)d.head_dim * d.head_dim;
  p.wbasis_floats = bh * (uint64_t)d.head_dim * QSA_MAX_RANK;
  return p;
}

hipError_t launch_project_residual(const qsa_dims& d, uint16_t* dr, int rank, float* basis,
                                   float* eigvals, float* work, hipStream_t s) {
  const ProjectPlan pl = project_plan(d, rank);
  float* partial = work;
  float* wbasis = work + pl.partial_floats;
  if (d.head_dim == 128) return launch_d<128>(d, dr, rank, basis, eigvals, partial, wbasis, s);
  return launch_d<64>(d, dr, rank, basis, eigvals, partial, wbasis, s);
}

}  // namespace qsa
