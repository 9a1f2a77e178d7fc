// SQuad two-pass attention on this path's attention core.
//
// SQuad (gist.science/es/paper/2608.16585, technical summary, methodology
// §1): a sequence of n tokens is cut into windows of w consecutive tokens;
// a local softmax pass mixes each window, then a global softmax pass mixes
// the tokens at the same position of every window, with the local output as
// its values.  Both passes here are the int8/bf16 attention of attn.hip in
// its windowed mode (each query block keeps the blocks of its own window,
// walked without kept lists): the local pass over windows of w tokens in the
// natural order, the global pass over groups of n/w tokens in position-major
// order (token p of window k at p*(n/w) + k), so every group is a run of
// whole blocks and both passes run as dense tiles.
//
// Kernels of their own: the kept lists of block-diagonal attention (exported
// for callers that run the passes through qsa_sparse_attn), and the reorder
// between window-major and position-major order (a row gather of 16-byte
// chunks, HBM-bound; exported for callers that need it).  The
// operator itself reorders nothing: each pass quantises its own query rows
// from bf16 Q (gathered in position-major order for the global pass) and a
// launch per pass quantises K likewise, the local pass writes its output
// rows in position-major order and the global pass writes its rows back in
// the natural order (row maps of the attention epilogue).
#include "qsa_internal.h"

namespace qsa {
namespace {

__global__ __launch_bounds__(256) void window_kept_kernel(int32_t* __restrict__ kept_idx,
                                                          int32_t* __restrict__ kept_cnt,
                                                          uint64_t rows, int nb, int per,
                                                          int kmax) {
  const uint64_t row = (uint64_t)blockIdx.x * 256 + threadIdx.x;
  if (row >= rows) return;
  const int i = (int)(row % (uint64_t)nb);
  const int first = (i / per) * per;
  int32_t* kl = kept_idx + row * (uint64_t)kmax;
  for (int j = 0; j < kmax; ++j) kl[j] = j < per ? first + j : -1;
  kept_cnt[row] = per;
}

// y row r takes x row src(r): forward (window-major -> position-major)
// src(p*m + k) = k*w + p; inverse src(k*w + p) = p*m + k.
template <int D>
__global__ __launch_bounds__(256) void reorder_kernel(const uint16_t* __restrict__ x,
                                                      uint16_t* __restrict__ y, int n, int w,
                                                      int inverse, uint64_t chunks) {
  constexpr int CPR = D / 8;  // 16-byte chunks per row
  const uint64_t c = (uint64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= chunks) return;
  const uint64_t grow = c / CPR;  // global row over (b, h, r)
  const int part = (int)(c % CPR);
  const uint64_t bh = grow / (uint64_t)n;
  const int r = (int)(grow % (uint64_t)n);
  const int m = n / w;
  const int src = inverse ? (r % w) * m + r / w : (r % m) * w + r / m;
  const uint4 v =
      *reinterpret_cast<const uint4*>(x + ((bh * (uint64_t)n + src) * D) + part * 8);
  *reinterpret_cast<uint4*>(y + grow * D + part * 8) = v;
}

}  // namespace

hipError_t launch_window_kept(const qsa_dims& d, int window, int kmax, int32_t* kept_idx,
                              int32_t* kept_cnt, hipStream_t s) {
  const int nb = d.seq_len / d.block;
  const uint64_t rows = (uint64_t)d.batch * d.heads * nb;
  hipLaunchKernelGGL(window_kept_kernel, dim3((uint32_t)((rows + 255) / 256)), dim3(256), 0, s,
                     kept_idx, kept_cnt, rows, nb, window / d.block, kmax);
  return hipGetLastError();
}

hipError_t launch_reorder(const qsa_dims& d, int window, int inverse, const uint16_t* x,
                          uint16_t* y, hipStream_t s) {
  const uint64_t chunks = (uint64_t)d.batch * d.heads * d.seq_len * (d.head_dim / 8);
  const dim3 grid((uint32_t)((chunks + 255) / 256));
  if (d.head_dim == 128)
    hipLaunchKernelGGL((reorder_kernel<128>), grid, dim3(256), 0, s, x, y, d.seq_len, window,
                       inverse, chunks);
  else
    hipLaunchKernelGGL((reorder_kernel<64>), grid, dim3(256), 0, s, x, y, d.seq_len, window,
                       inverse, chunks);
  return hipGetLastError();
}

SquadPlan squad_plan(const qsa_dims& d, int window) {
  SquadPlan p;
  const uint64_t bh = (uint64_t)d.batch * d.heads;
  const uint64_t n = (uint64_t)d.seq_len, D = (uint64_t)d.head_dim;
  const uint64_t nb = n / (uint64_t)d.block;
  auto take = [&](uint64_t bytes) {
    const uint64_t off = p.bytes;
    p.bytes += (bytes + 255) / 256 * 256;
    return off;
  };
  p.bytes = 0;
  p.k_codes = take(bh * n * D);
  p.k_scales = take(bh * nb * 4);
  p.o_local = take(bh * n * D * 2);
  return p;
}

hipError_t launch_squad(const qsa_dims& d, const uint16_t* q, const uint16_t* k,
                        const uint16_t* v, int window, float sm_scale, uint16_t* out, char* work,
                        hipStream_t s) {
  const SquadPlan p = squad_plan(d, window);
  int8_t* kc = reinterpret_cast<int8_t*>(work + p.k_codes);
  float* ks = reinterpret_cast<float*>(work + p.k_scales);
  uint16_t* o_local = reinterpret_cast<uint16_t*>(work + p.o_local);
  const int m = d.seq_len / window;

  AttnArgs a{};
  a.q_x = q;  // each pass quantises its own query rows
  a.k_codes = kc;
  a.k_scales = ks;
  a.order = nullptr;  // windowed kept sets: no lists
  a.sm_scale = sm_scale;

  hipError_t e;
#define QSA_TRY(x) \
  if ((e = (x)) != hipSuccess) return e
  // local pass: windows of w tokens, natural order, values V; its output
  // rows are written in position-major order, ready as the global values
  QSA_TRY(launch_quantize_codes(d, k, nullptr, 0, kc, nullptr, ks, nullptr, s));
  a.q_pm_w = 0;
  a.v = v;
  a.out = o_local;
  a.out_map = 1;
  a.out_w = window;
  a.win_blocks = window / d.block;
  QSA_TRY(launch_sparse_attn_window(d, a, s));
  // global pass: groups of n/w tokens in position-major order (Q and K
  // quantised from rows gathered in that order), values the local output;
  // its output rows are written back in the natural order
  QSA_TRY(launch_quantize_codes(d, k, nullptr, window, kc, nullptr, ks, nullptr, s));
  a.q_pm_w = window;
  a.v = o_local;
  a.out = out;
  a.out_map = 2;
  a.win_blocks = m / d.block;
  QSA_TRY(launch_sparse_attn_window(d, a, s));
#undef QSA_TRY
  return hipSuccess;
}

}  // namespace qsa
