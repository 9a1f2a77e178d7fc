// Internal declarations shared by the C-ABI layer and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qsa.h"

namespace qsa {

// ---------------------------------------------------------------------------
// vector types of the gfx950 MFMA builtins
// ---------------------------------------------------------------------------
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef short v4s __attribute__((ext_vector_type(4)));
// LDS (address space 3) pointer types for the gfx950 LDS builtins
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) v4s lds_v4s_t;

// bf16 bit pattern -> fp32 (exact)
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// two fp32 -> packed bf16 pair (round to nearest even; v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  v2f t = {a, b};
  v2bf r = __builtin_convertvector(t, v2bf);
  return __builtin_bit_cast(uint32_t, r);
}

// Map a linear workgroup id onto a logical work index so that each of the 8
// XCDs (which receive workgroups round-robin) walks one contiguous range of
// logical indices.  A bijection on [0, n).
__device__ __forceinline__ uint32_t xcd_contiguous(uint32_t p, uint32_t n) {
  const uint32_t q = n >> 3, rem = n & 7u;
  const uint32_t x = p & 7u, k = p >> 3;
  return x * q + (x < rem ? x : rem) + k;
}

struct Band {
  int32_t off[QSA_MAX_BAND];
  int32_t n;
};

// ---------------------------------------------------------------------------
// kernel launchers (one per entry point); arguments already validated
// ---------------------------------------------------------------------------
hipError_t launch_quantize(const qsa_dims& d, const uint16_t* x, int8_t* codes, float* scales,
                           int32_t* pooled, hipStream_t s);

hipError_t launch_quantize_rotated(const qsa_dims& d, const uint16_t* x, int8_t* codes,
                                   float* scales, int32_t* pooled, hipStream_t s);

// The codes and scales of qsa_quantize (no pooled sums) of x and, when x2 is
// not NULL, of a second tensor of the same shape in the same launch; with
// window > 0, of their rows in position-major order of windows of `window`
// tokens (row p*(L/window) + k is row k*window + p of x), gathered from x.
hipError_t launch_quantize_codes(const qsa_dims& d, const uint16_t* x, const uint16_t* x2,
                                 int window, int8_t* codes, int8_t* codes2, float* scales,
                                 float* scales2, hipStream_t s);

hipError_t launch_select(const qsa_dims& d, const int32_t* pooled_q, const float* scale_q,
                         const int32_t* pooled_k, const float* scale_k, int32_t topk,
                         const Band& band, int32_t kmax, int32_t* kept_idx, int32_t* kept_cnt,
                         hipStream_t s);

// launch_select through a workspace: the order keys of whole (b, h) slices
// (select_slice_bytes each) are written to `work`, then selected one query
// block per wave; as many slices per pass as work_bytes holds.  With no room
// for one slice, or more than 2048 blocks, it is launch_select.
uint64_t select_slice_bytes(const qsa_dims& d);
hipError_t launch_select_work(const qsa_dims& d, const int32_t* pooled_q, const float* scale_q,
                              const int32_t* pooled_k, const float* scale_k, int32_t topk,
                              const Band& band, int32_t kmax, int32_t* kept_idx,
                              int32_t* kept_cnt, void* work, uint64_t work_bytes, hipStream_t s);

struct AttnArgs {
  const int8_t* q_codes;
  const float* q_scales;
  const int8_t* k_codes;
  const float* k_scales;
  const uint16_t* v;
  const int32_t* kept_idx;
  const int32_t* kept_cnt;
  // optional processing order of the query blocks, int32 [B,H,nb] (a
  // permutation of 0..nb-1 per head), or NULL for ascending order
  const int32_t* order;
  int32_t kmax;
  float sm_scale;
  // sparse step: optional residual inputs; refresh step: r in/out, dr out
  const uint16_t* r_in;
  const uint16_t* dr_in;
  uint16_t* r_out;
  uint16_t* dr_out;
  int32_t has_prev;
  uint16_t* out;
  // sparse step only: where query row r's output (and r, dr) rows live.
  // 0: row r; 1: row (r % out_w) * (L / out_w) + r / out_w (window-major to
  // position-major); 2: row (r % m) * out_w + r / m with m = L / out_w (the
  // inverse).  out_w must divide L.
  int32_t out_map;
  int32_t out_w;
  // launch_sparse_attn_window only: query block i keeps the win_blocks blocks
  // of its own window, [i - i % win_blocks, ...) (kept_idx, kept_cnt unused)
  int32_t win_blocks;
  // launch_sparse_attn_window only, optional: bf16 Q [B,H,L,D], quantised in
  // the kernel as qsa_quantize would (q_codes, q_scales unused); with
  // q_pm_w > 0 its rows are taken in position-major order of windows of
  // q_pm_w tokens (row p*(L/q_pm_w) + k is token k*q_pm_w + p)
  const uint16_t* q_x;
  int32_t q_pm_w;
};

hipError_t launch_sparse_attn(const qsa_dims& d, const AttnArgs& a, hipStream_t s);
hipError_t launch_full_attn_residual(const qsa_dims& d, const AttnArgs& a, hipStream_t s);
// launch_sparse_attn for windowed kept sets (a.win_blocks), walked without
// kept lists; the query blocks in natural order (a.order unused)
hipError_t launch_sparse_attn_window(const qsa_dims& d, const AttnArgs& a, hipStream_t s);

hipError_t launch_order(const qsa_dims& d, const int32_t* kept_idx, const int32_t* kept_cnt,
                        int32_t kmax, int32_t* order, hipStream_t s);

// Chunking of qsa_project_residual's Gram matrices and its scratch layout:
// partial Gram matrices fp32 [B*H][chunks][D][D], then the zero-padded
// working basis fp32 [B*H][D][rank_pad] (room for QSA_MAX_RANK columns).
struct ProjectPlan {
  int chunk;      // tokens per chunk, a multiple of 64
  int chunks;     // chunks per (b, h)
  int rank_pad;   // rank rounded up to 8, 16, 32 or 64
  uint64_t partial_floats;
  uint64_t wbasis_floats;
};
ProjectPlan project_plan(const qsa_dims& d, int rank);

hipError_t launch_project_residual(const qsa_dims& d, uint16_t* dr, int rank, float* basis,
                                   float* eigvals, float* work, hipStream_t s);

// qsa_l1_change: per-block partial sums (2 doubles per block) in the scratch
constexpr int kL1MaxBlocks = QSA_L1_WORK_BYTES / 16;
int l1_change_blocks(uint64_t n_elements);
hipError_t launch_l1_change(uint64_t n_elements, const uint16_t* prev, const uint16_t* cur,
                            double* sums, double* work, hipStream_t s);
// The current device's address of the library's own QSA_L1_WORK_BYTES scratch
// (looked up once per device, on that device's first call).
hipError_t l1_static_scratch(double** work);

// SQuad two-pass attention: scratch layout (byte offsets, 256-aligned).
struct SquadPlan {
  uint64_t bytes;
  uint64_t k_codes, k_scales;
  uint64_t o_local;
};
SquadPlan squad_plan(const qsa_dims& d, int window);
hipError_t launch_window_kept(const qsa_dims& d, int window, int kmax, int32_t* kept_idx,
                              int32_t* kept_cnt, hipStream_t s);
hipError_t launch_reorder(const qsa_dims& d, int window, int inverse, const uint16_t* x,
                          uint16_t* y, hipStream_t s);
hipError_t launch_squad(const qsa_dims& d, const uint16_t* q, const uint16_t* k,
                        const uint16_t* v, int window, float sm_scale, uint16_t* out, char* work,
                        hipStream_t s);

hipError_t launch_apply_residual(const qsa_dims& d, const uint16_t* sparse_out,
                                 const uint16_t* r, const uint16_t* dr, uint16_t* out,
                                 hipStream_t s);

}  // namespace qsa
