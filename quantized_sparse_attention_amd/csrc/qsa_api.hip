// C ABI of the QuantSparse attention hot path: argument validation, device
// check and kernel launch on the caller's stream.  No allocation, no state
// kept across calls (beyond a per-device cache of the architecture check),
// no exceptions across the boundary.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <atomic>

#include "qsa_internal.h"

namespace {

thread_local char g_detail[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_detail, sizeof(g_detail), fmt, ap);
  va_end(ap);
  return status;
}

int ok() {
  g_detail[0] = '\0';
  return QSA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

#define REQUIRE_PTR(p)                                                          \
  do {                                                                          \
    if ((p) == nullptr) return fail(QSA_ERR_NULL, "%s: %s is NULL", fn, #p);    \
    if (!aligned16(p))                                                          \
      return fail(QSA_ERR_ALIGN, "%s: %s is not 16-byte aligned", fn, #p);      \
  } while (0)

#define OPTIONAL_PTR(p)                                                         \
  do {                                                                          \
    if ((p) != nullptr && !aligned16(p))                                        \
      return fail(QSA_ERR_ALIGN, "%s: %s is not 16-byte aligned", fn, #p);      \
  } while (0)

int check_dims(const char* fn, const qsa_dims* d) {
  if (d == nullptr) return fail(QSA_ERR_NULL, "%s: dims is NULL", fn);
  if (d->batch < 1 || d->heads < 1 || d->seq_len < 1)
    return fail(QSA_ERR_SHAPE, "%s: batch=%d heads=%d seq_len=%d must all be >= 1", fn,
                d->batch, d->heads, d->seq_len);
  if (d->head_dim != 64 && d->head_dim != 128)
    return fail(QSA_ERR_SHAPE, "%s: head_dim=%d must be 64 or 128", fn, d->head_dim);
  if (d->block != 64 && d->block != 128)
    return fail(QSA_ERR_SHAPE, "%s: block=%d must be 64 or 128", fn, d->block);
  const int64_t nb = (d->seq_len + (int64_t)d->block - 1) / d->block;
  const int64_t work = (int64_t)d->batch * d->heads * nb;
  if (work > QSA_MAX_WORK_BLOCKS)
    return fail(QSA_ERR_SHAPE, "%s: batch*heads*blocks=%lld exceeds QSA_MAX_WORK_BLOCKS=%d", fn,
                (long long)work, QSA_MAX_WORK_BLOCKS);
  return QSA_OK;
}

// Cached per-device answer to "is this a gfx950": 0 unknown, 1 yes, 2 no.
constexpr int kMaxDevices = 64;
std::atomic<int> g_arch_ok[kMaxDevices];

int check_device(const char* fn) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return fail(QSA_ERR_DEVICE, "%s: no current HIP device (%s)", fn, hipGetErrorString(e));
  int st = g_arch_ok[dev].load(std::memory_order_relaxed);
  if (st == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess)
      return fail(QSA_ERR_DEVICE, "%s: hipGetDeviceProperties failed (%s)", fn,
                  hipGetErrorString(e));
    st = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_arch_ok[dev].store(st, std::memory_order_relaxed);
    if (st == 2)
      return fail(QSA_ERR_DEVICE, "%s: device %d is %s, the kernels are built for gfx950 only",
                  fn, dev, prop.gcnArchName);
  }
  if (st != 1) return fail(QSA_ERR_DEVICE, "%s: device %d is not a gfx950", fn, dev);
  return QSA_OK;
}

int launched(const char* fn, hipError_t e) {
  if (e != hipSuccess)
    return fail(QSA_ERR_LAUNCH, "%s: kernel launch failed (%s)", fn, hipGetErrorString(e));
  return ok();
}

int check_attn_common(const char* fn, const qsa_dims* dims, const int8_t* q_codes,
                      const float* q_scales, const int8_t* k_codes, const float* k_scales,
                      const uint16_t* v, const int32_t* kept_idx, const int32_t* kept_cnt,
                      int32_t kmax, float sm_scale) {
  int st = check_dims(fn, dims);
  if (st) return st;
  const long long nb = ((long long)dims->seq_len + dims->block - 1) / dims->block;
  if (nb > QSA_MAX_BLOCKS)  // the kept sets are held as LDS bitmaps of this many bits
    return fail(QSA_ERR_SHAPE, "%s: %lld blocks exceed QSA_MAX_BLOCKS=%d", fn, nb,
                QSA_MAX_BLOCKS);
  REQUIRE_PTR(q_codes);
  REQUIRE_PTR(q_scales);
  REQUIRE_PTR(k_codes);
  REQUIRE_PTR(k_scales);
  REQUIRE_PTR(v);
  REQUIRE_PTR(kept_idx);
  REQUIRE_PTR(kept_cnt);
  if (kmax < 1) return fail(QSA_ERR_PARAM, "%s: kmax=%d must be >= 1", fn, kmax);
  if (!(sm_scale > 0.0f) || !isfinite(sm_scale))
    return fail(QSA_ERR_PARAM, "%s: sm_scale=%g must be finite and > 0", fn, (double)sm_scale);
  return QSA_OK;
}

}  // namespace

extern "C" {

int qsa_version(void) { return QSA_VERSION; }

const char* qsa_last_error_detail(void) { return g_detail; }

const char* qsa_status_string(int status) {
  switch (status) {
    case QSA_OK: return "QSA_OK";
    case QSA_ERR_NULL: return "QSA_ERR_NULL: a required pointer is NULL";
    case QSA_ERR_SHAPE: return "QSA_ERR_SHAPE: unsupported or invalid shape";
    case QSA_ERR_PARAM: return "QSA_ERR_PARAM: a scalar argument is out of range";
    case QSA_ERR_ALIGN: return "QSA_ERR_ALIGN: a tensor pointer is not 16-byte aligned";
    case QSA_ERR_DEVICE: return "QSA_ERR_DEVICE: no usable gfx950 device";
    case QSA_ERR_LAUNCH: return "QSA_ERR_LAUNCH: kernel launch failed";
    default: return "unknown qsa status";
  }
}

int qsa_quantize(const qsa_dims* dims, const uint16_t* x, int8_t* codes, float* scales,
                 int32_t* pooled, void* stream) {
  const char* fn = "qsa_quantize";
  int st = check_dims(fn, dims);
  if (st) return st;
  REQUIRE_PTR(x);
  REQUIRE_PTR(codes);
  REQUIRE_PTR(scales);
  REQUIRE_PTR(pooled);
  if ((st = check_device(fn))) return st;
  (void)hipGetLastError();
  return launched(fn, qsa::launch_quantize(*dims, x, codes, scales, pooled,
                                           static_cast<hipStream_t>(stream)));
}

int qsa_quantize_rotated(const qsa_dims* dims, const uint16_t* x, int8_t* codes, float* scales,
                         int32_t* pooled, void* stream) {
  const char* fn = "qsa_quantize_rotated";
  int st = check_dims(fn, dims);
  if (st) return st;
  REQUIRE_PTR(x);
  REQUIRE_PTR(codes);
  REQUIRE_PTR(scales);
  REQUIRE_PTR(pooled);
  if ((st = check_device(fn))) return st;
  (void)hipGetLastError();
  return launched(fn, qsa::launch_quantize_rotated(*dims, x, codes, scales, pooled,
                                           static_cast<hipStream_t>(stream)));
}

namespace {
// Arguments of both select entry points; fills band on success.
int check_select(const char* fn, const qsa_dims* dims, const int32_t* pooled_q,
                 const float* scale_q, const int32_t* pooled_k, const float* scale_k,
                 int32_t topk, const int32_t* band_offsets, int32_t n_band, int32_t kmax,
                 int32_t* kept_idx, int32_t* kept_cnt, qsa::Band& band) {
  int st = check_dims(fn, dims);
  if (st) return st;
  REQUIRE_PTR(pooled_q);
  REQUIRE_PTR(scale_q);
  REQUIRE_PTR(pooled_k);
  REQUIRE_PTR(scale_k);
  REQUIRE_PTR(kept_idx);
  REQUIRE_PTR(kept_cnt);
  const int64_t nb = (dims->seq_len + (int64_t)dims->block - 1) / dims->block;
  if (nb > QSA_MAX_BLOCKS)
    return fail(QSA_ERR_SHAPE, "%s: %lld blocks exceed QSA_MAX_BLOCKS=%d", fn, (long long)nb,
                QSA_MAX_BLOCKS);
  if (topk < 0) return fail(QSA_ERR_PARAM, "%s: topk=%d must be >= 0", fn, topk);
  if (n_band < 0 || n_band > QSA_MAX_BAND)
    return fail(QSA_ERR_PARAM, "%s: n_band=%d must be in [0, %d]", fn, n_band, QSA_MAX_BAND);
  if (n_band > 0 && band_offsets == nullptr)
    return fail(QSA_ERR_NULL, "%s: band_offsets is NULL with n_band=%d", fn, n_band);
  band = qsa::Band{};
  bool has_diag = false;
  for (int b = 0; b < n_band; ++b) {
    band.off[b] = band_offsets[b];
    has_diag |= band_offsets[b] == 0;
  }
  band.n = n_band;
  if (topk == 0 && !has_diag)
    return fail(QSA_ERR_PARAM, "%s: topk=0 without band offset 0 can leave a row empty", fn);
  const int64_t need = nb < (int64_t)topk + n_band ? nb : (int64_t)topk + n_band;
  if (kmax < 1 || kmax < need)
    return fail(QSA_ERR_PARAM, "%s: kmax=%d must be >= min(nb, topk + n_band)=%lld", fn, kmax,
                (long long)need);
  return QSA_OK;
}
}  // namespace

int qsa_select_blocks(const qsa_dims* dims, const int32_t* pooled_q, const float* scale_q,
                      const int32_t* pooled_k, const float* scale_k, int32_t topk,
                      const int32_t* band_offsets, int32_t n_band, int32_t kmax,
                      int32_t* kept_idx, int32_t* kept_cnt, void* stream) {
  const char* fn = "qsa_select_blocks";
  qsa::Band band;
  int st = check_select(fn, dims, pooled_q, scale_q, pooled_k, scale_k, topk, band_offsets,
                        n_band, kmax, kept_idx, kept_cnt, band);
  if (st) return st;
  if ((st = check_device(fn))) return st;
  (void)hipGetLastError();
  return launched(fn, qsa::launch_select(*dims, pooled_q, scale_q, pooled_k, scale_k, topk, band,
                                         kmax, kept_idx, kept_cnt,
                                         static_cast<hipStream_t>(stream)));
}

uint64_t qsa_select_slice_bytes(const qsa_dims* dims) {
  if (check_dims("qsa_select_slice_bytes", dims)) return 0;
  return qsa::select_slice_bytes(*dims);
}

int qsa_select_blocks_work(const qsa_dims* dims, const int32_t* pooled_q, const float* scale_q,
                           const int32_t* pooled_k, const float* scale_k, int32_t topk,
                           const int32_t* band_offsets, int32_t n_band, int32_t kmax,
                           int32_t* kept_idx, int32_t* kept_cnt, void* work,
                           uint64_t work_bytes, void* stream) {
  const char* fn = "qsa_select_blocks_work";
  qsa::Band band;
  int st = check_select(fn, dims, pooled_q, scale_q, pooled_k, scale_k, topk, band_offsets,
                        n_band, kmax, kept_idx, kept_cnt, band);
  if (st) return st;
  OPTIONAL_PTR(work);
  if ((st = check_device(fn))) return st;
  (void)hipGetLastError();
  return launched(fn, qsa::launch_select_work(*dims, pooled_q, scale_q, pooled_k, scale_k, topk,
                                              band, kmax, kept_idx, kept_cnt, work, work_bytes,
                                              static_cast<hipStream_t>(stream)));
}

int qsa_sparse_attn(const qsa_dims* dims, const int8_t* q_codes, const float* q_scales,
                    const int8_t* k_codes, const float* k_scales, const uint16_t* v,
                    const int32_t* kept_idx, const int32_t* kept_cnt, int32_t kmax,
                    float sm_scale, const uint16_t* r, const uint16_t* dr, uint16_t* out,
                    void* stream) {
  const char* fn = "qsa_sparse_attn";
  int st = check_attn_common(fn, dims, q_codes, q_scales, k_codes, k_scales, v, kept_idx,
                             kept_cnt, kmax, sm_scale);
  if (st) return st;
  OPTIONAL_PTR(r);
  OPTIONAL_PTR(dr);
  REQUIRE_PTR(out);
  if ((st = check_device(fn))) return st;
  qsa::AttnArgs a{};
  a.q_codes = q_codes;
  a.q_scales = q_scales;
  a.k_codes = k_codes;
  a.k_scales = k_scales;
  a.v = v;
  a.kept_idx = kept_idx;
  a.kept_cnt = kept_cnt;
  a.kmax = kmax;
  a.sm_scale = sm_scale;
  a.r_in = r;
  a.dr_in = dr;
  a.out = out;
  (void)hipGetLastError();
  return launched(fn, qsa::launch_sparse_attn(*dims, a, static_cast<hipStream_t>(stream)));
}

int qsa_order_query_blocks(const qsa_dims* dims, const int32_t* kept_idx,
                           const int32_t* kept_cnt, int32_t kmax, int32_t* order, void* stream) {
  const char* fn = "qsa_order_query_blocks";
  int st = check_dims(fn, dims);
  if (st) return st;
  const long long nb = ((long long)dims->seq_len + dims->block - 1) / dims->block;
  if (nb > QSA_MAX_BLOCKS)
    return fail(QSA_ERR_SHAPE, "%s: %lld blocks exceed QSA_MAX_BLOCKS=%d", fn, nb,
                QSA_MAX_BLOCKS);
  REQUIRE_PTR(kept_idx);
  REQUIRE_PTR(kept_cnt);
  REQUIRE_PTR(order);
  if (kmax < 1) return fail(QSA_ERR_PARAM, "%s: kmax=%d must be >= 1", fn, kmax);
  if ((st = check_device(fn))) return st;
  (void)hipGetLastError();
  return launched(fn, qsa::launch_order(*dims, kept_idx, kept_cnt, kmax, order,
                                        static_cast<hipStream_t>(stream)));
}

int qsa_sparse_attn_ordered(const qsa_dims* dims, const int8_t* q_codes, const float* q_scales,
                            const int8_t* k_codes, const float* k_scales, const uint16_t* v,
                            const int32_t* kept_idx, const int32_t* kept_cnt, int32_t kmax,
                            const int32_t* order, float sm_scale, const uint16_t* r,
                            const uint16_t* dr, uint16_t* out, void* stream) {
  const char* fn = "qsa_sparse_attn_ordered";
  REQUIRE_PTR(order);
  int st = check_attn_common(fn, dims, q_codes, q_scales, k_codes, k_scales, v, kept_idx,
                             kept_cnt, kmax, sm_scale);
  if (st) return st;
  OPTIONAL_PTR(r);
  OPTIONAL_PTR(dr);
  REQUIRE_PTR(out);
  if ((st = check_device(fn))) return st;
  qsa::AttnArgs a{};
  a.q_codes = q_codes;
  a.q_scales = q_scales;
  a.k_codes = k_codes;
  a.k_scales = k_scales;
  a.v = v;
  a.kept_idx = kept_idx;
  a.kept_cnt = kept_cnt;
  a.order = order;
  a.kmax = kmax;
  a.sm_scale = sm_scale;
  a.r_in = r;
  a.dr_in = dr;
  a.out = out;
  (void)hipGetLastError();
  return launched(fn, qsa::launch_sparse_attn(*dims, a, static_cast<hipStream_t>(stream)));
}

namespace {
int full_attn_residual(const char* fn, const qsa_dims* dims, const int8_t* q_codes,
                       const float* q_scales, const int8_t* k_codes, const float* k_scales,
                       const uint16_t* v, const int32_t* kept_idx, const int32_t* kept_cnt,
                       int32_t kmax, const int32_t* order, float sm_scale, int32_t has_prev,
                       uint16_t* r, uint16_t* dr, uint16_t* out_full, void* stream) {
  int st = check_attn_common(fn, dims, q_codes, q_scales, k_codes, k_scales, v, kept_idx,
                             kept_cnt, kmax, sm_scale);
  if (st) return st;
  REQUIRE_PTR(r);
  REQUIRE_PTR(dr);
  REQUIRE_PTR(out_full);
  if (has_prev != 0 && has_prev != 1)
    return fail(QSA_ERR_PARAM, "%s: has_prev=%d must be 0 or 1", fn, has_prev);
  if ((st = check_device(fn))) return st;
  qsa::AttnArgs a{};
  a.q_codes = q_codes;
  a.q_scales = q_scales;
  a.k_codes = k_codes;
  a.k_scales = k_scales;
  a.v = v;
  a.kept_idx = kept_idx;
  a.kept_cnt = kept_cnt;
  a.order = order;
  a.kmax = kmax;
  a.sm_scale = sm_scale;
  a.r_out = r;
  a.dr_out = dr;
  a.has_prev = has_prev;
  a.out = out_full;
  (void)hipGetLastError();
  return launched(fn, qsa::launch_full_attn_residual(*dims, a, static_cast<hipStream_t>(stream)));
}
}  // namespace

int qsa_full_attn_residual(const qsa_dims* dims, const int8_t* q_codes, const float* q_scales,
                           const int8_t* k_codes, const float* k_scales, const uint16_t* v,
                           const int32_t* kept_idx, const int32_t* kept_cnt, int32_t kmax,
                           float sm_scale, int32_t has_prev, uint16_t* r, uint16_t* dr,
                           uint16_t* out_full, void* stream) {
  return full_attn_residual("qsa_full_attn_residual", dims, q_codes, q_scales, k_codes,
                            k_scales, v, kept_idx, kept_cnt, kmax, nullptr, sm_scale, has_prev,
                            r, dr, out_full, stream);
}

int qsa_full_attn_residual_ordered(const qsa_dims* dims, const int8_t* q_codes,
                                   const float* q_scales, const int8_t* k_codes,
                                   const float* k_scales, const uint16_t* v,
                                   const int32_t* kept_idx, const int32_t* kept_cnt,
                                   int32_t kmax, const int32_t* order, float sm_scale,
                                   int32_t has_prev, uint16_t* r, uint16_t* dr,
                                   uint16_t* out_full, void* stream) {
  const char* fn = "qsa_full_attn_residual_ordered";
  REQUIRE_PTR(order);
  return full_attn_residual(fn, dims, q_codes, q_scales, k_codes, k_scales, v, kept_idx,
                            kept_cnt, kmax, order, sm_scale, has_prev, r, dr, out_full, stream);
}

int qsa_apply_residual(const qsa_dims* dims, const uint16_t* sparse_out, const uint16_t* r,
                       const uint16_t* dr, uint16_t* out, void* stream) {
  const char* fn = "qsa_apply_residual";
  int st = check_dims(fn, dims);
  if (st) return st;
  REQUIRE_PTR(sparse_out);
  REQUIRE_PTR(r);
  OPTIONAL_PTR(dr);
  REQUIRE_PTR(out);
  if ((st = check_device(fn))) return st;
  (void)hipGetLastError();
  return launched(fn, qsa::launch_apply_residual(*dims, sparse_out, r, dr, out,
                                                 static_cast<hipStream_t>(stream)));
}

uint64_t qsa_project_work_bytes(const qsa_dims* dims, int32_t rank) {
  if (check_dims("qsa_project_work_bytes", dims) != QSA_OK) return 0;
  if (rank < 1 || rank > dims->head_dim || rank > QSA_MAX_RANK) return 0;
  const qsa::ProjectPlan p = qsa::project_plan(*dims, rank);
  return (p.partial_floats + p.wbasis_floats) * sizeof(float);
}

int qsa_project_residual(const qsa_dims* dims, uint16_t* dr, int32_t rank, float* basis,
                         float* eigvals, void* work, uint64_t work_bytes, void* stream) {
  const char* fn = "qsa_project_residual";
  int st = check_dims(fn, dims);
  if (st) return st;
  REQUIRE_PTR(dr);
  REQUIRE_PTR(basis);
  REQUIRE_PTR(eigvals);
  REQUIRE_PTR(work);
  if (rank < 1 || rank > dims->head_dim || rank > QSA_MAX_RANK)
    return fail(QSA_ERR_PARAM, "%s: rank=%d must be in [1, min(D=%d, %d)]", fn, rank,
                dims->head_dim, QSA_MAX_RANK);
  if ((int64_t)dims->batch * dims->heads > 65535)
    return fail(QSA_ERR_SHAPE, "%s: batch*heads=%lld exceeds 65535", fn,
                (long long)dims->batch * dims->heads);
  const uint64_t need = qsa_project_work_bytes(dims, rank);
  if (work_bytes < need)
    return fail(QSA_ERR_PARAM, "%s: work_bytes=%llu is less than the %llu needed", fn,
                (unsigned long long)work_bytes, (unsigned long long)need);
  if ((st = check_device(fn))) return st;
  (void)hipGetLastError();
  return launched(fn, qsa::launch_project_residual(*dims, dr, rank, basis, eigvals,
                                                   static_cast<float*>(work),
                                                   static_cast<hipStream_t>(stream)));
}

int qsa_l1_change(const qsa_dims* dims, const uint16_t* prev, const uint16_t* cur, double* sums,
                  void* work, uint64_t work_bytes, void* stream) {
  const char* fn = "qsa_l1_change";
  int st = check_dims(fn, dims);
  if (st) return st;
  REQUIRE_PTR(prev);
  REQUIRE_PTR(cur);
  REQUIRE_PTR(sums);
  REQUIRE_PTR(work);
  if (work_bytes < QSA_L1_WORK_BYTES)
    return fail(QSA_ERR_PARAM, "%s: work_bytes=%llu is less than %d", fn,
                (unsigned long long)work_bytes, QSA_L1_WORK_BYTES);
  if ((st = check_device(fn))) return st;
  const uint64_t n = (uint64_t)dims->batch * dims->heads * dims->seq_len * dims->head_dim;
  (void)hipGetLastError();
  return launched(fn, qsa::launch_l1_change(n, prev, cur, sums, static_cast<double*>(work),
                                            static_cast<hipStream_t>(stream)));
}

int qsa_l1_change_noalloc(const qsa_dims* dims, const uint16_t* prev, const uint16_t* cur,
                          double* sums, void* stream) {
  const char* fn = "qsa_l1_change_noalloc";
  int st = check_dims(fn, dims);
  if (st) return st;
  REQUIRE_PTR(prev);
  REQUIRE_PTR(cur);
  REQUIRE_PTR(sums);
  if ((st = check_device(fn))) return st;
  double* work = nullptr;
  hipError_t e = qsa::l1_static_scratch(&work);
  if (e != hipSuccess)
    return fail(QSA_ERR_DEVICE, "%s: the library's scratch is not available on this device (%s)",
                fn, hipGetErrorString(e));
  const uint64_t n = (uint64_t)dims->batch * dims->heads * dims->seq_len * dims->head_dim;
  (void)hipGetLastError();
  return launched(fn, qsa::launch_l1_change(n, prev, cur, sums, work,
                                            static_cast<hipStream_t>(stream)));
}

int qsa_window_kept(const qsa_dims* dims, int32_t window, int32_t kmax, int32_t* kept_idx,
                    int32_t* kept_cnt, void* stream) {
  const char* fn = "qsa_window_kept";
  int st = check_dims(fn, dims);
  if (st) return st;
  REQUIRE_PTR(kept_idx);
  REQUIRE_PTR(kept_cnt);
  if (window < dims->block || window % dims->block || dims->seq_len % window)
    return fail(QSA_ERR_PARAM, "%s: window=%d must be a multiple of block=%d dividing seq_len=%d",
                fn, window, dims->block, dims->seq_len);
  if (kmax < window / dims->block)
    return fail(QSA_ERR_PARAM, "%s: kmax=%d < window/block=%d", fn, kmax, window / dims->block);
  if ((st = check_device(fn))) return st;
  (void)hipGetLastError();
  return launched(fn, qsa::launch_window_kept(*dims, window, kmax, kept_idx, kept_cnt,
                                              static_cast<hipStream_t>(stream)));
}

int qsa_reorder_windows(const qsa_dims* dims, int32_t window, int32_t inverse, const uint16_t* x,
                        uint16_t* y, void* stream) {
  const char* fn = "qsa_reorder_windows";
  int st = check_dims(fn, dims);
  if (st) return st;
  REQUIRE_PTR(x);
  REQUIRE_PTR(y);
  if (window < 1 || dims->seq_len % window)
    return fail(QSA_ERR_PARAM, "%s: window=%d must divide seq_len=%d", fn, window,
                dims->seq_len);
  if (inverse != 0 && inverse != 1)
    return fail(QSA_ERR_PARAM, "%s: inverse=%d must be 0 or 1", fn, inverse);
  if ((st = check_device(fn))) return st;
  (void)hipGetLastError();
  return launched(fn, qsa::launch_reorder(*dims, window, inverse, x, y,
                                          static_cast<hipStream_t>(stream)));
}

static bool squad_window_ok(const qsa_dims* d, int32_t window) {
  return window >= d->block && window % d->block == 0 && d->seq_len % window == 0 &&
         (d->seq_len / window) % d->block == 0;
}

uint64_t qsa_squad_work_bytes(const qsa_dims* dims, int32_t window) {
  if (check_dims("qsa_squad_work_bytes", dims) != QSA_OK) return 0;
  if (!squad_window_ok(dims, window)) return 0;
  return qsa::squad_plan(*dims, window).bytes;
}

int qsa_squad_attention(const qsa_dims* dims, const uint16_t* q, const uint16_t* k,
                        const uint16_t* v, int32_t window, float sm_scale, uint16_t* out,
                        void* work, uint64_t work_bytes, void* stream) {
  const char* fn = "qsa_squad_attention";
  int st = check_dims(fn, dims);
  if (st) return st;
  REQUIRE_PTR(q);
  REQUIRE_PTR(k);
  REQUIRE_PTR(v);
  REQUIRE_PTR(out);
  REQUIRE_PTR(work);
  if (!squad_window_ok(dims, window))
    return fail(QSA_ERR_PARAM,
                "%s: window=%d and seq_len/window must both be multiples of block=%d", fn,
                window, dims->block);
  if (!(sm_scale > 0.0f) || !isfinite(sm_scale))
    return fail(QSA_ERR_PARAM, "%s: sm_scale=%g must be positive and finite", fn, sm_scale);
  const int64_t nb = dims->seq_len / dims->block;
  if (nb > QSA_MAX_BLOCKS)
    return fail(QSA_ERR_SHAPE, "%s: %lld blocks exceed %d", fn, (long long)nb, QSA_MAX_BLOCKS);
  const uint64_t need = qsa::squad_plan(*dims, window).bytes;
  if (work_bytes < need)
    return fail(QSA_ERR_PARAM, "%s: work_bytes=%llu is less than the %llu needed", fn,
                (unsigned long long)work_bytes, (unsigned long long)need);
  if ((st = check_device(fn))) return st;
  (void)hipGetLastError();
  return launched(fn, qsa::launch_squad(*dims, q, k, v, window, sm_scale, out,
                                        static_cast<char*>(work),
                                        static_cast<hipStream_t>(stream)));
}

}  // extern "C"
