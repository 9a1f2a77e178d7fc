/*
 * qsa.h -- C ABI of the QuantSparse attention hot path on MI355X (gfx950).
 *
 * The method: video diffusion transformers run with 8-bit activations and
 * attention sparsified down to ~15 % density, with the information lost by
 * sparsification recovered by a cache of first- and second-order residuals
 * ("QuantSparse: Comprehensively Compressing Video Diffusion Transformer with
 * Model Quantization and Attention Sparsification", gist.science summaries
 * es/paper/2509.23681 and ko/paper/2509.23681, technical summary §1, §2A, §2B,
 * §4).  One attention layer step is:
 *
 *   sparse step : qsa_quantize(Q), qsa_quantize(K), qsa_select_blocks,
 *                 qsa_sparse_attn (with the cached r, dr added in its epilogue)
 *   refresh step: qsa_quantize(Q), qsa_quantize(K), qsa_select_blocks,
 *                 qsa_full_attn_residual (updates r and dr, outputs full attention)
 *
 * Conventions for every entry point
 *   - Tensors are DEVICE pointers, row-major and contiguous.  [B,H,L,D] means
 *     batch, head, token, channel.  bf16 data are passed as uint16_t bit
 *     patterns.  nb = ceil(seq_len / block) token blocks per (batch, head);
 *     the last block is shorter when block does not divide seq_len.
 *   - Every tensor pointer must be 16-byte aligned (QSA_ERR_ALIGN).
 *   - The caller owns all memory.  The library allocates nothing and keeps no
 *     state between calls; calls are re-entrant.  Only qsa_project_residual,
 *     qsa_l1_change, qsa_squad_attention and qsa_select_blocks_work use
 *     scratch memory, which their caller passes in.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream)
 *     and runs asynchronously.  Argument errors are detected on the host
 *     before anything is enqueued; device faults surface at the caller's next
 *     synchronisation.
 *   - Return value: QSA_OK (0) or a negative QSA_ERR_* code; the text of the
 *     last error on the calling thread is available from qsa_last_error_detail.
 *   - There is no fallback path: on a device other than gfx950 every compute
 *     entry point returns QSA_ERR_DEVICE.
 *   - NaN or Inf inputs give undefined (but memory-safe) results.
 */
#ifndef QSA_H_
#define QSA_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QSA_VERSION 10000 /* 1.0.0 */

enum qsa_status {
  QSA_OK = 0,
  QSA_ERR_NULL = -1,   /* a required pointer is NULL */
  QSA_ERR_SHAPE = -2,  /* head_dim or block not in {64,128}, a size < 1, or too large */
  QSA_ERR_PARAM = -3,  /* a scalar argument is out of range */
  QSA_ERR_ALIGN = -4,  /* a tensor pointer is not 16-byte aligned */
  QSA_ERR_DEVICE = -5, /* no usable gfx950 device is current */
  QSA_ERR_LAUNCH = -6  /* the HIP runtime reported an error when enqueuing */
};

/* Problem shape shared by all calls. */
typedef struct qsa_dims {
  int32_t batch;    /* B >= 1 */
  int32_t heads;    /* H >= 1; batch * heads * nb <= QSA_MAX_WORK_BLOCKS */
  int32_t seq_len;  /* L >= 1 */
  int32_t head_dim; /* D: 64 or 128 */
  int32_t block;    /* token block used for quantisation and sparsity: 64 or 128 */
} qsa_dims;

/* Largest number of key blocks qsa_select_blocks supports (nb). */
#define QSA_MAX_BLOCKS 16384
/* Largest batch * heads * nb of any call (QSA_ERR_SHAPE above it): every
   launch's grid, in work-items, then fits the 32-bit dispatch size. */
#define QSA_MAX_WORK_BLOCKS 16777216
/* Largest number of band offsets. */
#define QSA_MAX_BAND 8
/* Largest rank of qsa_project_residual. */
#define QSA_MAX_RANK 64
/* Scratch bytes of qsa_l1_change. */
#define QSA_L1_WORK_BYTES 16384

/*
 * qsa_quantize -- per-block symmetric int8 quantisation of Q or K with pooled
 * code sums (8-bit activations, technical summary §1 and §4; the pooled sums
 * feed the block saliency of qsa_select_blocks, after the average-pooling
 * idea of §2A).
 *
 * For every (b, h, block i) with tokens T_i (n_i valid tokens):
 *   amax      = max |x| over T_i x D (exact, in fp32)
 *   scale[i]  = amax / 127 in IEEE fp32 (round to nearest even); 0 if amax = 0
 *   code[t,d] = clamp(rint(x[t,d] / scale[i]), -127, 127), the quotient an
 *               IEEE fp32 division, rint rounding half to even; 0 if scale is 0
 *   pooled[i,d] = sum over t in T_i of code[t,d]  (|pooled| <= 127 * block)
 *
 *   x      in : bf16 [B,H,L,D]
 *   codes  out: int8 [B,H,L,D]
 *   scales out: fp32 [B,H,nb]
 *   pooled out: int32 [B,H,nb,D]
 */
int qsa_quantize(const qsa_dims* dims, const uint16_t* x, int8_t* codes, float* scales,
                 int32_t* pooled, void* stream);

/*
 * qsa_quantize_rotated -- qsa_quantize of the Hadamard-rotated rows: every
 * token row x (D channels) is first replaced by y = x H_D, H_D the Sylvester
 * Hadamard matrix (entries +-1, H_1 = [1], H_2n = [[H_n, H_n], [H_n, -H_n]]),
 * computed in fp32 by the fast Walsh-Hadamard transform: stages h = 1, 2, 4,
 * ..., D/2, each replacing every pair (j, j+h) of a 2h-aligned group by
 * (v_j + v_{j+h}, v_j - v_{j+h}) with fp32 rounding; codes, scales and pooled
 * sums are then those of qsa_quantize applied to y.  The rotation spreads
 * extreme channels over all channels before quantisation (DVD-Quant,
 * gist.science/es/paper/2505.18663, technical summary §2B, rotated
 * quantisation).  H_D H_D^T = D I: before quantisation every q k^T and every
 * pooled saliency product is scaled by exactly D, so attention on rotated
 * codes uses sm_scale / D, and qsa_select_blocks on rotated pooled sums
 * ranks key blocks as on unrotated ones up to quantisation error (near-equal
 * scores may swap).
 *
 *   arguments, layouts and errors as qsa_quantize.
 */
int qsa_quantize_rotated(const qsa_dims* dims, const uint16_t* x, int8_t* codes, float* scales,
                         int32_t* pooled, void* stream);

/*
 * qsa_select_blocks -- block-sparse attention mask: for every query block i
 * keep its top-k key blocks by pooled saliency plus a fixed band of block
 * offsets (attention sparsification to ~15 % density, technical summary §1
 * and §4; saliency from average-pooled blocks and top-k salient keys after
 * §2A's global and local guidance).
 *
 * For every (b, h, i) and every key block j:
 *   S_ij     = sum_d pooled_q[i,d] * pooled_k[j,d]            (exact integer)
 *   score_ij = fl64( fl64(S_ij * (double)scale_q[i] * (double)scale_k[j])
 *                    / (n_i * n_j) )
 *   top-k(i) = the first min(topk, nb) key blocks ordered by score descending
 *              (IEEE comparison: -0 equals +0), ties to the lower index j
 *   kept(i)  = top-k(i) union { i + o : o in band_offsets, 0 <= i + o < nb }
 *
 *   pooled_q, pooled_k in: int32 [B,H,nb,D]  (from qsa_quantize)
 *   scale_q, scale_k   in: fp32 [B,H,nb]
 *   topk               in: >= 0
 *   band_offsets       in: HOST array of n_band block offsets (may be NULL
 *                          when n_band = 0); 0 <= n_band <= QSA_MAX_BAND
 *   kmax               in: row stride of kept_idx; must be >= min(nb, topk + n_band)
 *   kept_idx          out: int32 [B,H,nb,kmax], ascending, unused slots = -1
 *   kept_cnt          out: int32 [B,H,nb], number of kept blocks of each row
 * QSA_ERR_PARAM if topk < 0, n_band outside [0, QSA_MAX_BAND], kmax too small,
 * or a row could keep nothing (topk = 0 and no band offset 0).
 * QSA_ERR_SHAPE if nb > QSA_MAX_BLOCKS.
 */
int qsa_select_blocks(const qsa_dims* dims, const int32_t* pooled_q, const float* scale_q,
                      const int32_t* pooled_k, const float* scale_k, int32_t topk,
                      const int32_t* band_offsets, int32_t n_band, int32_t kmax,
                      int32_t* kept_idx, int32_t* kept_cnt, void* stream);

/*
 * qsa_select_blocks_work -- qsa_select_blocks through a caller-provided
 * workspace, with the same kept_idx and kept_cnt bit for bit (the mask of
 * technical summary §1, §2A and §4, as above).  The scores of whole (b, h)
 * slices are written to `work` as 64-bit order keys (nb rows of nb keys,
 * padded to a multiple of 16: qsa_select_slice_bytes per slice), then each
 * query block's top-k is selected
 * from them; a pass takes as many slices as work_bytes holds.  That spends
 * device memory and two passes over the keys in HBM on parallelism:
 * qsa_select_blocks keeps the keys of 16 query blocks in LDS, so one
 * workgroup fills a CU.  With work = NULL, work_bytes below one slice, or
 * nb > 2048, it runs as qsa_select_blocks.
 *
 *   work        in: device scratch, 16-byte aligned, or NULL; its contents are
 *                   undefined afterwards.  Calls that share it must not overlap.
 *   work_bytes  in: its size in bytes
 * Errors as qsa_select_blocks; QSA_ERR_ALIGN if work is not 16-byte aligned.
 */
int qsa_select_blocks_work(const qsa_dims* dims, const int32_t* pooled_q, const float* scale_q,
                           const int32_t* pooled_k, const float* scale_k, int32_t topk,
                           const int32_t* band_offsets, int32_t n_band, int32_t kmax,
                           int32_t* kept_idx, int32_t* kept_cnt, void* work,
                           uint64_t work_bytes, void* stream);

/* Bytes of one (b, h) slice of qsa_select_blocks_work's keys:
   nb * ceil(nb / 16) * 16 * 8 (0 for invalid dims). */
uint64_t qsa_select_slice_bytes(const qsa_dims* dims);

/*
 * qsa_sparse_attn -- block-sparse attention on int8 Q/K codes, with the
 * second-order residual correction of sparse steps fused in its epilogue
 * (sparse attention, technical summary §1; residual cache of §2B).
 *
 * For every query token t of block i, over the valid key tokens u of the
 * blocks in kept(i) -- the set of block indices in [0, nb) among the first
 * kept_cnt entries of the row, in any order (a repeated entry counts once,
 * entries outside [0, nb) are skipped):
 *   z_tu = sm_scale * scale_q[i] * scale_k[j(u)] * (q_codes[t] . k_codes[u])
 *   p    = softmax_u(z)   (fp32, online, max-subtracted)
 *   o_t  = sum_u p_tu * v[u]   (P rounded to bf16, fp32 accumulation)
 *   out_t = bf16(o_t + r_t + dr_t)   (r, dr each added only when non-NULL)
 * A row with kept_cnt = 0 has o_t = 0.
 *
 *   q_codes, k_codes in: int8 [B,H,L,D];  q_scales, k_scales in: fp32 [B,H,nb]
 *   v                in: bf16 [B,H,L,D]
 *   kept_idx, kept_cnt in: as written by qsa_select_blocks with row stride kmax
 *   sm_scale         in: finite, > 0 (usually 1/sqrt(D))
 *   r, dr            in: bf16 [B,H,L,D] or NULL
 *   out             out: bf16 [B,H,L,D]; must not alias any input
 * QSA_ERR_SHAPE if nb > QSA_MAX_BLOCKS (both attention entry points).
 */
int qsa_sparse_attn(const qsa_dims* dims, const int8_t* q_codes, const float* q_scales,
                    const int8_t* k_codes, const float* k_scales, const uint16_t* v,
                    const int32_t* kept_idx, const int32_t* kept_cnt, int32_t kmax,
                    float sm_scale, const uint16_t* r, const uint16_t* dr, uint16_t* out,
                    void* stream);

/*
 * qsa_order_query_blocks -- a processing order of the query blocks of every
 * (b, h) for qsa_sparse_attn_ordered and qsa_full_attn_residual_ordered.
 * Sparse attention gathers the key tiles of each query block's kept set
 * (technical summary §1); blocks whose kept sets overlap can share those
 * loads: positions 2k and 2k+1 of the order go to one workgroup, which walks
 * the union of the two kept sets, and neighbouring workgroups run together
 * on one XCD.  The blocks of each (b, h) are cut into chunks of 256
 * consecutive blocks.  Kept sets are compared through 256-bit signatures
 * (bit j mod 256 for key block j).  In each chunk the blocks are paired by
 * rounds of mutual best partners: every single block picks the single block
 * of largest signature overlap (saturated at 255; ties to the lower index)
 * and two blocks that pick each other pair up (blocks still single after 48
 * rounds pair in block order).  The pairs, indexed by their lower block, are
 * then ordered by a greedy chain from pair 0 that always continues with the
 * unused pair whose union signature shares the most bits with the current
 * one (ties to the lower pair index); an odd chunk's single block goes last.
 * Chunks of at most two blocks keep their order; chunks keep their natural
 * order.  Deterministic.
 *
 *   kept_idx, kept_cnt in: as for qsa_sparse_attn (row stride kmax)
 *   order             out: int32 [B,H,nb], a permutation of 0..nb-1 per (b, h)
 */
int qsa_order_query_blocks(const qsa_dims* dims, const int32_t* kept_idx,
                           const int32_t* kept_cnt, int32_t kmax, int32_t* order,
                           void* stream);

/*
 * qsa_sparse_attn_ordered -- qsa_sparse_attn with the query blocks of each
 * (b, h) processed in the given order (a permutation, normally from
 * qsa_order_query_blocks).  Every block is computed from its own kept set
 * with the same arithmetic, so the outputs are bit-identical to
 * qsa_sparse_attn's; only the sharing of key-tile loads changes.
 *
 *   order in: int32 [B,H,nb], a permutation of 0..nb-1 per (b, h).  Entries
 *             outside [0, nb) are skipped; the output rows of a block that
 *             the order does not list are left unwritten.
 *   other arguments as qsa_sparse_attn.
 */
int qsa_sparse_attn_ordered(const qsa_dims* dims, const int8_t* q_codes, const float* q_scales,
                            const int8_t* k_codes, const float* k_scales, const uint16_t* v,
                            const int32_t* kept_idx, const int32_t* kept_cnt, int32_t kmax,
                            const int32_t* order, float sm_scale, const uint16_t* r,
                            const uint16_t* dr, uint16_t* out, void* stream);

/*
 * qsa_full_attn_residual -- refresh step of the second-order sparse attention
 * reparameterisation (technical summary §2B): full attention over ALL key
 * blocks and sparse attention over kept(i), with the numerics of
 * qsa_sparse_attn, computed in one pass over the key blocks; then
 *   rho    = o_full - o_sparse                     (fp32)
 *   dr     = has_prev ? bf16(rho - r_prev) : 0     (second-order residual)
 *   r      = bf16(rho)                             (first-order residual)
 *   out_full = bf16(o_full)
 *
 *   inputs as qsa_sparse_attn;  has_prev in: 0 or 1
 *   r     in/out: bf16 [B,H,L,D]; read (r_prev) only when has_prev = 1
 *   dr       out: bf16 [B,H,L,D]
 *   out_full out: bf16 [B,H,L,D]
 * r, dr and out_full must not alias each other or any input.
 */
int qsa_full_attn_residual(const qsa_dims* dims, const int8_t* q_codes, const float* q_scales,
                           const int8_t* k_codes, const float* k_scales, const uint16_t* v,
                           const int32_t* kept_idx, const int32_t* kept_cnt, int32_t kmax,
                           float sm_scale, int32_t has_prev, uint16_t* r, uint16_t* dr,
                           uint16_t* out_full, void* stream);

/*
 * qsa_full_attn_residual_ordered -- qsa_full_attn_residual with the query
 * blocks of each (b, h) processed in the given order (a permutation,
 * normally from qsa_order_query_blocks).  Every block's two passes (kept
 * blocks, then the others) run over its own tiles in ascending order with the
 * same arithmetic, so r, dr and out_full are bit-identical to
 * qsa_full_attn_residual's; blocks whose kept sets overlap share more tile
 * loads (the workgroup's walks are the unions of its blocks' kept sets and of
 * their complements).
 *
 *   order in: int32 [B,H,nb], a permutation of 0..nb-1 per (b, h).  Entries
 *             outside [0, nb) are skipped; the rows of a block that the order
 *             does not list are left unwritten in r, dr and out_full.
 *   other arguments as qsa_full_attn_residual.
 */
int qsa_full_attn_residual_ordered(const qsa_dims* dims, const int8_t* q_codes,
                                   const float* q_scales, const int8_t* k_codes,
                                   const float* k_scales, const uint16_t* v,
                                   const int32_t* kept_idx, const int32_t* kept_cnt,
                                   int32_t kmax, const int32_t* order, float sm_scale,
                                   int32_t has_prev, uint16_t* r, uint16_t* dr,
                                   uint16_t* out_full, void* stream);

/*
 * qsa_apply_residual -- standalone sparse-step correction (technical summary
 * §2B: cached residuals correct the sparse output at small cost):
 *   out = bf16(sparse_out + r + dr)   elementwise in fp32; dr may be NULL
 *
 *   sparse_out, r, dr in: bf16 [B,H,L,D];  out: bf16 [B,H,L,D]
 * out may alias sparse_out (in place); it must not alias r or dr.
 */
int qsa_apply_residual(const qsa_dims* dims, const uint16_t* sparse_out, const uint16_t* r,
                       const uint16_t* dr, uint16_t* out, void* stream);

/*
 * qsa_project_residual -- rank-r projection of the second-order residual onto
 * its dominant principal components, in place (technical summary §2B: an SVD
 * projects the second-order residual onto its dominant, temporally stable
 * components; Korean summary §2.2: with no storage beyond the residual
 * cache).  Normally called right after a refresh step (qsa_full_attn_residual
 * with has_prev = 1) on its dr output.
 *
 * For every (b, h) slice X = dr[b,h] ([L, D], tokens by channels):
 *   G        = X^T X, bf16 products summed in fp32 over token chunks, the
 *              chunk sums added in a fixed order (deterministic)
 *   V, lam   = eigenvectors and eigenvalues of G by cyclic Jacobi rotations
 *              in fp32, until every off-diagonal entry is <= 2^-22 ||G||_F
 *              (at most 16 sweeps)
 *   V_r      = the eigenvectors of the `rank` largest eigenvalues (ties to the
 *              lower index), orthonormal columns
 *   dr[b,h]  = bf16((X V_r) V_r^T), fp32 arithmetic
 * The result is the best rank-r approximation of X (Eckart-Young); it is
 * unique when the rank-th and next eigenvalues differ.
 *
 *   dr       in/out: bf16 [B,H,L,D]
 *   rank         in: 1 <= rank <= min(D, QSA_MAX_RANK)
 *   basis       out: fp32 [B,H,D,rank], column k = the k-th eigenvector
 *   eigvals     out: fp32 [B,H,rank], descending
 *   work     in/out: device scratch of at least qsa_project_work_bytes(dims, rank)
 *                    bytes; contents undefined on return
 *   work_bytes   in: its size
 * QSA_ERR_PARAM if rank is out of range or work_bytes too small.
 * QSA_ERR_SHAPE if B*H > 65535.  dr, basis, eigvals and work must not overlap.
 */
int qsa_project_residual(const qsa_dims* dims, uint16_t* dr, int32_t rank, float* basis,
                         float* eigvals, void* work, uint64_t work_bytes, void* stream);

/* Bytes of scratch qsa_project_residual needs (0 for invalid dims or rank). */
uint64_t qsa_project_work_bytes(const qsa_dims* dims, int32_t rank);

/*
 * qsa_l1_change -- the two sums of the normalised L1 change between a layer's
 * consecutive outputs, for an adaptive refresh trigger (DVD-Quant,
 * gist.science/es/paper/2505.18663, technical summary §2C: the normalised L1
 * distance between consecutive output features accumulates against a
 * threshold; here it decides when the next step recomputes full attention):
 *   sums[0] = sum |cur - prev|,  sums[1] = sum |prev|
 * over all B*H*L*D elements.  Each term is formed in fp64 from the bf16
 * values and the terms are summed in fp64 in a fixed order (deterministic;
 * within ~2e-13 relative of an exactly rounded sum at 4e8 elements).  The
 * caller forms d = sums[0] / sums[1] and accumulates it.
 *
 *   prev, cur in: bf16 [B,H,L,D]
 *   sums     out: DEVICE fp64 [2]
 *   work  in/out: device scratch of at least QSA_L1_WORK_BYTES bytes
 * QSA_ERR_PARAM if work_bytes < QSA_L1_WORK_BYTES.
 */
int qsa_l1_change(const qsa_dims* dims, const uint16_t* prev, const uint16_t* cur, double* sums,
                  void* work, uint64_t work_bytes, void* stream);

/*
 * qsa_l1_change_noalloc -- qsa_l1_change for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, hosts that
 * forbid allocation): the same sums, with the scratch taken from a fixed
 * QSA_L1_WORK_BYTES array inside the library instead of a `work` argument.
 * That array exists once per GPU the library runs on and lives until the
 * process ends; its device address is looked up on the first call on each
 * device.  The scratch size does not depend on the input size (the partial
 * sums are bounded by QSA_L1_WORK_BYTES / 16 blocks), so every size
 * qsa_l1_change accepts is accepted.  No allocation of any kind.
 *
 *   prev, cur in: bf16 [B,H,L,D]
 *   sums     out: DEVICE fp64 [2]
 * Calls on one GPU share its scratch: calls that may overlap in time (on
 * different streams) race and must be serialised by the caller.  Errors as
 * qsa_l1_change; QSA_ERR_DEVICE if the scratch's address cannot be found on
 * the current device.
 */
int qsa_l1_change_noalloc(const qsa_dims* dims, const uint16_t* prev, const uint16_t* cur,
                          double* sums, void* stream);

/*
 * qsa_window_kept -- kept lists of block-diagonal attention over windows of
 * `window` consecutive tokens (the passes of SQuad attention, SQuad
 * gist.science/es/paper/2608.16585, technical summary, methodology §1):
 * query block i keeps the blocks of its own window, ascending:
 *   kept_idx[b,h,i,j] = (i / per) * per + j  for j < per = window / block,
 *                       -1 for per <= j < kmax;  kept_cnt[b,h,i] = per
 *
 *   window       in: a multiple of dims->block that divides seq_len
 *   kmax         in: row stride of kept_idx, >= window / block
 *   kept_idx    out: int32 [B,H,nb,kmax];  kept_cnt out: int32 [B,H,nb]
 * QSA_ERR_PARAM for a window or kmax out of range.
 */
int qsa_window_kept(const qsa_dims* dims, int32_t window, int32_t kmax, int32_t* kept_idx,
                    int32_t* kept_cnt, void* stream);

/*
 * qsa_reorder_windows -- reorder the rows of every (b, h) sequence of n
 * tokens between window-major order (token p of window k at k*w + p) and
 * position-major order (at p*(n/w) + k), the order of SQuad's global pass:
 *   inverse = 0:  y[p*(n/w) + k] = x[k*w + p]
 *   inverse = 1:  y[k*w + p] = x[p*(n/w) + k]
 *
 *   window   in: w, divides seq_len
 *   x, y     in / out: bf16 [B,H,L,D]; must not overlap
 * QSA_ERR_PARAM for a window that does not divide seq_len.
 */
int qsa_reorder_windows(const qsa_dims* dims, int32_t window, int32_t inverse, const uint16_t* x,
                        uint16_t* y, void* stream);

/*
 * qsa_squad_attention -- SQuad two-pass attention (technical summary,
 * methodology §1) on this path's attention core:
 *   1. local pass: the codes and scales of qsa_quantize(Q) and
 *      qsa_quantize(K) in the natural order, then block-sparse attention (as qsa_sparse_attn) over the windows of
 *      `window` tokens, values V; output O_local, bf16;
 *   2. global pass: Q, K and O_local reordered to position-major order
 *      (qsa_reorder_windows), Q and K quantised in that order, attention over
 *      groups of seq_len / window tokens with values O_local;
 *   3. out = the global output in the natural order.
 * The page sets window = sqrt(seq_len).
 *
 *   q, k, v     in: bf16 [B,H,L,D]
 *   window      in: window and seq_len / window both multiples of dims->block
 *   sm_scale    in: > 0 and finite (normally 1/sqrt(D))
 *   out        out: bf16 [B,H,L,D], must not overlap the inputs
 *   work    in/out: device scratch of qsa_squad_work_bytes(dims, window) bytes
 * QSA_ERR_PARAM for a window out of range, a bad sm_scale or too little work.
 */
int qsa_squad_attention(const qsa_dims* dims, const uint16_t* q, const uint16_t* k,
                        const uint16_t* v, int32_t window, float sm_scale, uint16_t* out,
                        void* work, uint64_t work_bytes, void* stream);

/* Bytes of scratch qsa_squad_attention needs (0 for invalid dims or window). */
uint64_t qsa_squad_work_bytes(const qsa_dims* dims, int32_t window);

/* Static text of a status code. */
const char* qsa_status_string(int status);
/* Text naming the cause of the last error on the calling thread ("" if none). */
const char* qsa_last_error_detail(void);
/* QSA_VERSION of the built library. */
int qsa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* QSA_H_ */
