"""CPU oracle of the QuantSparse attention hot path.  TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously correct NumPy code (fp64 unless a step's definition
fixes fp32).  It defines what the HIP path must compute.  Only the tests, the
smoke check in ``__graft_entry__`` and the benchmark's CPU-baseline leg may
import it; the product path never does.  It shares no code with the HIP path
(only the seeded input generator ``qsa_gen`` serves both).

Sources (gist.science summaries of arXiv 2509.23681, "QuantSparse:
Comprehensively Compressing Video Diffusion Transformer with Model
Quantization and Attention Sparsification"):

* [QS-es] gist.science/es/paper/2509.23681, "Resumen técnico";
* [QS-ko] gist.science/ko/paper/2509.23681, "기술 요약".

The pages describe the method, not its operational detail.  Where they are
silent the readings below are taken (each is also listed with its reason in
the design notes of this repository):

R1  8-bit activations ([QS-es] §1 and §4, W4A8): symmetric int8 codes for Q
    and K with one fp32 scale per (batch, head, token block) over all D.
R2  scale = fl32(amax / 127); code = clamp(rint(fl32(x / scale)), -127, 127)
    with IEEE fp32 division and round-half-to-even; an all-zero block has
    scale 0 and codes 0.
R3  tail blocks (seq_len not a multiple of the block) are shorter blocks:
    statistics over valid tokens only; no padding enters any softmax.
R4  block saliency for the inference mask: the dot product of the
    mean-pooled dequantised Q and K blocks, the pooling idea of MSAD's global
    guidance and the top-k idea of its local guidance ([QS-es] §2A,
    [QS-ko] §2.1) -- score_ij = fl64(fl64(S_ij * (sq_i * sk_j)) / (n_i * n_j))
    with S_ij the exact integer dot of the pooled code sums.
R5  kept(i) = band(i) union top-k(i); the top-k ranks all key blocks by score
    descending, ties to the lowest block index; lists ascending.  kept(i) is
    a set: attention over a given list uses each valid block index of its
    first kept_cnt entries once (repeats and indices outside [0, nb) add
    nothing).
R6  attention is non-causal; logits are sm_scale * sq_i * sk_j * (int dot).
R7  SSAR ([QS-es] §2B, [QS-ko] §2.2): the first-order residual is the
    difference of the attention OUTPUTS of full and sparse attention at a
    refresh step; the second-order residual is the change of that residual
    between consecutive refresh steps (0 at the first refresh); sparse steps
    output sparse + r + dr.  Both residuals are stored in bf16.
R8  SVD projection of the second-order residual ([QS-es] §2B, [QS-ko]
    §2.2: the residual is projected onto its dominant principal components,
    with no storage beyond the residual cache).  When a rank r is given, at
    every refresh step the second-order residual of each (batch, head), a
    [L, D] tokens-by-channels matrix X, is replaced by its best rank-r
    approximation X V_r V_r^T, V_r the r right singular vectors of largest
    singular value (the top-r eigenvectors of X^T X), in the same bf16
    cache.  The pages give no rank; without one nothing is projected.
R9  rotated quantisation (DVD-Quant, gist.science/es/paper/2505.18663,
    technical summary §2B: a Hadamard rotation spreads extreme channels
    before quantisation, with scales computed online): every Q and K row x
    becomes y = x H_D, H_D the unscaled Sylvester Hadamard matrix, computed
    in fp32 by the fast Walsh-Hadamard transform with stages h = 1, 2, ...,
    D/2; y is then quantised by R1/R2 (the per-block scale is the online
    scale).  H_D H_D^T = D I, so attention on rotated codes uses sm_scale/D.
R10 adaptive refresh (DVD-Quant, gist.science/es/paper/2505.18663,
    technical summary §2C: the normalised L1 distance between consecutive
    output features accumulates; once it passes a threshold delta the
    expensive mode is used and the count restarts), read as a refresh
    trigger: after every step t >= 1 of a layer, d_t = sum|O_t - O_{t-1}| /
    sum|O_{t-1}| over all elements of the layer's bf16 attention outputs
    (fp64); c += d_t; if c > delta the next step is a refresh step and c
    restarts at 0.  The first step is a refresh step (no cache yet).  A zero
    denominator gives d = 0 when the outputs agree, else +inf.
R11 SQuad two-pass attention (SQuad, gist.science/es/paper/2608.16585,
    technical summary, methodology §1): a (b, h) sequence of n tokens is cut
    into n/w windows of w consecutive tokens.  The local pass is softmax
    attention of every token over its own window, values V.  The global
    pass is softmax attention of every token over the tokens at the same
    position of every window (t = s mod w), values the local output, stored
    in bf16.  Both passes use the same Q and K and the attention of R1-R6:
    the local pass quantises Q and K in the natural order, the global pass in
    position-major order (token s of window k at index p*(n/w) + k), so that
    each pass's groups are runs of whole 64-token blocks; w and n/w must be
    multiples of the block.  The page sets w = sqrt(n).  The page does not
    say whether the global pass sees the same quantisation; re-quantising per
    pass is the reading that fits a per-block-scale attention core.  The
    other reading, one quantisation shared by both passes, changes only the
    global pass's scales and is not the one taken here.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "bf16_to_f64",
    "f64_to_bf16",
    "default_sm_scale",
    "block_bounds",
    "quantize",
    "fwht",
    "quantize_rotated",
    "project_residual",
    "l1_change",
    "RefreshTrigger",
    "window_kept_lists",
    "to_position_major",
    "from_position_major",
    "squad_attention",
    "block_scores",
    "select_blocks",
    "attention",
    "attention_block_probs",
    "full_kept_lists",
    "ResidualState",
    "refresh_step",
    "sparse_step",
]


# ---------------------------------------------------------------------------
# number formats
# ---------------------------------------------------------------------------

def bf16_to_f64(bits) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to float64; exact."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def _bf16_to_f32(bits) -> np.ndarray:
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32)


def f64_to_bf16(x) -> np.ndarray:
    """Round float64 to the nearest bf16 (ties to even); returns uint16 bits.

    bf16 keeps 8 significant bits; below 2**-126 the spacing is fixed at
    2**-133 (subnormals).  Values beyond the largest finite bf16 after
    rounding become +-inf.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros(x.shape, dtype=np.uint16)
    fin = np.isfinite(x) & (x != 0)
    m, e = np.frexp(np.where(fin, x, 1.0))  # x = m * 2**e, 0.5 <= |m| < 1
    quantum = np.ldexp(1.0, np.maximum(e, -125) - 8)
    y = np.where(fin, np.rint(x / quantum) * quantum, x)  # exact scaling by 2**k
    with np.errstate(over="ignore"):
        y32 = y.astype(np.float32)  # exact: y has <= 8 significant bits
    bits = (y32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    out[...] = bits
    return out


def default_sm_scale(head_dim: int) -> np.float32:
    """Softmax scale 1/sqrt(D) as the fp32 value handed to the kernels."""
    return np.float32(1.0 / np.sqrt(head_dim))


def block_bounds(seq_len: int, block: int):
    """[(start, end)] token ranges of the blocks; the last may be short (R3)."""
    nb = -(-seq_len // block)
    return [(i * block, min((i + 1) * block, seq_len)) for i in range(nb)]


# ---------------------------------------------------------------------------
# step 1: per-block symmetric int8 quantisation and pooled code sums
# ---------------------------------------------------------------------------

def quantize(x_bits, block: int):
    """Quantise one of Q/K, bf16 bits [B, H, L, D] (R1, R2, R3).

    Returns codes int8 [B, H, L, D], scales float32 [B, H, nb] and the pooled
    code sums int64 [B, H, nb, D] (sum of a block's codes per channel).
    """
    return _quantize_values(_bf16_to_f32(x_bits), block)


def fwht(x):
    """Rows of x (float32, last axis D, a power of two) times the Sylvester
    Hadamard matrix H_D, by the fast Walsh-Hadamard transform in float32 (R9).

    Stage h = 1, 2, 4, ..., D/2 replaces every pair (j, j+h) of each
    2h-aligned group by (v_j + v_{j+h}, v_j - v_{j+h}), rounding to float32.
    """
    y = np.array(x, dtype=np.float32, copy=True)
    D = y.shape[-1]
    lead = y.shape[:-1]
    h = 1
    while h < D:
        g = y.reshape(lead + (D // (2 * h), 2, h))
        a = g[..., 0, :].copy()
        b = g[..., 1, :].copy()
        g[..., 0, :] = a + b
        g[..., 1, :] = a - b
        y = g.reshape(lead + (D,))
        h *= 2
    return y


def quantize_rotated(x_bits, block: int):
    """quantize() of the rotated rows fwht(x) of bf16 x [B, H, L, D] (R9)."""
    return _quantize_values(fwht(_bf16_to_f32(x_bits)), block)


def _quantize_values(x, block: int):
    """R1/R2/R3 quantisation of float32 values x [B, H, L, D]."""
    B, H, L, D = x.shape
    bounds = block_bounds(L, block)
    codes = np.zeros((B, H, L, D), dtype=np.int8)
    scales = np.zeros((B, H, len(bounds)), dtype=np.float32)
    pooled = np.zeros((B, H, len(bounds), D), dtype=np.int64)
    f127 = np.float32(127.0)
    for b in range(B):
        for h in range(H):
            for i, (t0, t1) in enumerate(bounds):
                xs = x[b, h, t0:t1]                      # float32 [n_i, D]
                amax = np.max(np.abs(xs))                # exact
                if amax == 0:
                    continue                             # scale 0, codes 0
                s = np.float32(amax / f127)              # IEEE fp32 division
                q = np.rint(xs / s)                      # fp32 division, half-even
                c = np.clip(q, -127, 127).astype(np.int8)
                scales[b, h, i] = s
                codes[b, h, t0:t1] = c
                pooled[b, h, i] = c.astype(np.int64).sum(axis=0)
    return codes, scales, pooled


# ---------------------------------------------------------------------------
# step 2: block saliency and top-k + band selection
# ---------------------------------------------------------------------------

def block_scores(pooled_q, scale_q, pooled_k, scale_k, seq_len: int, block: int):
    """score[b, h, i, j] in float64 (R4).

    S_ij is the exact integer dot product of pooled code sums (an fp64
    matrix product of integer-valued arrays is exact here: every partial sum
    is an integer below 2**53).  a_ij = sq_i * sk_j is exact in fp64.
    """
    n = np.array([t1 - t0 for t0, t1 in block_bounds(seq_len, block)], dtype=np.float64)
    pq = np.asarray(pooled_q, dtype=np.float64)
    pk = np.asarray(pooled_k, dtype=np.float64)
    S = np.einsum("bhid,bhjd->bhij", pq, pk, optimize=True)
    assert np.all(np.abs(S) < 2.0 ** 53)
    a = (np.asarray(scale_q, np.float64)[..., :, None]
         * np.asarray(scale_k, np.float64)[..., None, :])
    b = S * a
    c = n[:, None] * n[None, :]
    return b / c


def select_blocks(scores, topk: int, band, kmax: int, rows=None):
    """kept_idx int32 [B, H, nb, kmax] (ascending, padded with -1), kept_cnt (R5).

    top-k orders all key blocks by score descending (IEEE comparison, so
    -0 equals +0) and then by block index ascending, and keeps the first
    min(topk, nb); band(i) = {i + o : 0 <= i + o < nb}.

    ``rows``: optional query block indices of the rows of ``scores``
    ([B, H, len(rows), nb], a subset of the rows of the full score matrix);
    the results then cover those rows only, in that order.
    """
    B, H, nr, nb = scores.shape
    rows = list(range(nb)) if rows is None else [int(i) for i in rows]
    assert len(rows) == nr
    k = min(int(topk), nb)
    kept_idx = np.full((B, H, nr, kmax), -1, dtype=np.int32)
    kept_cnt = np.zeros((B, H, nr), dtype=np.int32)
    j = np.arange(nb)
    for b in range(B):
        for h in range(H):
            # lexsort: last key is primary -> score descending, then j ascending
            order = np.lexsort((np.broadcast_to(j, (nr, nb)), -scores[b, h]), axis=-1)
            for n, i in enumerate(rows):
                chosen = set(order[n, :k].tolist())
                chosen.update(i + o for o in band if 0 <= i + o < nb)
                lst = sorted(chosen)
                if len(lst) > kmax:
                    raise ValueError("kmax too small for top-k plus band")
                kept_idx[b, h, n, : len(lst)] = lst
                kept_cnt[b, h, n] = len(lst)
    return kept_idx, kept_cnt


def full_kept_lists(B: int, H: int, nb: int):
    """Kept lists that keep every block (dense attention)."""
    idx = np.broadcast_to(np.arange(nb, dtype=np.int32), (B, H, nb, nb)).copy()
    return idx, np.full((B, H, nb), nb, dtype=np.int32)


# ---------------------------------------------------------------------------
# step 3: block-sparse attention on the int8 codes
# ---------------------------------------------------------------------------

def _block_logits(q_codes, q_scales, k_codes, k_scales, b, h, i, blocks, block, seq_len,
                  sm_scale):
    t0, t1 = i * block, min((i + 1) * block, seq_len)
    keys, sk = [], []
    for j in blocks:
        u0, u1 = j * block, min((j + 1) * block, seq_len)
        keys.append(np.arange(u0, u1))
        sk.append(np.full(u1 - u0, k_scales[b, h, j], dtype=np.float64))
    keys = np.concatenate(keys)
    sk = np.concatenate(sk)
    dots = q_codes[b, h, t0:t1].astype(np.float64) @ k_codes[b, h, keys].astype(np.float64).T
    z = (np.float64(sm_scale) * np.float64(q_scales[b, h, i])) * sk[None, :] * dots
    return z, keys


def attention_block_probs(q_codes, q_scales, k_codes, k_scales, b, h, i, blocks, block,
                          seq_len, sm_scale):
    """Softmax probabilities [n_i, n_keys] of query block i over ``blocks``."""
    z, keys = _block_logits(q_codes, q_scales, k_codes, k_scales, b, h, i, blocks, block,
                            seq_len, sm_scale)
    z = z - z.max(axis=1, keepdims=True)
    e = np.exp(z)
    return e / e.sum(axis=1, keepdims=True), keys


def attention(q_codes, q_scales, k_codes, k_scales, v_bits, kept_idx, kept_cnt, block: int,
              sm_scale, which=None):
    """Block-sparse attention output in float64 (R3, R6).

    For each query block i the keys are the valid tokens of the blocks in
    kept(i); logits z = sm_scale * sq_i * sk_j * (q_codes . k_codes); softmax
    in fp64 (max-subtracted); O = P V with V the bf16 values widened to fp64.
    A query block with an empty kept set outputs zeros.

    ``which``: optional iterable of (b, h, i); then only those query blocks
    are computed and a dict {(b, h, i): O_block} is returned.
    """
    B, H, L, D = q_codes.shape
    nb = -(-L // block)
    sel = which if which is not None else [(b, h, i) for b in range(B) for h in range(H)
                                           for i in range(nb)]
    res = {}
    for (b, h, i) in sel:
        t0, t1 = i * block, min((i + 1) * block, L)
        blocks = sorted({int(j) for j in kept_idx[b, h, i, : kept_cnt[b, h, i]]
                         if 0 <= j < nb})  # kept(i) as a set (R5)
        if not blocks:
            res[(b, h, i)] = np.zeros((t1 - t0, D))
            continue
        p, keys = attention_block_probs(q_codes, q_scales, k_codes, k_scales, b, h, i,
                                        blocks, block, L, sm_scale)
        res[(b, h, i)] = p @ bf16_to_f64(v_bits[b, h, keys])
    if which is not None:
        return res
    out = np.zeros((B, H, L, D), dtype=np.float64)
    for (b, h, i), o in res.items():
        out[b, h, i * block: i * block + o.shape[0]] = o
    return out


# ---------------------------------------------------------------------------
# step 4: second-order sparse attention reparameterisation (SSAR)
# ---------------------------------------------------------------------------

class ResidualState:
    """Per-layer residual cache ([QS-es] §2B): r and dr in bf16, has_prev."""

    def __init__(self, shape):
        self.r = np.zeros(shape, dtype=np.uint16)
        self.dr = np.zeros(shape, dtype=np.uint16)
        self.has_prev = False


def project_residual(dr_bits, rank: int):
    """Best rank-``rank`` approximation of every (b, h) slice of the bf16
    second-order residual [B, H, L, D] (R8), in fp64.

    X = dr[b, h] ([L, D]); G = X^T X; V_r = the eigenvectors of G of the
    ``rank`` largest eigenvalues (the right singular vectors of X of largest
    singular value); result X V_r V_r^T.  Returns (projected [B, H, L, D]
    fp64, eigenvalues [B, H, rank] descending).  The projection is unique
    when the rank-th and next eigenvalues differ.
    """
    x = bf16_to_f64(dr_bits)
    B, H, L, D = x.shape
    if not 1 <= rank <= D:
        raise ValueError("rank must be in [1, D]")
    out = np.empty_like(x)
    vals = np.empty((B, H, rank), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            X = x[b, h]
            w, V = np.linalg.eigh(X.T @ X)
            top = np.argsort(-w, kind="stable")[:rank]
            Vr = V[:, top]
            out[b, h] = (X @ Vr) @ Vr.T
            vals[b, h] = w[top]
    return out, vals


def refresh_step(state: ResidualState, o_full, o_sparse, rank: int | None = None):
    """Full-attention refresh step (R7, and R8 when ``rank`` is given).

    rho = O_full - O_sparse (fp64); dr = bf16(rho - r_prev) if a previous
    refresh exists, else 0; with a rank, dr = bf16(rank-r projection of dr);
    r = bf16(rho).  Returns O_full.
    """
    rho = np.asarray(o_full, np.float64) - np.asarray(o_sparse, np.float64)
    if state.has_prev:
        state.dr = f64_to_bf16(rho - bf16_to_f64(state.r))
        if rank is not None:
            state.dr = f64_to_bf16(project_residual(state.dr, rank)[0])
    else:
        state.dr = np.zeros(rho.shape, dtype=np.uint16)
    state.r = f64_to_bf16(rho)
    state.has_prev = True
    return np.asarray(o_full, np.float64)


def sparse_step(state: ResidualState, o_sparse, order: int = 2):
    """Sparse step output (R7): sparse + r + dr (order 2) or sparse + r (order 1)."""
    if not state.has_prev:
        raise RuntimeError("sparse step before any full-attention refresh")
    out = np.asarray(o_sparse, np.float64) + bf16_to_f64(state.r)
    if order == 2:
        out = out + bf16_to_f64(state.dr)
    return out


# ---------------------------------------------------------------------------
# adaptive refresh trigger (R10)
# ---------------------------------------------------------------------------

def l1_change(prev_bits, cur_bits):
    """(sum |cur - prev|, sum |prev|) over all elements of two bf16 tensors, fp64."""
    p = bf16_to_f64(prev_bits)
    c = bf16_to_f64(cur_bits)
    return float(np.abs(c - p).sum()), float(np.abs(p).sum())


class RefreshTrigger:
    """Cumulative normalised-L1 refresh trigger of one layer (R10)."""

    def __init__(self, delta: float):
        self.delta = float(delta)
        self.c = 0.0
        self.refresh_next = True  # the first step fills the residual cache

    def update(self, num: float | None = None, den: float | None = None) -> bool:
        """Account the step just computed, given its (sum|O_t - O_{t-1}|,
        sum|O_{t-1}|), or no sums for the layer's first step (no previous
        output: the next step is sparse).  Returns whether the next step is a
        refresh step."""
        if num is None:
            self.refresh_next = False
            return False
        if den > 0:
            d = num / den
        else:
            d = 0.0 if num == 0 else float("inf")
        self.c += d
        self.refresh_next = self.c > self.delta
        if self.refresh_next:
            self.c = 0.0
        return self.refresh_next


# ---------------------------------------------------------------------------
# SQuad two-pass attention (R11)
# ---------------------------------------------------------------------------

def window_kept_lists(B: int, H: int, seq_len: int, window: int, block: int):
    """Kept lists of block-diagonal attention over windows of ``window``
    tokens: query block i keeps the blocks of its own window, ascending."""
    if window % block or seq_len % window:
        raise ValueError("window must be a multiple of the block and divide seq_len")
    nb = seq_len // block
    per = window // block
    idx = np.empty((B, H, nb, per), dtype=np.int32)
    for i in range(nb):
        idx[:, :, i, :] = (i // per) * per + np.arange(per)
    return idx, np.full((B, H, nb), per, dtype=np.int32)


def to_position_major(x, window: int):
    """[B, H, n, ...] in window-major order (token p of window k at k*w + p) to
    position-major order (at p*(n/w) + k)."""
    B, H, n = x.shape[:3]
    m = n // window
    return np.ascontiguousarray(
        x.reshape((B, H, m, window) + x.shape[3:]).swapaxes(2, 3).reshape(x.shape))


def from_position_major(x, window: int):
    """Inverse of to_position_major."""
    B, H, n = x.shape[:3]
    m = n // window
    return np.ascontiguousarray(
        x.reshape((B, H, window, m) + x.shape[3:]).swapaxes(2, 3).reshape(x.shape))


def squad_attention(q_bits, k_bits, v_bits, window: int, block: int, sm_scale=None):
    """SQuad two-pass attention of bf16 q, k, v [B, H, n, D] (R11), fp64 output.

    Local pass over windows of ``window`` tokens with values v; its output is
    rounded to bf16; global pass over the n/window tokens at each window
    position with those values.
    """
    B, H, n, D = q_bits.shape
    if n % window or window % block or (n // window) % block:
        raise ValueError("window and n/window must be multiples of the block")
    sm = default_sm_scale(D) if sm_scale is None else np.float32(sm_scale)
    qc, sq, _ = quantize(q_bits, block)
    kc, sk, _ = quantize(k_bits, block)
    idx, cnt = window_kept_lists(B, H, n, window, block)
    o_local = f64_to_bf16(attention(qc, sq, kc, sk, v_bits, idx, cnt, block, sm))
    m = n // window
    qc, sq, _ = quantize(to_position_major(q_bits, window), block)
    kc, sk, _ = quantize(to_position_major(k_bits, window), block)
    idx, cnt = window_kept_lists(B, H, n, m, block)
    o = attention(qc, sq, kc, sk, to_position_major(o_local, window), idx, cnt, block, sm)
    return from_position_major(o, window)
