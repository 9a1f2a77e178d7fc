"""ctypes binding of libqsa.so: same names as the C ABI, argument marshalling only.

Every step of the hot path runs in the library's HIP kernels; this module
checks tensor dtypes, shapes and devices, allocates outputs with torch when
the caller passes none, and forwards device pointers plus the current torch
stream.  There is no fallback: without the built library or without a
gfx950 GPU the calls raise.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("QSA_LIB", os.path.join(_HERE, "libqsa.so"))

# status codes of include/qsa.h
QSA_OK = 0
QSA_ERR_NULL = -1
QSA_ERR_SHAPE = -2
QSA_ERR_PARAM = -3
QSA_ERR_ALIGN = -4
QSA_ERR_DEVICE = -5
QSA_ERR_LAUNCH = -6
QSA_MAX_BAND = 8
QSA_MAX_BLOCKS = 16384
QSA_MAX_WORK_BLOCKS = 1 << 24
QSA_MAX_RANK = 64
QSA_L1_WORK_BYTES = 16384

EXPORTED = ("qsa_quantize", "qsa_select_blocks", "qsa_sparse_attn", "qsa_full_attn_residual",
            "qsa_apply_residual", "qsa_order_query_blocks", "qsa_sparse_attn_ordered",
            "qsa_quantize_rotated", "qsa_project_residual", "qsa_project_work_bytes",
            "qsa_l1_change", "qsa_l1_change_noalloc", "qsa_window_kept", "qsa_reorder_windows",
            "qsa_squad_attention",
            "qsa_squad_work_bytes", "qsa_full_attn_residual_ordered",
            "qsa_select_blocks_work", "qsa_select_slice_bytes",
            "qsa_status_string", "qsa_last_error_detail", "qsa_version")


class QSAError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{detail} [{status}]")
        self.status = status
        self.detail = detail


class qsa_dims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("heads", ctypes.c_int32),
                ("seq_len", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("block", ctypes.c_int32)]


_lib = None


def load_library(path: str | None = None) -> ctypes.CDLL:
    """Load libqsa.so (built by ``python -m quantized_sparse_attention_amd.build``)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} not found: build it with "
                           "`python -m quantized_sparse_attention_amd.build`")
    lib = ctypes.CDLL(p)
    vp, i32, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float
    pd = ctypes.POINTER(qsa_dims)
    lib.qsa_quantize.argtypes = [pd, vp, vp, vp, vp, vp]
    lib.qsa_quantize_rotated.argtypes = [pd, vp, vp, vp, vp, vp]
    lib.qsa_select_blocks.argtypes = [pd, vp, vp, vp, vp, i32, vp, i32, i32, vp, vp, vp]
    lib.qsa_select_blocks_work.argtypes = [pd, vp, vp, vp, vp, i32, vp, i32, i32, vp, vp, vp,
                                           ctypes.c_uint64, vp]
    lib.qsa_select_slice_bytes.argtypes = [pd]
    lib.qsa_select_slice_bytes.restype = ctypes.c_uint64
    lib.qsa_sparse_attn.argtypes = [pd, vp, vp, vp, vp, vp, vp, vp, i32, f32, vp, vp, vp, vp]
    lib.qsa_full_attn_residual.argtypes = [pd, vp, vp, vp, vp, vp, vp, vp, i32, f32, i32, vp, vp,
                                           vp, vp]
    lib.qsa_full_attn_residual_ordered.argtypes = [pd, vp, vp, vp, vp, vp, vp, vp, i32, vp, f32,
                                                   i32, vp, vp, vp, vp]
    lib.qsa_apply_residual.argtypes = [pd, vp, vp, vp, vp, vp]
    lib.qsa_order_query_blocks.argtypes = [pd, vp, vp, i32, vp, vp]
    lib.qsa_sparse_attn_ordered.argtypes = [pd, vp, vp, vp, vp, vp, vp, vp, i32, vp, f32, vp, vp,
                                            vp, vp]
    lib.qsa_project_residual.argtypes = [pd, vp, i32, vp, vp, vp, ctypes.c_uint64, vp]
    lib.qsa_l1_change.argtypes = [pd, vp, vp, vp, vp, ctypes.c_uint64, vp]
    lib.qsa_l1_change_noalloc.argtypes = [pd, vp, vp, vp, vp]
    lib.qsa_window_kept.argtypes = [pd, i32, i32, vp, vp, vp]
    lib.qsa_reorder_windows.argtypes = [pd, i32, i32, vp, vp, vp]
    lib.qsa_squad_attention.argtypes = [pd, vp, vp, vp, i32, f32, vp, vp, ctypes.c_uint64, vp]
    lib.qsa_squad_work_bytes.argtypes = [pd, i32]
    lib.qsa_squad_work_bytes.restype = ctypes.c_uint64
    lib.qsa_project_work_bytes.argtypes = [pd, i32]
    lib.qsa_project_work_bytes.restype = ctypes.c_uint64
    for f in ("qsa_quantize", "qsa_quantize_rotated", "qsa_select_blocks",
              "qsa_select_blocks_work", "qsa_sparse_attn",
              "qsa_full_attn_residual", "qsa_apply_residual", "qsa_order_query_blocks",
              "qsa_sparse_attn_ordered", "qsa_project_residual", "qsa_l1_change",
              "qsa_l1_change_noalloc",
              "qsa_window_kept", "qsa_reorder_windows", "qsa_squad_attention",
              "qsa_full_attn_residual_ordered"):
        getattr(lib, f).restype = ctypes.c_int
    lib.qsa_status_string.argtypes = [ctypes.c_int]
    lib.qsa_status_string.restype = ctypes.c_char_p
    lib.qsa_last_error_detail.argtypes = []
    lib.qsa_last_error_detail.restype = ctypes.c_char_p
    lib.qsa_version.argtypes = []
    lib.qsa_version.restype = ctypes.c_int
    if path is None:
        _lib = lib
    return lib


def _check(status: int) -> None:
    if status != QSA_OK:
        lib = load_library()
        raise QSAError(status, lib.qsa_last_error_detail().decode() or
                       lib.qsa_status_string(status).decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _need(t, name, dtype, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t


def n_blocks(seq_len: int, block: int) -> int:
    return -(-seq_len // block)


def make_dims(B: int, H: int, L: int, D: int, block: int) -> qsa_dims:
    return qsa_dims(B, H, L, D, block)


def _quantize(fn, x, block, codes, scales, pooled, stream):
    B, H, L, D = x.shape
    nb = n_blocks(L, block)
    _need(x, "x", torch.bfloat16)
    dev = x.device
    codes = torch.empty((B, H, L, D), dtype=torch.int8, device=dev) if codes is None else codes
    scales = torch.empty((B, H, nb), dtype=torch.float32, device=dev) if scales is None else scales
    pooled = (torch.empty((B, H, nb, D), dtype=torch.int32, device=dev) if pooled is None
              else pooled)
    _need(codes, "codes", torch.int8, (B, H, L, D))
    _need(scales, "scales", torch.float32, (B, H, nb))
    _need(pooled, "pooled", torch.int32, (B, H, nb, D))
    d = make_dims(B, H, L, D, block)
    _check(getattr(load_library(), fn)(ctypes.byref(d), _ptr(x), _ptr(codes), _ptr(scales),
                                       _ptr(pooled), _stream(stream)))
    return codes, scales, pooled


def qsa_quantize(x: torch.Tensor, block: int, codes=None, scales=None, pooled=None, stream=None):
    """int8 codes, fp32 block scales and int32 pooled code sums of bf16 x [B,H,L,D]."""
    return _quantize("qsa_quantize", x, block, codes, scales, pooled, stream)


def qsa_quantize_rotated(x: torch.Tensor, block: int, codes=None, scales=None, pooled=None,
                         stream=None):
    """qsa_quantize of the Hadamard-rotated rows x H_D (attention then uses sm_scale / D)."""
    return _quantize("qsa_quantize_rotated", x, block, codes, scales, pooled, stream)


def qsa_select_blocks(pooled_q, scale_q, pooled_k, scale_k, seq_len: int, block: int, topk: int,
                      band=(0,), kmax: int | None = None, kept_idx=None, kept_cnt=None,
                      stream=None, work=None):
    """Kept key-block lists [B,H,nb,kmax] (ascending, -1 padded) and counts [B,H,nb].
    With ``work`` (a uint8 device tensor) the call is qsa_select_blocks_work,
    which writes the scores' order keys there (same outputs)."""
    B, H, nb, D = pooled_q.shape
    if nb != n_blocks(seq_len, block):
        raise ValueError("pooled_q block count does not match seq_len/block")
    band = [int(o) for o in band]
    if kmax is None:
        kmax = min(nb, topk + len(band))
    dev = pooled_q.device
    _need(pooled_q, "pooled_q", torch.int32)
    _need(pooled_k, "pooled_k", torch.int32, (B, H, nb, D))
    _need(scale_q, "scale_q", torch.float32, (B, H, nb))
    _need(scale_k, "scale_k", torch.float32, (B, H, nb))
    kept_idx = (torch.empty((B, H, nb, kmax), dtype=torch.int32, device=dev) if kept_idx is None
                else kept_idx)
    kept_cnt = (torch.empty((B, H, nb), dtype=torch.int32, device=dev) if kept_cnt is None
                else kept_cnt)
    _need(kept_idx, "kept_idx", torch.int32, (B, H, nb, kmax))
    _need(kept_cnt, "kept_cnt", torch.int32, (B, H, nb))
    arr = (ctypes.c_int32 * max(1, len(band)))(*band) if band else None
    d = make_dims(B, H, seq_len, D, block)
    lib = load_library()
    if work is None:
        _check(lib.qsa_select_blocks(
            ctypes.byref(d), _ptr(pooled_q), _ptr(scale_q), _ptr(pooled_k), _ptr(scale_k),
            int(topk), arr, len(band), int(kmax), _ptr(kept_idx), _ptr(kept_cnt),
            _stream(stream)))
    else:
        _need(work, "work", torch.uint8)
        _check(lib.qsa_select_blocks_work(
            ctypes.byref(d), _ptr(pooled_q), _ptr(scale_q), _ptr(pooled_k), _ptr(scale_k),
            int(topk), arr, len(band), int(kmax), _ptr(kept_idx), _ptr(kept_cnt), _ptr(work),
            ctypes.c_uint64(work.numel()), _stream(stream)))
    return kept_idx, kept_cnt


def qsa_select_slice_bytes(B: int, H: int, L: int, D: int, block: int) -> int:
    """Workspace bytes of one (b, h) slice of qsa_select_blocks_work
    (nb rows of nb keys padded to a multiple of 16, 8 bytes each)."""
    d = make_dims(B, H, L, D, block)
    return int(load_library().qsa_select_slice_bytes(ctypes.byref(d)))


def default_sm_scale(head_dim: int) -> float:
    return float(torch.tensor(1.0 / math.sqrt(head_dim), dtype=torch.float32))


def _attn_checks(q_codes, q_scales, k_codes, k_scales, v, kept_idx, kept_cnt, block):
    B, H, L, D = q_codes.shape
    nb = n_blocks(L, block)
    _need(q_codes, "q_codes", torch.int8)
    _need(k_codes, "k_codes", torch.int8, (B, H, L, D))
    _need(q_scales, "q_scales", torch.float32, (B, H, nb))
    _need(k_scales, "k_scales", torch.float32, (B, H, nb))
    _need(v, "v", torch.bfloat16, (B, H, L, D))
    _need(kept_idx, "kept_idx", torch.int32)
    if kept_idx.dim() != 4 or tuple(kept_idx.shape[:3]) != (B, H, nb):
        raise ValueError(f"kept_idx must be [B,H,nb,kmax] with nb={nb}")
    _need(kept_cnt, "kept_cnt", torch.int32, (B, H, nb))
    return B, H, L, D, kept_idx.shape[3]


def qsa_sparse_attn(q_codes, q_scales, k_codes, k_scales, v, kept_idx, kept_cnt, block: int,
                    sm_scale: float | None = None, r=None, dr=None, out=None, stream=None):
    """bf16 block-sparse attention output, plus r and dr when given."""
    B, H, L, D, kmax = _attn_checks(q_codes, q_scales, k_codes, k_scales, v, kept_idx, kept_cnt,
                                    block)
    if r is not None:
        _need(r, "r", torch.bfloat16, (B, H, L, D))
    if dr is not None:
        _need(dr, "dr", torch.bfloat16, (B, H, L, D))
    out = torch.empty_like(v) if out is None else out
    _need(out, "out", torch.bfloat16, (B, H, L, D))
    sm = default_sm_scale(D) if sm_scale is None else float(sm_scale)
    d = make_dims(B, H, L, D, block)
    _check(load_library().qsa_sparse_attn(
        ctypes.byref(d), _ptr(q_codes), _ptr(q_scales), _ptr(k_codes), _ptr(k_scales), _ptr(v),
        _ptr(kept_idx), _ptr(kept_cnt), int(kmax), ctypes.c_float(sm), _ptr(r), _ptr(dr),
        _ptr(out), _stream(stream)))
    return out


def qsa_order_query_blocks(kept_idx, kept_cnt, seq_len: int, block: int, head_dim: int,
                           order=None, stream=None):
    """int32 [B,H,nb] processing order grouping query blocks with overlapping kept sets."""
    _need(kept_idx, "kept_idx", torch.int32)
    if kept_idx.dim() != 4:
        raise ValueError("kept_idx must be [B,H,nb,kmax]")
    B, H, nb, kmax = kept_idx.shape
    if nb != n_blocks(seq_len, block):
        raise ValueError(f"kept_idx has {nb} rows, seq_len/block gives {n_blocks(seq_len, block)}")
    _need(kept_cnt, "kept_cnt", torch.int32, (B, H, nb))
    order = (torch.empty((B, H, nb), dtype=torch.int32, device=kept_idx.device) if order is None
             else order)
    _need(order, "order", torch.int32, (B, H, nb))
    d = make_dims(B, H, seq_len, head_dim, block)
    _check(load_library().qsa_order_query_blocks(ctypes.byref(d), _ptr(kept_idx), _ptr(kept_cnt),
                                                 int(kmax), _ptr(order), _stream(stream)))
    return order


def qsa_sparse_attn_ordered(q_codes, q_scales, k_codes, k_scales, v, kept_idx, kept_cnt, order,
                            block: int, sm_scale: float | None = None, r=None, dr=None, out=None,
                            stream=None):
    """qsa_sparse_attn with the query blocks processed in ``order`` (same outputs)."""
    B, H, L, D, kmax = _attn_checks(q_codes, q_scales, k_codes, k_scales, v, kept_idx, kept_cnt,
                                    block)
    _need(order, "order", torch.int32, (B, H, n_blocks(L, block)))
    if r is not None:
        _need(r, "r", torch.bfloat16, (B, H, L, D))
    if dr is not None:
        _need(dr, "dr", torch.bfloat16, (B, H, L, D))
    out = torch.empty_like(v) if out is None else out
    _need(out, "out", torch.bfloat16, (B, H, L, D))
    sm = default_sm_scale(D) if sm_scale is None else float(sm_scale)
    d = make_dims(B, H, L, D, block)
    _check(load_library().qsa_sparse_attn_ordered(
        ctypes.byref(d), _ptr(q_codes), _ptr(q_scales), _ptr(k_codes), _ptr(k_scales), _ptr(v),
        _ptr(kept_idx), _ptr(kept_cnt), int(kmax), _ptr(order), ctypes.c_float(sm), _ptr(r),
        _ptr(dr), _ptr(out), _stream(stream)))
    return out


def qsa_full_attn_residual(q_codes, q_scales, k_codes, k_scales, v, kept_idx, kept_cnt,
                           block: int, r, dr, has_prev: bool, sm_scale: float | None = None,
                           out_full=None, stream=None, order=None):
    """Refresh step: full attention output; r (in/out) and dr (out) updated in place.
    With ``order`` (int32 [B,H,nb], e.g. from qsa_order_query_blocks) the query
    blocks are processed in that order (qsa_full_attn_residual_ordered)."""
    B, H, L, D, kmax = _attn_checks(q_codes, q_scales, k_codes, k_scales, v, kept_idx, kept_cnt,
                                    block)
    _need(r, "r", torch.bfloat16, (B, H, L, D))
    _need(dr, "dr", torch.bfloat16, (B, H, L, D))
    out_full = torch.empty_like(v) if out_full is None else out_full
    _need(out_full, "out_full", torch.bfloat16, (B, H, L, D))
    sm = default_sm_scale(D) if sm_scale is None else float(sm_scale)
    d = make_dims(B, H, L, D, block)
    lib = load_library()
    if order is None:
        _check(lib.qsa_full_attn_residual(
            ctypes.byref(d), _ptr(q_codes), _ptr(q_scales), _ptr(k_codes), _ptr(k_scales),
            _ptr(v), _ptr(kept_idx), _ptr(kept_cnt), int(kmax), ctypes.c_float(sm),
            int(bool(has_prev)), _ptr(r), _ptr(dr), _ptr(out_full), _stream(stream)))
    else:
        _need(order, "order", torch.int32, (B, H, kept_cnt.shape[-1]))
        _check(lib.qsa_full_attn_residual_ordered(
            ctypes.byref(d), _ptr(q_codes), _ptr(q_scales), _ptr(k_codes), _ptr(k_scales),
            _ptr(v), _ptr(kept_idx), _ptr(kept_cnt), int(kmax), _ptr(order), ctypes.c_float(sm),
            int(bool(has_prev)), _ptr(r), _ptr(dr), _ptr(out_full), _stream(stream)))
    return out_full


def qsa_apply_residual(sparse_out, r, dr=None, out=None, block: int = 64, stream=None):
    """out = bf16(sparse_out + r + dr) elementwise (out may be sparse_out)."""
    B, H, L, D = sparse_out.shape
    _need(sparse_out, "sparse_out", torch.bfloat16)
    _need(r, "r", torch.bfloat16, (B, H, L, D))
    if dr is not None:
        _need(dr, "dr", torch.bfloat16, (B, H, L, D))
    out = torch.empty_like(sparse_out) if out is None else out
    _need(out, "out", torch.bfloat16, (B, H, L, D))
    d = make_dims(B, H, L, D, block)
    _check(load_library().qsa_apply_residual(ctypes.byref(d), _ptr(sparse_out), _ptr(r), _ptr(dr),
                                             _ptr(out), _stream(stream)))
    return out


def qsa_project_work_bytes(B: int, H: int, L: int, D: int, rank: int) -> int:
    """Scratch bytes qsa_project_residual needs (0 for invalid sizes)."""
    d = make_dims(B, H, L, D, 64)
    return int(load_library().qsa_project_work_bytes(ctypes.byref(d), int(rank)))


def qsa_project_residual(dr: torch.Tensor, rank: int, basis=None, eigvals=None, work=None,
                         stream=None):
    """Rank-``rank`` projection of the bf16 second-order residual dr [B,H,L,D]
    onto its dominant principal components, in place.  Returns (basis fp32
    [B,H,D,rank], eigvals fp32 [B,H,rank] descending)."""
    _need(dr, "dr", torch.bfloat16)
    B, H, L, D = dr.shape
    dev = dr.device
    basis = (torch.empty((B, H, D, rank), dtype=torch.float32, device=dev) if basis is None
             else basis)
    eigvals = (torch.empty((B, H, rank), dtype=torch.float32, device=dev) if eigvals is None
               else eigvals)
    _need(basis, "basis", torch.float32, (B, H, D, rank))
    _need(eigvals, "eigvals", torch.float32, (B, H, rank))
    need = qsa_project_work_bytes(B, H, L, D, rank)
    if work is None:
        work = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    _need(work, "work", torch.uint8)
    d = make_dims(B, H, L, D, 64)
    _check(load_library().qsa_project_residual(ctypes.byref(d), _ptr(dr), int(rank), _ptr(basis),
                                               _ptr(eigvals), _ptr(work),
                                               ctypes.c_uint64(work.numel()), _stream(stream)))
    return basis, eigvals


def qsa_l1_change(prev: torch.Tensor, cur: torch.Tensor, sums=None, work=None, stream=None):
    """Device fp64 [2]: (sum |cur - prev|, sum |prev|) of two bf16 [B,H,L,D] tensors."""
    _need(prev, "prev", torch.bfloat16)
    _need(cur, "cur", torch.bfloat16, tuple(prev.shape))
    Bn, H, L, D = prev.shape
    dev = prev.device
    sums = torch.empty(2, dtype=torch.float64, device=dev) if sums is None else sums
    work = torch.empty(QSA_L1_WORK_BYTES, dtype=torch.uint8, device=dev) if work is None else work
    _need(sums, "sums", torch.float64, (2,))
    _need(work, "work", torch.uint8)
    d = make_dims(Bn, H, L, D, 64)
    _check(load_library().qsa_l1_change(ctypes.byref(d), _ptr(prev), _ptr(cur), _ptr(sums),
                                        _ptr(work), ctypes.c_uint64(work.numel()),
                                        _stream(stream)))
    return sums


def qsa_l1_change_noalloc(prev: torch.Tensor, cur: torch.Tensor, sums: torch.Tensor,
                          stream=None):
    """qsa_l1_change with the library's own fixed scratch: the call allocates
    nothing (``sums``, device fp64 [2], is the caller's)."""
    _need(prev, "prev", torch.bfloat16)
    _need(cur, "cur", torch.bfloat16, tuple(prev.shape))
    _need(sums, "sums", torch.float64, (2,))
    Bn, H, L, D = prev.shape
    d = make_dims(Bn, H, L, D, 64)
    _check(load_library().qsa_l1_change_noalloc(ctypes.byref(d), _ptr(prev), _ptr(cur),
                                                _ptr(sums), _stream(stream)))
    return sums


def qsa_window_kept(B: int, H: int, L: int, block: int, window: int, kmax=None, kept_idx=None,
                    kept_cnt=None, device="cuda", stream=None):
    """Kept lists of block-diagonal attention over windows of ``window`` tokens."""
    nb = n_blocks(L, block)
    kmax = window // block if kmax is None else kmax
    kept_idx = (torch.empty((B, H, nb, kmax), dtype=torch.int32, device=device)
                if kept_idx is None else kept_idx)
    kept_cnt = (torch.empty((B, H, nb), dtype=torch.int32, device=device)
                if kept_cnt is None else kept_cnt)
    _need(kept_idx, "kept_idx", torch.int32, (B, H, nb, kmax))
    _need(kept_cnt, "kept_cnt", torch.int32, (B, H, nb))
    d = make_dims(B, H, L, 64, block)
    _check(load_library().qsa_window_kept(ctypes.byref(d), int(window), int(kmax),
                                          _ptr(kept_idx), _ptr(kept_cnt), _stream(stream)))
    return kept_idx, kept_cnt


def qsa_reorder_windows(x: torch.Tensor, window: int, inverse: bool = False, out=None,
                        stream=None):
    """Rows of bf16 x [B,H,L,D] from window-major to position-major order
    (or back with ``inverse``)."""
    _need(x, "x", torch.bfloat16)
    B, H, L, D = x.shape
    out = torch.empty_like(x) if out is None else out
    _need(out, "out", torch.bfloat16, (B, H, L, D))
    d = make_dims(B, H, L, D, 64)
    _check(load_library().qsa_reorder_windows(ctypes.byref(d), int(window), int(bool(inverse)),
                                              _ptr(x), _ptr(out), _stream(stream)))
    return out


def qsa_squad_work_bytes(B: int, H: int, L: int, D: int, block: int, window: int) -> int:
    d = make_dims(B, H, L, D, block)
    return int(load_library().qsa_squad_work_bytes(ctypes.byref(d), int(window)))


def qsa_squad_attention(q, k, v, window: int, block: int = 64, sm_scale: float | None = None,
                        out=None, work=None, stream=None):
    """SQuad two-pass attention of bf16 q, k, v [B,H,L,D]: local windows of
    ``window`` tokens, then same-position groups with the local output as
    values."""
    for t, name in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, name, torch.bfloat16, tuple(q.shape))
    B, H, L, D = q.shape
    out = torch.empty_like(q) if out is None else out
    _need(out, "out", torch.bfloat16, (B, H, L, D))
    need = qsa_squad_work_bytes(B, H, L, D, block, window)
    if work is None:
        work = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _need(work, "work", torch.uint8)
    sm = default_sm_scale(D) if sm_scale is None else float(sm_scale)
    d = make_dims(B, H, L, D, block)
    _check(load_library().qsa_squad_attention(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v),
                                              int(window), ctypes.c_float(sm), _ptr(out),
                                              _ptr(work), ctypes.c_uint64(work.numel()),
                                              _stream(stream)))
    return out
