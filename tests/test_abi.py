"""The C ABI library loads, exports every declared symbol, and validates its
arguments on the host (exact status codes, nothing launched).  Runs without a
GPU: fake device pointers are only ever passed where validation must reject
them first, and the checks that rely on "no device present" skip on a GPU machine.
"""
import ctypes
import os
import re
import subprocess

import pytest

from quantized_sparse_attention_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qsa.h")


def _gpu_present() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


NO_GPU = not _gpu_present()
needs_no_gpu = pytest.mark.skipif(not NO_GPU, reason="uses fake device pointers")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        pytest.skip("libqsa.so not built")
    return B.load_library()


def _declared():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(qsa_[a-z0-9_]+)\s*\(", txt)))


def test_header_declares_the_entry_points():
    names = _declared()
    for n in ("qsa_quantize", "qsa_select_blocks", "qsa_sparse_attn", "qsa_full_attn_residual",
              "qsa_apply_residual", "qsa_status_string", "qsa_last_error_detail", "qsa_version"):
        assert n in names
    assert set(names) == set(B.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (qsa_\w+)", out))
    for n in _declared():
        assert n in exported, n
        assert hasattr(lib, n)


def test_version_and_status_strings(lib):
    assert lib.qsa_version() == 10000
    for st in (0, -1, -2, -3, -4, -5, -6):
        assert lib.qsa_status_string(st)
    assert b"unknown" in lib.qsa_status_string(-99)


def _d(B_=1, H=2, L=128, D=64, bs=64):
    return ctypes.byref(B.qsa_dims(B_, H, L, D, bs))


P = [ctypes.c_void_p(0x1000 * (i + 1)) for i in range(12)]  # aligned, never dereferenced


def _q(lib, dims, ptrs=None):
    p = ptrs or P[:4]
    return lib.qsa_quantize(dims, *p, None)


def test_quantize_validation(lib):
    assert lib.qsa_quantize(None, *P[:4], None) == B.QSA_ERR_NULL
    assert _q(lib, _d(D=96)) == B.QSA_ERR_SHAPE
    assert _q(lib, _d(bs=32)) == B.QSA_ERR_SHAPE
    assert _q(lib, _d(B_=0)) == B.QSA_ERR_SHAPE
    assert _q(lib, _d(L=0)) == B.QSA_ERR_SHAPE
    assert _q(lib, _d(H=-1)) == B.QSA_ERR_SHAPE
    assert _q(lib, _d(), [None] + P[1:4]) == B.QSA_ERR_NULL
    assert b"x is NULL" in lib.qsa_last_error_detail()
    assert _q(lib, _d(), P[:3] + [None]) == B.QSA_ERR_NULL
    assert _q(lib, _d(), [ctypes.c_void_p(0x1008)] + P[1:4]) == B.QSA_ERR_ALIGN
    assert _q(lib, _d(B_=1 << 20, H=1 << 10, L=1 << 12, bs=64)) == B.QSA_ERR_SHAPE
    # batch * heads * blocks above QSA_MAX_WORK_BLOCKS (grids beyond 32-bit work-item counts)
    assert _q(lib, _d(B_=256, H=1 << 10, L=64 * 64 + 1)) == B.QSA_ERR_SHAPE
    assert b"QSA_MAX_WORK_BLOCKS" in lib.qsa_last_error_detail()


def test_work_limit_matches_the_header():
    txt = open(HEADER).read()
    assert re.search(r"#define QSA_MAX_WORK_BLOCKS (\d+)", txt).group(1) == str(B.QSA_MAX_WORK_BLOCKS)
    assert B.QSA_MAX_WORK_BLOCKS == 1 << 24


@needs_no_gpu
def test_valid_arguments_reach_the_device_check(lib):
    assert _q(lib, _d()) == B.QSA_ERR_DEVICE
    assert _q(lib, _d(B_=256, H=1 << 10, L=64 * 64)) == B.QSA_ERR_DEVICE  # at QSA_MAX_WORK_BLOCKS
    band = (ctypes.c_int32 * 1)(0)
    assert lib.qsa_select_blocks(_d(), *P[:4], 1, band, 1, 2, P[4], P[5], None) == B.QSA_ERR_DEVICE
    assert lib.qsa_sparse_attn(_d(), *P[:7], 2, ctypes.c_float(0.125), None, None, P[7],
                               None) == B.QSA_ERR_DEVICE
    assert lib.qsa_full_attn_residual(_d(), *P[:7], 2, ctypes.c_float(0.125), 1, P[7], P[8], P[9],
                                      None) == B.QSA_ERR_DEVICE
    assert lib.qsa_apply_residual(_d(), P[0], P[1], None, P[0], None) == B.QSA_ERR_DEVICE
    assert lib.qsa_order_query_blocks(_d(), P[0], P[1], 2, P[2], None) == B.QSA_ERR_DEVICE
    assert lib.qsa_sparse_attn_ordered(_d(), *P[:7], 2, P[8], ctypes.c_float(0.125), None, None,
                                       P[7], None) == B.QSA_ERR_DEVICE
    assert lib.qsa_full_attn_residual_ordered(_d(), *P[:7], 2, P[10], ctypes.c_float(0.125), 1,
                                              P[7], P[8], P[9], None) == B.QSA_ERR_DEVICE


def _sel(lib, topk=1, band=(0,), n_band=None, kmax=2, dims=None, ptrs=None):
    arr = (ctypes.c_int32 * max(1, len(band)))(*band) if band is not None else None
    nb_ = len(band) if n_band is None and band is not None else (n_band or 0)
    p = ptrs or P[:6]
    return lib.qsa_select_blocks(dims or _d(), p[0], p[1], p[2], p[3], topk, arr, nb_, kmax, p[4],
                                 p[5], None)


def test_select_validation(lib):
    assert _sel(lib, topk=-1) == B.QSA_ERR_PARAM
    assert _sel(lib, band=tuple(range(9))) == B.QSA_ERR_PARAM
    assert _sel(lib, band=None, n_band=2) == B.QSA_ERR_NULL
    assert _sel(lib, topk=0, band=(1,)) == B.QSA_ERR_PARAM           # a row could keep nothing
    assert _sel(lib, topk=2, band=(0,), kmax=1) == B.QSA_ERR_PARAM    # kmax < min(nb, k+band)
    assert _sel(lib, topk=1, kmax=0) == B.QSA_ERR_PARAM
    assert _sel(lib, ptrs=[P[0], None] + P[2:6]) == B.QSA_ERR_NULL
    assert _sel(lib, ptrs=P[:5] + [ctypes.c_void_p(0x2004)]) == B.QSA_ERR_ALIGN
    big = _d(L=64 * (B.QSA_MAX_BLOCKS + 1))
    assert _sel(lib, dims=big, kmax=2) == B.QSA_ERR_SHAPE


def test_attention_validation(lib):
    f = ctypes.c_float

    def sp(sm=0.125, kmax=2, ptrs=None, out=P[7]):
        p = ptrs or P[:7]
        return lib.qsa_sparse_attn(_d(), *p, kmax, f(sm), None, None, out, None)

    assert sp(sm=0.0) == B.QSA_ERR_PARAM
    assert sp(sm=-1.0) == B.QSA_ERR_PARAM
    assert sp(sm=float("nan")) == B.QSA_ERR_PARAM
    assert sp(sm=float("inf")) == B.QSA_ERR_PARAM
    assert sp(kmax=0) == B.QSA_ERR_PARAM
    assert sp(out=None) == B.QSA_ERR_NULL
    assert sp(ptrs=P[:6] + [None]) == B.QSA_ERR_NULL
    assert lib.qsa_sparse_attn(_d(), *P[:7], 2, f(0.1), ctypes.c_void_p(0x3002), None, P[7],
                               None) == B.QSA_ERR_ALIGN
    assert lib.qsa_full_attn_residual(_d(), *P[:7], 2, f(0.1), 2, P[7], P[8], P[9],
                                      None) == B.QSA_ERR_PARAM
    assert lib.qsa_full_attn_residual(_d(), *P[:7], 2, f(0.1), 0, None, P[8], P[9],
                                      None) == B.QSA_ERR_NULL
    assert lib.qsa_apply_residual(_d(), P[0], None, None, P[0], None) == B.QSA_ERR_NULL
    assert lib.qsa_apply_residual(_d(D=80), P[0], P[1], None, P[0], None) == B.QSA_ERR_SHAPE
    assert lib.qsa_sparse_attn_ordered(_d(), *P[:7], 2, None, f(0.1), None, None, P[7],
                                       None) == B.QSA_ERR_NULL
    assert lib.qsa_sparse_attn_ordered(_d(), *P[:7], 2, P[8], f(0.0), None, None, P[7],
                                       None) == B.QSA_ERR_PARAM
    assert lib.qsa_full_attn_residual_ordered(_d(), *P[:7], 2, None, f(0.1), 0, P[7], P[8],
                                              P[9], None) == B.QSA_ERR_NULL
    assert lib.qsa_full_attn_residual_ordered(_d(), *P[:7], 2, ctypes.c_void_p(0x3004), f(0.1),
                                              0, P[7], P[8], P[9], None) == B.QSA_ERR_ALIGN
    assert lib.qsa_full_attn_residual_ordered(_d(), *P[:7], 2, P[10], f(0.1), 2, P[7], P[8],
                                              P[9], None) == B.QSA_ERR_PARAM
    assert lib.qsa_full_attn_residual_ordered(_d(), *P[:7], 2, P[10], f(0.1), 0, None, P[8],
                                              P[9], None) == B.QSA_ERR_NULL
    assert lib.qsa_order_query_blocks(_d(), P[0], P[1], 0, P[2], None) == B.QSA_ERR_PARAM
    assert lib.qsa_order_query_blocks(_d(), P[0], None, 2, P[2], None) == B.QSA_ERR_NULL
    assert lib.qsa_order_query_blocks(_d(), P[0], P[1], 2, ctypes.c_void_p(0x3004),
                                      None) == B.QSA_ERR_ALIGN
    big = _d(L=64 * (B.QSA_MAX_BLOCKS + 1))
    assert lib.qsa_order_query_blocks(big, P[0], P[1], 2, P[2], None) == B.QSA_ERR_SHAPE
    assert lib.qsa_sparse_attn(big, *P[:7], 2, f(0.1), None, None, P[7], None) == B.QSA_ERR_SHAPE


def test_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros((1, 1, 64, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        B.qsa_quantize(x, 64)
    with pytest.raises(TypeError):
        B.qsa_quantize(x.float(), 64)


def test_project_residual_validation(lib):
    u64 = ctypes.c_uint64
    need = lib.qsa_project_work_bytes(_d(L=1000, D=128), 32)
    # partial Gram matrices (2 heads x 1 chunk of 1000 tokens x 128 x 128) + padded basis
    assert need == 4 * (2 * 1 * 128 * 128 + 2 * 128 * B.QSA_MAX_RANK)
    assert lib.qsa_project_work_bytes(_d(D=64), 65) == 0
    assert lib.qsa_project_work_bytes(_d(D=64), 0) == 0
    assert lib.qsa_project_work_bytes(None, 4) == 0

    def pr(rank=8, dims=None, ptrs=None, wb=None):
        p = ptrs or P[:4]
        dd = dims or _d()
        w = lib.qsa_project_work_bytes(dd, max(1, min(rank, 64))) if wb is None else wb
        return lib.qsa_project_residual(dd, p[0], rank, p[1], p[2], p[3], u64(w), None)

    assert pr(rank=0) == B.QSA_ERR_PARAM
    assert pr(rank=65, dims=_d(D=128)) == B.QSA_ERR_PARAM
    assert pr(rank=65, dims=_d(D=64)) == B.QSA_ERR_PARAM
    assert pr(wb=16) == B.QSA_ERR_PARAM
    assert b"work_bytes" in lib.qsa_last_error_detail()
    assert pr(ptrs=[None] + P[1:4]) == B.QSA_ERR_NULL
    assert pr(ptrs=P[:3] + [None]) == B.QSA_ERR_NULL
    assert pr(ptrs=P[:1] + [ctypes.c_void_p(0x1004)] + P[2:4]) == B.QSA_ERR_ALIGN
    assert pr(dims=_d(B_=300, H=300)) == B.QSA_ERR_SHAPE
    assert pr(dims=_d(D=96)) == B.QSA_ERR_SHAPE
    if NO_GPU:
        assert pr() == B.QSA_ERR_DEVICE


def test_l1_change_validation(lib):
    u64 = ctypes.c_uint64

    def l1(dims=None, ptrs=None, wb=B.QSA_L1_WORK_BYTES):
        p = ptrs or P[:4]
        return lib.qsa_l1_change(dims or _d(), p[0], p[1], p[2], p[3], u64(wb), None)

    assert l1(wb=B.QSA_L1_WORK_BYTES - 1) == B.QSA_ERR_PARAM
    assert l1(ptrs=[None] + P[1:4]) == B.QSA_ERR_NULL
    assert l1(ptrs=P[:2] + [None, P[3]]) == B.QSA_ERR_NULL
    assert l1(ptrs=P[:2] + [ctypes.c_void_p(0x3008), P[3]]) == B.QSA_ERR_ALIGN
    assert l1(dims=_d(D=32)) == B.QSA_ERR_SHAPE
    if NO_GPU:
        assert l1() == B.QSA_ERR_DEVICE


def test_l1_change_noalloc_validation(lib):
    def l1(dims=None, ptrs=None):
        p = ptrs or P[:3]
        return lib.qsa_l1_change_noalloc(dims or _d(), p[0], p[1], p[2], None)

    assert l1(ptrs=[None] + P[1:3]) == B.QSA_ERR_NULL
    assert l1(ptrs=P[:2] + [None]) == B.QSA_ERR_NULL
    assert l1(ptrs=P[:2] + [ctypes.c_void_p(0x3008)]) == B.QSA_ERR_ALIGN
    assert l1(dims=_d(D=32)) == B.QSA_ERR_SHAPE
    if NO_GPU:
        assert l1() == B.QSA_ERR_DEVICE


def test_squad_validation(lib):
    u64, f = ctypes.c_uint64, ctypes.c_float
    d = _d(L=4096, D=64)
    need = lib.qsa_squad_work_bytes(d, 64)
    assert need > 0
    assert lib.qsa_squad_work_bytes(d, 96) == 0       # not a multiple of the block
    assert lib.qsa_squad_work_bytes(d, 2048) == 0     # n / w = 2 is not
    assert lib.qsa_squad_work_bytes(_d(L=4100, D=64), 64) == 0

    def sq(window=64, sm=0.125, wb=None, ptrs=None):
        p = ptrs or P[:5]
        return lib.qsa_squad_attention(d, p[0], p[1], p[2], window, f(sm), p[3], p[4],
                                       u64(need if wb is None else wb), None)

    assert sq(window=96) == B.QSA_ERR_PARAM
    assert sq(sm=0.0) == B.QSA_ERR_PARAM
    assert sq(sm=float("inf")) == B.QSA_ERR_PARAM
    assert sq(wb=need - 1) == B.QSA_ERR_PARAM
    assert sq(ptrs=[None] + P[1:5]) == B.QSA_ERR_NULL
    assert sq(ptrs=P[:4] + [ctypes.c_void_p(0x1002)]) == B.QSA_ERR_ALIGN
    assert lib.qsa_window_kept(d, 96, 4, P[0], P[1], None) == B.QSA_ERR_PARAM
    assert lib.qsa_window_kept(d, 128, 1, P[0], P[1], None) == B.QSA_ERR_PARAM
    assert lib.qsa_reorder_windows(d, 100, 0, P[0], P[1], None) == B.QSA_ERR_PARAM
    assert lib.qsa_reorder_windows(d, 64, 2, P[0], P[1], None) == B.QSA_ERR_PARAM
    if NO_GPU:
        assert sq() == B.QSA_ERR_DEVICE
        assert lib.qsa_window_kept(d, 128, 2, P[0], P[1], None) == B.QSA_ERR_DEVICE
        assert lib.qsa_reorder_windows(d, 64, 1, P[0], P[1], None) == B.QSA_ERR_DEVICE


PROBE_LIB = os.path.join(ROOT, "quantized_sparse_attention_amd", "libqsa_probe.so")


def test_probe_library_is_separate_and_checks_its_arguments():
    """The benchmark's MFMA-rate probe lives in libqsa_probe.so, not in the
    attention library, and rejects bad arguments before any launch."""
    if not os.path.exists(PROBE_LIB):
        pytest.skip("libqsa_probe.so not built")
    out = subprocess.run(["nm", "-D", "--defined-only", PROBE_LIB], capture_output=True,
                         text=True, check=True).stdout
    assert set(re.findall(r"\bT (qsa_\w+)", out)) == {"qsa_probe_mfma", "qsa_probe_mfma_ops"}
    main = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True,
                          text=True, check=True).stdout
    assert "qsa_probe" not in main
    p = ctypes.CDLL(PROBE_LIB)
    p.qsa_probe_mfma.argtypes = [ctypes.c_int32] * 3 + [ctypes.c_void_p] * 2
    p.qsa_probe_mfma_ops.argtypes = [ctypes.c_int32] * 3
    p.qsa_probe_mfma_ops.restype = ctypes.c_double
    for args in ((3, 10, 4, 16), (0, 0, 4, 16), (1, 10, 0, 16), (2, 10, 4, None)):
        assert p.qsa_probe_mfma(*args, None) == -1, args
    # ops per launch: waves x iterations x (ops of the MFMAs of one iteration)
    assert p.qsa_probe_mfma_ops(0, 10, 2) == 8 * 10 * 4 * 65536
    assert p.qsa_probe_mfma_ops(1, 10, 2) == 8 * 10 * 4 * 32768
    assert p.qsa_probe_mfma_ops(2, 10, 2) == 8 * 10 * (2 * 65536 + 4 * 32768)
