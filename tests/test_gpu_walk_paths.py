"""GPU parity where the two-buffer tile walk of the 64-token / 128-channel
kernels cannot take its precomputed tile list and walks the kept-set bitmaps
instead.

The list of a phase lives in the LDS words past the two kept-set bitmaps:
2 * (1024 - 2 * ceil(nb / 32) - 2) entries.  A phase whose tiles outnumber
that walks the bitmaps.  Two workloads force it, with ragged last blocks:

* a sparse step over 4,096 key blocks keeping 2,000 per query block: every
  group's union (>= 2,000 tiles) exceeds the 1,532 entries, so the kept phase
  walks the bitmaps;
* a refresh step over 2,304 key blocks keeping 300: the kept phase (<= 600
  tiles) takes the list, the complement phase (>= 2,004 tiles against 1,756
  entries) the bitmaps.

The oracle checks sampled query blocks (first, second, middle, the ragged last
one, two random) to the attention tolerance; the kept lists bit-exactly.
"""
import numpy as np
import pytest
import torch

import oracle
import qsa_gen
from quantized_sparse_attention_amd import binding as B
from tests.gpu_util import MAX_ABS, REL_L2, host_bits, host_f64, rel_l2

pytestmark = pytest.mark.gpu


def _list_entries(nb):
    return 2 * (1024 - 2 * (-(-nb // 32)) - 2)


def _front_end(w):
    dev = torch.device("cuda:0")
    x = qsa_gen.make_qkv_torch(w, dev)[0]
    qc, qs, qp = B.qsa_quantize(x["q"], w.block)
    kc, ks, kp = B.qsa_quantize(x["k"], w.block)
    idx, cnt = B.qsa_select_blocks(qp, qs, kp, ks, w.seq_len, w.block, w.topk, w.band, w.kmax)
    host = {t: host_bits(x[t]) for t in "qkv"}
    oqc, osq, opq = oracle.quantize(host["q"], w.block)
    okc, osk, opk = oracle.quantize(host["k"], w.block)
    sc = oracle.block_scores(opq, osq, opk, osk, w.seq_len, w.block)
    oidx, ocnt = oracle.select_blocks(sc, w.topk, w.band, w.kmax)
    assert np.array_equal(idx.cpu().numpy(), oidx) and np.array_equal(cnt.cpu().numpy(), ocnt)
    return x, (qc, qs, kc, ks, idx, cnt), host, (oqc, osq, okc, osk, oidx, ocnt)


def _samples(nb):
    rng = np.random.default_rng(nb)
    extra = [int(v) for v in rng.choice(np.arange(2, nb - 2), size=2, replace=False)]
    return sorted({0, 1, nb // 2, nb - 1, *extra})


def _check(got, want, w, what):
    for (b, h, i), ref in want.items():
        t0 = i * w.block
        g = got[b, h, t0:t0 + ref.shape[0]]
        r, m = rel_l2(g, ref), float(np.abs(g - ref).max())
        assert r <= REL_L2 and m <= MAX_ABS, f"{what} block {i}: rel_l2={r:.3e} max_abs={m:.3e}"


def test_sparse_kept_phase_on_bitmaps():
    w = qsa_gen.get_workload("tiny").with_(cfg_id=31, heads=1, head_dim=128, grid=(4, 255, 257),
                                           block=64, topk_override=2000, noise_std=0.3)
    assert w.n_blocks == 4096 and w.seq_len % 64 and w.topk > _list_entries(w.n_blocks)
    print(f"\n[walk paths] sparse L={w.seq_len} nb={w.n_blocks} topk={w.topk}", flush=True)
    x, (qc, qs, kc, ks, idx, cnt), host, (oqc, osq, okc, osk, oidx, ocnt) = _front_end(w)
    out = B.qsa_sparse_attn(qc, qs, kc, ks, x["v"], idx, cnt, w.block)
    order = B.qsa_order_query_blocks(idx, cnt, w.seq_len, w.block, w.head_dim)
    out_o = B.qsa_sparse_attn_ordered(qc, qs, kc, ks, x["v"], idx, cnt, order, w.block)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out_o.view(torch.int16))
    sm = oracle.default_sm_scale(w.head_dim)
    want = oracle.attention(oqc, osq, okc, osk, host["v"], oidx, ocnt, w.block, sm,
                            which=[(0, 0, i) for i in _samples(w.n_blocks)])
    _check(host_f64(out), want, w, "sparse")
    print("[walk paths] sparse ok", flush=True)


def test_refresh_complement_phase_on_bitmaps():
    w = qsa_gen.get_workload("tiny").with_(cfg_id=32, heads=1, head_dim=128, grid=(9, 127, 129),
                                           block=64, topk_override=300, noise_std=0.3)
    nb = w.n_blocks
    assert nb == 2304 and w.seq_len % 64
    assert 2 * w.kmax <= _list_entries(nb) < nb - w.kmax
    print(f"\n[walk paths] refresh L={w.seq_len} nb={nb} topk={w.topk}", flush=True)
    x, (qc, qs, kc, ks, idx, cnt), host, (oqc, osq, okc, osk, oidx, ocnt) = _front_end(w)
    r = torch.zeros_like(x["v"])
    dr = torch.zeros_like(r)
    full = B.qsa_full_attn_residual(qc, qs, kc, ks, x["v"], idx, cnt, w.block, r, dr, 0)
    sparse = B.qsa_sparse_attn(qc, qs, kc, ks, x["v"], idx, cnt, w.block)
    torch.cuda.synchronize()
    sm = oracle.default_sm_scale(w.head_dim)
    which = [(0, 0, i) for i in _samples(nb)]
    fi, fc = oracle.full_kept_lists(1, 1, nb)
    want_full = oracle.attention(oqc, osq, okc, osk, host["v"], fi, fc, w.block, sm, which=which)
    _check(host_f64(full), want_full, w, "refresh output")
    want_sparse = oracle.attention(oqc, osq, okc, osk, host["v"], oidx, ocnt, w.block, sm,
                                   which=which)
    _check(host_f64(sparse), want_sparse, w, "sparse output")
    # r = bf16(full - sparse) against the oracle's residual of the same blocks
    got_r = host_f64(r)
    for key, ref in want_full.items():
        i = key[2]
        t0 = i * w.block
        rho = ref - want_sparse[key]
        err = got_r[0, 0, t0:t0 + ref.shape[0]] - rho
        assert np.linalg.norm(err) / np.linalg.norm(ref) <= REL_L2, f"r block {i}"
        assert float(np.abs(err).max()) <= 2 * MAX_ABS + 2.0 ** -8 * float(np.abs(rho).max())
    print("[walk paths] refresh ok", flush=True)


def test_maximum_block_count():
    """QSA_MAX_BLOCKS = 16,384 key blocks of 64 tokens with a ragged last
    block (1,048,575 tokens, one head): the select runs one row per workgroup
    with its keys in LDS, and the attention walks the bitmaps at their full
    width (no words are left for a tile list).  Codes bit-exact on the whole
    tensor; kept lists bit-exact on sampled rows (the oracle's top-k of those
    rows plus the band); sparse outputs (plain and ordered) on sampled query
    blocks and the refresh output on the first and the ragged last block."""
    w = qsa_gen.get_workload("tiny").with_(cfg_id=33, heads=1, head_dim=128, grid=(25, 1271, 33),
                                           block=64, topk_override=6, noise_std=0.3)
    nb = w.n_blocks
    assert nb == B.QSA_MAX_BLOCKS and w.seq_len % 64 == 63 and w.kmax == w.topk + 1
    print(f"\n[walk paths] maximum L={w.seq_len} nb={nb} topk={w.topk}", flush=True)
    dev = torch.device("cuda:0")
    x = qsa_gen.make_qkv_torch(w, dev)[0]
    qc, qs, qp = B.qsa_quantize(x["q"], w.block)
    kc, ks, kp = B.qsa_quantize(x["k"], w.block)
    idx, cnt = B.qsa_select_blocks(qp, qs, kp, ks, w.seq_len, w.block, w.topk, w.band, w.kmax)
    out = B.qsa_sparse_attn(qc, qs, kc, ks, x["v"], idx, cnt, w.block)
    order = B.qsa_order_query_blocks(idx, cnt, w.seq_len, w.block, w.head_dim)
    out_o = B.qsa_sparse_attn_ordered(qc, qs, kc, ks, x["v"], idx, cnt, order, w.block)
    r = torch.zeros_like(x["v"])
    dr = torch.zeros_like(r)
    full = B.qsa_full_attn_residual(qc, qs, kc, ks, x["v"], idx, cnt, w.block, r, dr, 0)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out_o.view(torch.int16))
    print("[walk paths] maximum: GPU done", flush=True)
    host = {t: host_bits(x[t]) for t in "qkv"}
    oqc, osq, opq = oracle.quantize(host["q"], w.block)
    okc, osk, opk = oracle.quantize(host["k"], w.block)
    assert np.array_equal(qc.cpu().numpy(), oqc) and np.array_equal(kc.cpu().numpy(), okc)
    assert np.array_equal(qs.cpu().numpy().view(np.uint32), osq.view(np.uint32))
    assert np.array_equal(kp.cpu().numpy(), opk)
    print("[walk paths] maximum: codes ok", flush=True)
    rows = _samples(nb)
    sc = oracle.block_scores(opq, osq, opk, osk, w.seq_len, w.block)[:, :, rows].copy()
    oidx, ocnt = oracle.select_blocks(sc, w.topk, w.band, w.kmax, rows=rows)
    del sc
    gidx, gcnt = idx.cpu().numpy(), cnt.cpu().numpy()
    assert np.array_equal(gidx[:, :, rows], oidx) and np.array_equal(gcnt[:, :, rows], ocnt)
    print("[walk paths] maximum: kept lists ok", flush=True)
    sm = oracle.default_sm_scale(w.head_dim)
    want = oracle.attention(oqc, osq, okc, osk, host["v"], gidx, gcnt, w.block, sm,
                            which=[(0, 0, i) for i in rows])
    _check(host_f64(out), want, w, "sparse")
    fi, fc = oracle.full_kept_lists(1, 1, nb)
    want_full = oracle.attention(oqc, osq, okc, osk, host["v"], fi, fc, w.block, sm,
                                 which=[(0, 0, 0), (0, 0, nb - 1)])
    _check(host_f64(full), want_full, w, "refresh output")
    print("[walk paths] maximum ok", flush=True)
