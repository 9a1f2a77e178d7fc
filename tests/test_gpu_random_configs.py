"""A seeded sweep of random configurations through the whole path.

Each case draws batch, heads, sequence length (mostly ragged), head_dim,
block size, top-k, a band of block offsets (QuantSparse, gist.science/es/paper/
2509.23681, technical summary §2A: top-k local guidance plus the pooled
global guidance) and the generator's value mix, then checks, through the C
ABI against the oracle:

* codes, scales, pooled sums and kept lists bit-exact;
* the sparse attention and its fused correction out = sparse + r + dr
  (technical summary §2B) within rel-L2 5e-3 and max-abs 2e-2;
* the refresh step: full output within the same bound, and r = full - sparse
  against its fp64 value (both sides round a cancellation to bf16, so the
  measure is relative to the full output, as in the parity tests);
* the ordered entry points give the same bits as the plain ones.

The draws are fixed by the seed, so a failure names a reproducible case.
"""
import numpy as np
import pytest
import torch

import oracle
import qsa_gen
from quantized_sparse_attention_amd import binding as B
from tests.gpu_util import assert_close, dev_bf16, host_bits, host_f64, oracle_front

pytestmark = pytest.mark.gpu

TINY = qsa_gen.get_workload("tiny")
N_CASES = 48


def _draw(seed):
    rng = np.random.default_rng(1000 + seed)
    D = int(rng.choice([64, 128]))
    block = int(rng.choice([64, 128]))
    nb_target = int(rng.integers(1, 25))
    L = max(1, nb_target * block - int(rng.integers(0, block)))  # mostly ragged
    nb = -(-L // block)
    band_pool = [-3, -2, -1, 0, 1, 2, 3]
    band = {int(b) for b in rng.choice(band_pool, size=int(rng.integers(0, 4)), replace=False)}
    topk = int(rng.integers(0, nb + 1))
    if topk == 0:
        band.add(0)  # every row must keep something (the diagonal then)
    band = tuple(sorted(band))
    w = TINY.with_(batch=int(rng.integers(1, 3)), heads=int(rng.integers(1, 4)),
                   grid=(1, 1, L), block=block, head_dim=D,
                   noise_std=float(rng.choice([0.3, 1.0])),
                   outlier_channels=int(rng.integers(0, 4)),
                   outlier_gain=float(rng.choice([4.0, 10.0])))
    return w, topk, band


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_config(seed):
    w, topk, band = _draw(seed)
    case = (f"seed={seed} B={w.batch} H={w.heads} L={w.seq_len} D={w.head_dim} "
            f"block={w.block} topk={topk} band={band}")
    print(case, flush=True)
    x = qsa_gen.make_qkv(w, step=seed % 3)
    o = oracle_front(x, w, topk=topk, band=band)
    q, k, v = dev_bf16(x["q"]), dev_bf16(x["k"]), dev_bf16(x["v"])
    qc, qs, qp = B.qsa_quantize(q, w.block)
    kc, ks, kp = B.qsa_quantize(k, w.block)
    idx, cnt = B.qsa_select_blocks(qp, qs, kp, ks, w.seq_len, w.block, topk, band, o["kmax"])
    torch.cuda.synchronize()
    for got, want, nm in ((qc, o["qc"], "q codes"), (kc, o["kc"], "k codes"),
                          (qp, o["pq"], "q pooled"), (kp, o["pk"], "k pooled"),
                          (cnt, o["cnt"], "counts"), (idx, o["idx"], "kept lists")):
        assert np.array_equal(got.cpu().numpy(), want), f"{case}: {nm}"
    for got, want, nm in ((qs, o["sq"], "q scales"), (ks, o["sk"], "k scales")):
        assert np.array_equal(got.cpu().numpy().view(np.uint32), want.view(np.uint32)), \
            f"{case}: {nm}"

    sm = oracle.default_sm_scale(w.head_dim)
    o_sp = oracle.attention(o["qc"], o["sq"], o["kc"], o["sk"], x["v"], o["idx"], o["cnt"],
                            w.block, sm)
    full_lists = oracle.full_kept_lists(w.batch, w.heads, w.n_blocks)
    o_full = oracle.attention(o["qc"], o["sq"], o["kc"], o["sk"], x["v"], *full_lists, w.block,
                              sm)

    rng = np.random.default_rng(seed)
    noise = lambda a: qsa_gen.f32_to_bf16_bits(  # noqa: E731
        rng.standard_normal(x["v"].shape).astype(np.float32) * a)
    r_bits, dr_bits = noise(0.05), noise(0.01)
    out = B.qsa_sparse_attn(qc, qs, kc, ks, v, idx, cnt, w.block)
    assert_close(host_f64(out), o_sp, what=f"{case}: sparse")
    out_c = B.qsa_sparse_attn(qc, qs, kc, ks, v, idx, cnt, w.block, r=dev_bf16(r_bits),
                              dr=dev_bf16(dr_bits))
    want_c = o_sp + oracle.bf16_to_f64(r_bits) + oracle.bf16_to_f64(dr_bits)
    assert_close(host_f64(out_c), want_c, what=f"{case}: sparse + r + dr")

    order = B.qsa_order_query_blocks(idx, cnt, w.seq_len, w.block, w.head_dim)
    out_o = B.qsa_sparse_attn_ordered(qc, qs, kc, ks, v, idx, cnt, order, w.block)
    assert np.array_equal(host_bits(out), host_bits(out_o)), f"{case}: ordered sparse"

    res = []
    for od in (None, order):
        r = torch.zeros_like(v)
        dr = torch.zeros_like(v)
        full = B.qsa_full_attn_residual(qc, qs, kc, ks, v, idx, cnt, w.block, r, dr, 0,
                                        order=od)
        res.append((host_bits(full), host_bits(r), host_bits(dr)))
    full_b, r_b, dr_b = res[0]
    for a_, b_ in zip(res[0], res[1]):
        assert np.array_equal(a_, b_), f"{case}: ordered refresh"
    full_f = oracle.bf16_to_f64(full_b)
    assert_close(full_f, o_full, what=f"{case}: refresh full")
    err = oracle.bf16_to_f64(r_b) - (o_full - o_sp)
    scale = np.linalg.norm(o_full)
    assert np.linalg.norm(err) / (scale if scale > 0 else 1.0) <= 5e-3, f"{case}: r"
    assert np.max(np.abs(err)) <= 2e-2, f"{case}: r max-abs"
    assert np.all(dr_b == 0), f"{case}: dr without a previous refresh"
