"""GPU parity of the HIP path (through the C ABI) against the CPU oracle.

Bit-exact: int8 codes, fp32 scales, pooled sums and kept block lists.
Within tolerance (rel-L2 <= 5e-3 and max-abs <= 2e-2 against fp64): every
bf16 attention output, and the residuals relative to the full output.
Shapes span several tiles and a ragged tail at sizes the oracle finishes in
seconds.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import qsa_gen
from quantized_sparse_attention_amd import binding as B
from tests.gpu_util import (assert_close, dev_bf16, host_bits, host_f64, oracle_front, rel_l2)

pytestmark = pytest.mark.gpu

TINY = qsa_gen.get_workload("tiny")
CFGS = {
    "tiny": (TINY, {}),
    "tail64_d128": (TINY.with_(grid=(1, 10, 30), block=64, head_dim=128, outlier_channels=3,
                               outlier_gain=10.0), dict(topk=2, band=(0,))),
    "tail128_d128": (TINY.with_(grid=(1, 1, 333), block=128, head_dim=128),
                     dict(topk=1, band=(-1, 0))),
    "d64_b128": (TINY.with_(grid=(3, 7, 11), block=128, head_dim=64), dict(topk=1, band=())),
    "batch2_h3": (TINY.with_(batch=2, heads=3, grid=(2, 12, 40), block=64, head_dim=128,
                             noise_std=0.3, outlier_channels=3, outlier_gain=10.0),
                  dict(topk=3, band=(0,))),
    "wide_band": (TINY.with_(grid=(1, 20, 64), block=64, head_dim=128),
                  dict(topk=4, band=(-3, -1, 0, 1, 3))),
}


def _gpu_front(x, w, topk, band, kmax, select_work=False):
    """GPU quantise + select; select_work: through qsa_select_blocks_work with
    room for every slice in one pass."""
    q, k = dev_bf16(x["q"]), dev_bf16(x["k"])
    qc, qs, qp = B.qsa_quantize(q, w.block)
    kc, ks, kp = B.qsa_quantize(k, w.block)
    work = None
    if select_work:
        n = B.qsa_select_slice_bytes(w.batch, w.heads, w.seq_len, w.head_dim, w.block)
        work = torch.empty(n * w.batch * w.heads, dtype=torch.uint8, device=q.device)
    idx, cnt = B.qsa_select_blocks(qp, qs, kp, ks, w.seq_len, w.block, topk, band, kmax,
                                   work=work)
    torch.cuda.synchronize()
    return dict(qc=qc, qs=qs, qp=qp, kc=kc, ks=ks, kp=kp, idx=idx, cnt=cnt)


def _setup(name, step=0):
    w, kw = CFGS[name]
    x = qsa_gen.make_qkv(w, step)
    o = oracle_front(x, w, **kw)
    g = _gpu_front(x, w, o["topk"], o["band"], o["kmax"])
    return w, x, o, g


@pytest.mark.parametrize("name", list(CFGS))
def test_quantize_bit_exact(name):
    w, x, o, g = _setup(name)
    assert np.array_equal(g["qc"].cpu().numpy(), o["qc"])
    assert np.array_equal(g["kc"].cpu().numpy(), o["kc"])
    assert np.array_equal(g["qs"].cpu().numpy().view(np.uint32), o["sq"].view(np.uint32))
    assert np.array_equal(g["ks"].cpu().numpy().view(np.uint32), o["sk"].view(np.uint32))
    assert np.array_equal(g["qp"].cpu().numpy(), o["pq"])
    assert np.array_equal(g["kp"].cpu().numpy(), o["pk"])


@pytest.mark.parametrize("select_work", [False, True])
@pytest.mark.parametrize("name", list(CFGS))
def test_select_bit_exact(name, select_work):
    w, x, o, _ = _setup(name)
    g = _gpu_front(x, w, o["topk"], o["band"], o["kmax"], select_work)
    assert np.array_equal(g["cnt"].cpu().numpy(), o["cnt"])
    assert np.array_equal(g["idx"].cpu().numpy(), o["idx"])


def _oracle_attn(o, x, w, kept=None):
    idx, cnt = (o["idx"], o["cnt"]) if kept is None else kept
    return oracle.attention(o["qc"], o["sq"], o["kc"], o["sk"], x["v"], idx, cnt, w.block,
                            oracle.default_sm_scale(w.head_dim))


@pytest.mark.parametrize("name", list(CFGS))
def test_sparse_attn_parity(name):
    w, x, o, g = _setup(name)
    v = dev_bf16(x["v"])
    out = B.qsa_sparse_attn(g["qc"], g["qs"], g["kc"], g["ks"], v, g["idx"], g["cnt"], w.block)
    want = _oracle_attn(o, x, w)
    assert_close(host_f64(out), want, what=f"{name} sparse")
    # residual inputs fused in the epilogue
    rng = np.random.default_rng(1)
    r = qsa_gen.f32_to_bf16_bits(rng.standard_normal(x["v"].shape).astype(np.float32) * 0.05)
    dr = qsa_gen.f32_to_bf16_bits(rng.standard_normal(x["v"].shape).astype(np.float32) * 0.01)
    out2 = B.qsa_sparse_attn(g["qc"], g["qs"], g["kc"], g["ks"], v, g["idx"], g["cnt"], w.block,
                             r=dev_bf16(r), dr=dev_bf16(dr))
    want2 = want + oracle.bf16_to_f64(r) + oracle.bf16_to_f64(dr)
    assert_close(host_f64(out2), want2, what=f"{name} sparse+r+dr")
    out1 = B.qsa_sparse_attn(g["qc"], g["qs"], g["kc"], g["ks"], v, g["idx"], g["cnt"], w.block,
                             r=dev_bf16(r))
    assert_close(host_f64(out1), want + oracle.bf16_to_f64(r), what=f"{name} sparse+r")


@pytest.mark.parametrize("name", list(CFGS))
@pytest.mark.parametrize("has_prev", [0, 1])
def test_refresh_parity(name, has_prev):
    w, x, o, g = _setup(name)
    v = dev_bf16(x["v"])
    shape = x["v"].shape
    rng = np.random.default_rng(2)
    r_prev = qsa_gen.f32_to_bf16_bits(rng.standard_normal(shape).astype(np.float32) * 0.02)
    r = dev_bf16(r_prev)
    dr = torch.zeros_like(v)
    out = B.qsa_full_attn_residual(g["qc"], g["qs"], g["kc"], g["ks"], v, g["idx"], g["cnt"],
                                   w.block, r, dr, has_prev)
    o_sp = _oracle_attn(o, x, w)
    o_full = _oracle_attn(o, x, w, oracle.full_kept_lists(w.batch, w.heads, w.n_blocks))
    st = oracle.ResidualState(shape)
    if has_prev:
        st.r, st.has_prev = r_prev.copy(), True
    oracle.refresh_step(st, o_full, o_sp)
    assert_close(host_f64(out), o_full, what=f"{name} full")
    # r and dr are stored in bf16 by both sides; compare each against its
    # unrounded fp64 value (a bf16 rounding flip is not an error of the path).
    # They are cancellations, so the relative measure uses the full output.
    rho = o_full - o_sp
    dr_ref = rho - oracle.bf16_to_f64(r_prev) if has_prev else np.zeros_like(rho)
    scale = np.linalg.norm(o_full)
    for got, ref, nm in ((host_f64(r), rho, "r"), (host_f64(dr), dr_ref, "dr")):
        err = got - ref
        assert np.linalg.norm(err) / scale <= 5e-3, (nm, np.linalg.norm(err) / scale)
        assert np.max(np.abs(err)) <= 2e-2, (nm, np.max(np.abs(err)))
    if not has_prev:
        assert np.all(host_bits(dr) == 0)


@pytest.mark.parametrize("name", ["tiny", "tail64_d128", "tail128_d128"])
def test_refresh_sparse_part_matches_sparse_kernel(name):
    # The refresh kernel's sparse partition uses the sparse kernel's numerics:
    # r + (sparse output) reproduces the full output up to bf16 rounding.
    w, x, o, g = _setup(name)
    v = dev_bf16(x["v"])
    sp = B.qsa_sparse_attn(g["qc"], g["qs"], g["kc"], g["ks"], v, g["idx"], g["cnt"], w.block)
    r = torch.zeros_like(v)
    dr = torch.zeros_like(v)
    full = B.qsa_full_attn_residual(g["qc"], g["qs"], g["kc"], g["ks"], v, g["idx"], g["cnt"],
                                    w.block, r, dr, 0)
    recon = host_f64(sp) + host_f64(r)
    assert rel_l2(recon, host_f64(full)) < 4e-3


def _rotated_front(x, w, topk, band):
    qc, sq, pq = oracle.quantize_rotated(x["q"], w.block)
    kc, sk, pk = oracle.quantize_rotated(x["k"], w.block)
    sc = oracle.block_scores(pq, sq, pk, sk, w.seq_len, w.block)
    idx, cnt = oracle.select_blocks(sc, topk, band, min(w.n_blocks, topk + len(band)))
    return dict(qc=qc, sq=sq, kc=kc, sk=sk, idx=idx, cnt=cnt)


@pytest.mark.parametrize("schedule,order,rotate,rank",
                         [(s, o, False, None) for s in ("FSS", "FSFS", "FSSFSS") for o in (2, 1)]
                         + [("FSFS", 2, True, None), ("FSFSFS", 2, False, 8)])
def test_schedule_against_oracle_state_machine(schedule, order, rotate, rank):
    from quantized_sparse_attention_amd import QSAConfig, QuantSparseAttention
    w = TINY.with_(grid=(2, 8, 24), head_dim=64)  # 384 tokens, 6 blocks
    topk, band = 2, (0,)
    steps = qsa_gen.make_qkv_steps(w, len(schedule))
    layer = QuantSparseAttention(QSAConfig(block=w.block, topk=topk, band=band, order=order,
                                           rotate=rotate, rank=rank))
    st = oracle.ResidualState(steps[0]["v"].shape)
    sm = oracle.default_sm_scale(w.head_dim)
    if rotate:
        sm = np.float32(sm / np.float32(w.head_dim))
    cache = None
    for s, kind in enumerate(schedule):
        x = steps[s]
        r_prev = None if layer.r is None else host_f64(layer.r)
        v = dev_bf16(x["v"])
        out = layer.step(dev_bf16(x["q"]), dev_bf16(x["k"]), v, kind == "F")
        o = (_rotated_front(x, w, topk, band) if rotate
             else oracle_front(x, w, topk=topk, band=band))
        o_sp = oracle.attention(o["qc"], o["sq"], o["kc"], o["sk"], x["v"], o["idx"], o["cnt"],
                                w.block, sm)
        if kind == "F":
            fi, fc = oracle.full_kept_lists(w.batch, w.heads, w.n_blocks)
            o_full = oracle.attention(o["qc"], o["sq"], o["kc"], o["sk"], x["v"], fi, fc,
                                      w.block, sm)
            want = oracle.refresh_step(st, o_full, o_sp, rank=rank)
            got = host_f64(out)
            assert_close(got, want, what=f"step {s} {kind}")
            # r and dr are differences of the full and the sparse attention:
            # each element is held to the errors of those two outputs
            # (measured: the refresh output and the sparse kernel's output on
            # the same inputs, which takes the refresh kernel's sparse walk)
            # plus their bf16 roundings
            lb = layer.last
            sp = host_f64(B.qsa_sparse_attn(lb.q_codes, lb.q_scales, lb.k_codes, lb.k_scales, v,
                                            lb.kept_idx, lb.kept_cnt, w.block, float(sm)))
            src = (np.abs(got - o_full) + _half_ulp(got) + np.abs(sp - o_sp) + _half_ulp(sp)
                   + 2.0 ** -22 * np.abs(got))
            rho = o_full - o_sp
            r = host_f64(layer.r)
            assert np.all(np.abs(r - rho) <= src + _half_ulp(r)), f"step {s} r"
            if r_prev is not None and rank is None:
                dr = host_f64(layer.dr)
                assert np.all(np.abs(dr - (rho - r_prev)) <= src + _half_ulp(dr)), f"step {s} dr"
            elif r_prev is None:
                assert np.all(host_bits(layer.dr) == 0), f"step {s} dr at the first refresh"
            cache = (host_bits(layer.r), host_bits(layer.dr))
            if rank is not None and s > 0:
                # the cached second-order residual is numerically of rank <= r
                # (bf16 rounding of a rank-r matrix moves its singular values
                # by at most 2^-9 of its norm) and holds the optimal energy
                g, rf = host_f64(layer.dr), oracle.bf16_to_f64(st.dr)
                for b in range(w.batch):
                    for h in range(w.heads):
                        sv = np.linalg.svd(g[b, h], compute_uv=False)
                        assert sv[rank] <= 2.0 ** -8 * np.linalg.norm(g[b, h]), (s, b, h)
                        eg, er = np.sum(g[b, h] ** 2), np.sum(rf[b, h] ** 2)
                        assert abs(eg - er) <= 2e-2 * er, (s, b, h, eg, er)
        else:
            want = oracle.sparse_step(st, o_sp, order=order)
            # end to end against the oracle's own state machine
            r_ = rel_l2(host_f64(out), want)
            assert r_ <= 5e-3, (s, kind, r_)
            # the epilogue adds exactly the cached residuals to the sparse
            # output, and sparse steps leave the caches as the refresh wrote them
            assert np.array_equal(host_bits(layer.r), cache[0]), f"step {s}: r changed"
            assert np.array_equal(host_bits(layer.dr), cache[1]), f"step {s}: dr changed"
            cached = host_f64(layer.r) + (host_f64(layer.dr) if order == 2 else 0.0)
            assert_close(host_f64(out), o_sp + cached, what=f"step {s} {kind}")
        assert np.array_equal(layer.last.kept_idx.cpu().numpy(), o["idx"])


def _half_ulp(x):
    """Half the bf16 spacing at |x| (normal range)."""
    return np.exp2(np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** -126))) - 8)


def test_apply_residual():
    rng = np.random.default_rng(4)
    shape = (1, 3, 200, 128)
    a, r, dr = (qsa_gen.f32_to_bf16_bits(rng.standard_normal(shape).astype(np.float32) * s)
                for s in (1.0, 0.1, 0.01))
    want = oracle.bf16_to_f64(a) + oracle.bf16_to_f64(r) + oracle.bf16_to_f64(dr)
    got = B.qsa_apply_residual(dev_bf16(a), dev_bf16(r), dev_bf16(dr))
    assert_close(host_f64(got), want, what="apply")
    # bf16 rounding of an fp32 sum: within half a bf16 ulp of the fp64 sum (plus fp32 rounding)
    assert np.all(np.abs(host_f64(got) - want) <= np.abs(want) * (2.0 ** -8 + 2.0 ** -22) + 1e-30)
    # in place, and without dr
    ta = dev_bf16(a)
    B.qsa_apply_residual(ta, dev_bf16(r), None, out=ta)
    assert_close(host_f64(ta), oracle.bf16_to_f64(a) + oracle.bf16_to_f64(r), what="apply r only")


def test_quantize_map_sweep():
    # Every finite bf16 x against a ladder of bf16 amax values across the whole
    # exponent range (subnormal scales included): codes and scales bit-exact.
    allx = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    xf = qsa_gen.bf16_bits_to_f32(allx)
    xf = xf[np.isfinite(xf)]
    mags = np.unique(np.abs(xf))
    amaxes = [m for m in mags[1:] if True][::97] + [mags[-1]]
    rows = []
    for am in amaxes:
        xs = xf[np.abs(xf) <= am]
        blk = np.concatenate([[am], xs]).astype(np.float32)
        pad = (-len(blk)) % (64 * 128)
        blk = np.concatenate([blk, np.full(pad, am, np.float32)])  # fill with amax itself
        rows.append(blk.reshape(-1, 64, 128))
    data = np.concatenate(rows).reshape(1, 1, -1, 128)
    bits = qsa_gen.f32_to_bf16_bits(data)
    c_o, s_o, p_o = oracle.quantize(bits, 64)
    c_g, s_g, p_g = B.qsa_quantize(dev_bf16(bits), 64)
    assert np.array_equal(s_g.cpu().numpy().view(np.uint32), s_o.view(np.uint32))
    assert np.array_equal(c_g.cpu().numpy(), c_o)
    assert np.array_equal(p_g.cpu().numpy(), p_o)


def test_quantize_half_integer_quotients():
    # Quotients x / scale at and next to every half-integer k + 1/2 (k < 127):
    # scales that are powers of two (amax = 127 * 2^e: the ties are exact) and
    # others (amax = 127 * 2^e * (1 + j/128) rounded to bf16), for exponents on
    # both sides of 2^-100 and up to 2^120.  Each block holds its amax first,
    # then the bf16 values nearest to +-(k + 1/2) * scale and their bf16
    # neighbours, padded with amax.  Codes, scales and sums bit-exact.
    blocks = []
    for e in [-122, -110, -104, -101, -100, -99, -98, -60, -20, -3, 0, 7, 60, 120]:
        for j in (0, 1, 37, 101):
            am_bits = qsa_gen.f32_to_bf16_bits(
                np.array([127.0 * 2.0 ** e * (1 + j / 128)], np.float32))
            am = np.float32(qsa_gen.bf16_bits_to_f32(am_bits)[0])
            sc = am / np.float32(127.0)
            t = ((np.arange(127) + 0.5) * np.float64(sc)).astype(np.float32)
            tb = qsa_gen.f32_to_bf16_bits(t).astype(np.int32)
            near = np.concatenate([tb - 1, tb, tb + 1]).astype(np.uint16)
            v = qsa_gen.bf16_bits_to_f32(near)
            v = v[np.isfinite(v) & (np.abs(v) <= am)]
            blk = np.concatenate([[am], v, -v]).astype(np.float32)
            assert blk.size <= 64 * 128
            blk = np.concatenate([blk, np.full(64 * 128 - blk.size, am, np.float32)])
            blocks.append(blk.reshape(64, 128))
    data = np.stack(blocks).reshape(1, 1, -1, 128)
    bits = qsa_gen.f32_to_bf16_bits(data)
    c_o, s_o, p_o = oracle.quantize(bits, 64)
    c_g, s_g, p_g = B.qsa_quantize(dev_bf16(bits), 64)
    assert np.array_equal(s_g.cpu().numpy().view(np.uint32), s_o.view(np.uint32))
    assert np.array_equal(c_g.cpu().numpy(), c_o)
    assert np.array_equal(p_g.cpu().numpy(), p_o)
    # the set really holds exact ties and codes rounded both ways
    q = data.reshape(-1)[: 64 * 128].astype(np.float64) / np.float64(s_o.reshape(-1)[0])
    assert np.any(np.abs(q - np.round(q - 0.5) - 0.5) == 0)


GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_examples.json")


@pytest.mark.parametrize("name", ["H1", "H2_noband", "H2_band0"])
def test_hand_examples_on_gpu(name):
    with open(GOLDEN) as f:
        gd = json.load(f)[name]
    blk, D = gd["block"], gd["head_dim"]
    nb = len(gd["q_blocks"])

    def const(vals):
        xx = np.concatenate([np.full((blk, D), v, np.float32) for v in vals])
        return qsa_gen.f32_to_bf16_bits(xx)[None, None]

    L = nb * blk
    t = np.arange(L)[:, None]
    d = np.arange(D)[None, :]
    vf = ((((7 * t + 3 * d) % 17) - 8) / 8.0).astype(np.float32)
    q, k, v = const(gd["q_blocks"]), const(gd["k_blocks"]), qsa_gen.f32_to_bf16_bits(vf)[None, None]
    qc, qs, qp = B.qsa_quantize(dev_bf16(q), blk)
    kc, ks, kp = B.qsa_quantize(dev_bf16(k), blk)
    idx, cnt = B.qsa_select_blocks(qp, qs, kp, ks, L, blk, gd["topk"], gd["band"], nb)
    got = [idx[0, 0, i, : cnt[0, 0, i]].tolist() for i in range(nb)]
    assert got == gd["kept"]
    out = host_f64(B.qsa_sparse_attn(qc, qs, kc, ks, dev_bf16(v), idx, cnt, blk))[0, 0]
    means = [vf[j * blk:(j + 1) * blk].astype(np.float64).mean(axis=0) for j in range(nb)]
    for i, kept in enumerate(gd["kept"]):
        if len(kept) == 1:
            want = means[kept[0]]
        elif name == "H2_band0" and kept == [1, 2]:
            # both kept blocks have the same keys: a uniform softmax over them
            want = (means[1] + means[2]) / 2
        else:
            # H2_band0 block 0: keys of block 0 (codes -127) and block 1 (codes
            # +127) against queries of codes +127, all scales fl32(1/127):
            # logits -z and +z with z = sm_scale * s^2 * 64 * 127^2, so the
            # weight of block 1 is 1 / (1 + exp(-2 z))
            assert name == "H2_band0" and kept == [0, 1]
            s = float(np.float32(1.0) / np.float32(127.0))
            z = float(oracle.default_sm_scale(D)) * s * s * 64 * 127 * 127
            w1 = 1.0 / (1.0 + np.exp(-2.0 * z))
            want = w1 * means[1] + (1.0 - w1) * means[0]
        want = np.broadcast_to(want, (blk, D))
        assert np.max(np.abs(out[i * blk:(i + 1) * blk] - want)) <= 2e-2, (name, i, kept)


@pytest.mark.parametrize("select_work", [False, True])
def test_select_edges(select_work):
    w = TINY.with_(grid=(1, 9, 64), head_dim=128)  # 576 tokens, 9 blocks
    x = qsa_gen.make_qkv(w)
    # an all-zero key block gives +-0 scores that tie
    x["k"][0, 0, 128:192] = 0
    for topk, band in [(0, (0,)), (9, (0,)), (20, (0,)), (3, (-8, 0, 8)), (1, (0, 2, -2, 5))]:
        o = oracle_front(x, w, topk=topk, band=band, kmax=9)
        g = _gpu_front(x, w, topk, band, 9, select_work)
        assert np.array_equal(g["idx"].cpu().numpy(), o["idx"]), (topk, band)
        assert np.array_equal(g["cnt"].cpu().numpy(), o["cnt"]), (topk, band)
    assert np.all(g["ks"].cpu().numpy()[0, 0, 2] == 0)


@pytest.mark.parametrize("select_work", [False, True])
@pytest.mark.parametrize("case", ["all_equal", "two_values", "few_values", "wide_range"])
def test_select_ties_and_ranges(case, select_work):
    """Score rows with every key equal (no radix pass at all), two or a few
    distinct values (ties straddling the k-th place) and a wide exponent
    range (every pass): kept lists bit-exact."""
    w = TINY.with_(grid=(2, 20, 64), head_dim=128)  # 2560 tokens, 40 blocks
    x = qsa_gen.make_qkv(w)
    rng = np.random.default_rng(3)
    kv = oracle.bf16_to_f64(x["k"])
    if case == "all_equal":
        x["q"][:] = 0  # every score 0
    elif case == "two_values":
        blk = np.arange(w.seq_len) // 64
        kv[:] = np.where((blk % 2 == 0)[None, None, :, None], 1.0, 2.0)
        x["k"] = oracle.f64_to_bf16(kv)
    elif case == "few_values":
        blk = np.arange(w.seq_len) // 64
        kv[:] = ((blk % 3) + 1.0)[None, None, :, None]
        x["k"] = oracle.f64_to_bf16(kv)
    else:
        scale = 2.0 ** rng.integers(-12, 12, size=w.seq_len // 64)
        kv *= np.repeat(scale, 64)[None, None, :, None]
        x["k"] = oracle.f64_to_bf16(kv)
    for topk, band in [(1, (0,)), (7, ()), (13, (0, 3)), (39, (0,))]:
        o = oracle_front(x, w, topk=topk, band=band)
        g = _gpu_front(x, w, topk, band, o["kmax"], select_work)
        assert np.array_equal(g["cnt"].cpu().numpy(), o["cnt"]), (case, topk, band)
        assert np.array_equal(g["idx"].cpu().numpy(), o["idx"]), (case, topk, band)


def test_attention_edges():
    w, x, o, g = _setup("tail64_d128")
    v = dev_bf16(x["v"])
    idx, cnt = g["idx"].clone(), g["cnt"].clone()
    cnt[0, 0, 1] = 0            # an empty row outputs zeros
    idx[0, 1, 2, 0] = -1        # entries outside [0, nb) are skipped
    idx[0, 1, 3, 0] = 10 ** 6
    out = host_f64(B.qsa_sparse_attn(g["qc"], g["qs"], g["kc"], g["ks"], v, idx, cnt, w.block))
    assert np.all(out[0, 0, 64:128] == 0)
    oi, oc = o["idx"].copy(), o["cnt"].copy()
    oc[0, 0, 1] = 0
    for (h, i) in [(1, 2), (1, 3)]:
        lst = [j for j in oi[0, h, i, 1:oc[0, h, i]]]
        oi[0, h, i] = -1
        oi[0, h, i, :len(lst)] = lst
        oc[0, h, i] = len(lst)
    want = _oracle_attn(o, x, w, (oi, oc))
    assert_close(out, want, what="edges")


@pytest.mark.parametrize("L,bs,D", [(1, 64, 128), (37, 64, 64), (64, 64, 128), (100, 128, 128),
                                    (129, 128, 64)])
def test_short_sequences(L, bs, D):
    """Sequences of one block or less (a single token included), and one full
    block plus one token, through the whole path: front end bit-exact; sparse
    and refresh outputs against the oracle; the ordered entry points give the
    same bits."""
    w = TINY.with_(grid=(1, 1, L), block=bs, head_dim=D)
    x = qsa_gen.make_qkv(w)
    o = oracle_front(x, w, topk=1, band=(0,))
    g = _gpu_front(x, w, o["topk"], o["band"], o["kmax"])
    for gk, ok in (("qc", "qc"), ("kc", "kc"), ("qp", "pq"), ("kp", "pk"), ("idx", "idx"),
                   ("cnt", "cnt")):
        assert np.array_equal(g[gk].cpu().numpy(), o[ok]), gk
    assert np.array_equal(g["qs"].cpu().numpy().view(np.uint32), o["sq"].view(np.uint32))
    v = dev_bf16(x["v"])
    out = B.qsa_sparse_attn(g["qc"], g["qs"], g["kc"], g["ks"], v, g["idx"], g["cnt"], w.block)
    assert_close(host_f64(out), _oracle_attn(o, x, w), what=f"L={L} sparse")
    order = B.qsa_order_query_blocks(g["idx"], g["cnt"], w.seq_len, w.block, w.head_dim)
    out_o = B.qsa_sparse_attn_ordered(g["qc"], g["qs"], g["kc"], g["ks"], v, g["idx"], g["cnt"],
                                      order, w.block)
    assert np.array_equal(host_bits(out), host_bits(out_o))
    o_full = _oracle_attn(o, x, w, oracle.full_kept_lists(w.batch, w.heads, w.n_blocks))
    rng = np.random.default_rng(L)
    r_prev = dev_bf16(qsa_gen.f32_to_bf16_bits(
        rng.standard_normal(x["v"].shape).astype(np.float32) * 0.02))
    for has_prev in (0, 1):
        res = []
        for od in (None, order):
            r = r_prev.clone()
            dr = torch.zeros_like(v)
            full = B.qsa_full_attn_residual(g["qc"], g["qs"], g["kc"], g["ks"], v, g["idx"],
                                            g["cnt"], w.block, r, dr, has_prev, order=od)
            res.append([host_bits(t) for t in (full, r, dr)])
        assert_close(oracle.bf16_to_f64(res[0][0]), o_full, what=f"L={L} full")
        for a_, b_ in zip(*res):
            assert np.array_equal(a_, b_)


def _boost_block(bits, h, blk, block, gain):
    """bf16 bits with the rows of key block blk of head h scaled by gain."""
    x = oracle.bf16_to_f64(bits)
    x[:, h, blk * block:(blk + 1) * block] *= gain
    return qsa_gen.f32_to_bf16_bits(x.astype(np.float32))


@pytest.mark.parametrize("D", [128, 64])
def test_running_max_moves_mid_walk(D):
    """Rows whose first kept tile has far smaller logits than a later one: the
    walk's running max (taken on the first tile) must move up, rescaling the
    state, when a later tile holds a P above 2^64.  Head 0 has a large middle
    block, head 1 a large ragged last block (the masked tail tile).  Sparse
    step with all blocks and with the selected blocks, refresh step (the
    large block falls in the kept or in the complement phase), against the
    oracle."""
    w = TINY.with_(grid=(1, 10, 30), block=64, head_dim=D, heads=2)  # 300 tokens, 5 blocks
    x = dict(qsa_gen.make_qkv(w))
    x["k"] = _boost_block(x["k"], 0, 2, w.block, 60.0)
    x["k"] = _boost_block(x["k"], 1, w.n_blocks - 1, w.block, 60.0)
    o = oracle_front(x, w, topk=1, band=(0,))
    # the case is what it claims: in log2 units the large block's logits exceed
    # block 0's by more than 64 for most query rows of both heads
    sm = oracle.default_sm_scale(D) * np.log2(np.e)
    qf = o["qc"].astype(np.float64) * np.repeat(o["sq"], w.block, axis=2)[:, :, :w.seq_len, None]
    kf = o["kc"].astype(np.float64) * np.repeat(o["sk"], w.block, axis=2)[:, :, :w.seq_len, None]
    z = np.einsum("bhid,bhjd->bhij", qf, kf) * sm
    for h, blk in ((0, 2), (1, w.n_blocks - 1)):
        big = z[0, h, :, blk * w.block:(blk + 1) * w.block].max(axis=1)
        first = z[0, h, :, :w.block].max(axis=1)
        assert np.mean(big - first > 64) > 0.9, h
    g = _gpu_front(x, w, o["topk"], o["band"], o["kmax"])
    for gk, ok in (("qc", "qc"), ("kc", "kc"), ("idx", "idx"), ("cnt", "cnt")):
        assert np.array_equal(g[gk].cpu().numpy(), o[ok]), gk
    v = dev_bf16(x["v"])
    full_lists = oracle.full_kept_lists(w.batch, w.heads, w.n_blocks)
    o_full = _oracle_attn(o, x, w, full_lists)
    fi, fc = (torch.from_numpy(a).cuda() for a in full_lists)
    out = B.qsa_sparse_attn(g["qc"], g["qs"], g["kc"], g["ks"], v, fi, fc, w.block)
    assert_close(host_f64(out), o_full, what=f"D={D} all blocks")
    out = B.qsa_sparse_attn(g["qc"], g["qs"], g["kc"], g["ks"], v, g["idx"], g["cnt"], w.block)
    o_sp = _oracle_attn(o, x, w)
    assert_close(host_f64(out), o_sp, what=f"D={D} selected blocks")
    r, dr = torch.zeros_like(v), torch.zeros_like(v)
    full = B.qsa_full_attn_residual(g["qc"], g["qs"], g["kc"], g["ks"], v, g["idx"], g["cnt"],
                                    w.block, r, dr, 0)
    assert_close(host_f64(full), o_full, what=f"D={D} refresh full")
    err = host_f64(r) - (o_full - o_sp)
    assert np.linalg.norm(err) / np.linalg.norm(o_full) <= 5e-3
    assert np.max(np.abs(err)) <= 2e-2


def _messy_lists(w, seed):
    """Kept lists with repeats, entries outside [0, nb) and shuffled order."""
    nb = w.n_blocks
    rng = np.random.default_rng(seed)
    kmax = 12
    idx = np.full((w.batch, w.heads, nb, kmax), -1, np.int32)
    cnt = np.zeros((w.batch, w.heads, nb), np.int32)
    for b in range(w.batch):
        for h in range(w.heads):
            for i in range(nb):
                base = list(rng.choice(nb, size=int(rng.integers(1, min(nb, 5) + 1)),
                                       replace=False))
                lst = base + [base[-1], -7, nb, 2 ** 30]
                rng.shuffle(lst)
                idx[b, h, i, :len(lst)] = lst
                cnt[b, h, i] = len(lst)
    return idx, cnt, kmax


@pytest.mark.parametrize("name", ["tail64_d128", "batch2_h3", "d64_b128"])
def test_kept_lists_are_sets(name):
    """Both kernels take kept(i) as the set of its valid entries."""
    w, x, o, g = _setup(name)
    v = dev_bf16(x["v"])
    idx, cnt, kmax = _messy_lists(w, 11)
    di = torch.from_numpy(idx).cuda()
    dc = torch.from_numpy(cnt).cuda()
    out = B.qsa_sparse_attn(g["qc"], g["qs"], g["kc"], g["ks"], v, di, dc, w.block)
    want = _oracle_attn(o, x, w, (idx, cnt))
    assert_close(host_f64(out), want, what=f"{name} messy sparse")
    r = torch.zeros_like(v)
    dr = torch.zeros_like(v)
    full = B.qsa_full_attn_residual(g["qc"], g["qs"], g["kc"], g["ks"], v, di, dc, w.block, r,
                                    dr, 0)
    o_full = _oracle_attn(o, x, w, oracle.full_kept_lists(w.batch, w.heads, w.n_blocks))
    assert_close(host_f64(full), o_full, what=f"{name} messy full")
    rho = o_full - want
    err = host_f64(r) - rho
    assert np.linalg.norm(err) / np.linalg.norm(o_full) <= 5e-3


def test_deterministic():
    w, x, o, g = _setup("batch2_h3")
    v = dev_bf16(x["v"])
    a = host_bits(B.qsa_sparse_attn(g["qc"], g["qs"], g["kc"], g["ks"], v, g["idx"], g["cnt"],
                                    w.block))
    b = host_bits(B.qsa_sparse_attn(g["qc"], g["qs"], g["kc"], g["ks"], v, g["idx"], g["cnt"],
                                    w.block))
    assert np.array_equal(a, b)


def _assert_permutation(order, nb):
    srt, _ = torch.sort(order.long(), dim=-1)
    assert bool((srt == torch.arange(nb, device=order.device)).all()), "order is not a permutation"


@pytest.mark.parametrize("name", list(CFGS))
def test_ordered_attention_is_identical(name):
    """Processing the query blocks in the computed order changes no output bit."""
    w, x, o, g = _setup(name)
    v = dev_bf16(x["v"])
    order = B.qsa_order_query_blocks(g["idx"], g["cnt"], w.seq_len, w.block, w.head_dim)
    again = B.qsa_order_query_blocks(g["idx"], g["cnt"], w.seq_len, w.block, w.head_dim)
    torch.cuda.synchronize()
    _assert_permutation(order, w.n_blocks)
    assert torch.equal(order, again), "order is not deterministic"
    rng = np.random.default_rng(4)
    r = dev_bf16(qsa_gen.f32_to_bf16_bits(rng.standard_normal(x["v"].shape).astype(np.float32)))
    for rr in (None, r):
        a = B.qsa_sparse_attn(g["qc"], g["qs"], g["kc"], g["ks"], v, g["idx"], g["cnt"], w.block,
                              r=rr, dr=rr)
        b = B.qsa_sparse_attn_ordered(g["qc"], g["qs"], g["kc"], g["ks"], v, g["idx"], g["cnt"],
                                      order, w.block, r=rr, dr=rr)
        assert np.array_equal(host_bits(a), host_bits(b))
    # a reversed order, and kept lists with repeats / outside entries / any order
    rev = torch.flip(order, dims=[-1]).contiguous()
    c = B.qsa_sparse_attn_ordered(g["qc"], g["qs"], g["kc"], g["ks"], v, g["idx"], g["cnt"], rev,
                                  w.block)
    plain = B.qsa_sparse_attn(g["qc"], g["qs"], g["kc"], g["ks"], v, g["idx"], g["cnt"], w.block)
    assert np.array_equal(host_bits(plain), host_bits(c))
    idx, cnt, kmax = _messy_lists(w, 3)
    di, dc = torch.from_numpy(idx).cuda(), torch.from_numpy(cnt).cuda()
    om = B.qsa_order_query_blocks(di, dc, w.seq_len, w.block, w.head_dim)
    _assert_permutation(om, w.n_blocks)
    a = B.qsa_sparse_attn(g["qc"], g["qs"], g["kc"], g["ks"], v, di, dc, w.block)
    b = B.qsa_sparse_attn_ordered(g["qc"], g["qs"], g["kc"], g["ks"], v, di, dc, om, w.block)
    assert np.array_equal(host_bits(a), host_bits(b))


@pytest.mark.parametrize("name", list(CFGS))
@pytest.mark.parametrize("has_prev", [0, 1])
def test_ordered_refresh_is_identical(name, has_prev):
    """A refresh step over the query blocks in the computed order (and in its
    reverse) writes the same full output, r and dr, bit for bit."""
    w, x, o, g = _setup(name)
    v = dev_bf16(x["v"])
    order = B.qsa_order_query_blocks(g["idx"], g["cnt"], w.seq_len, w.block, w.head_dim)
    rev = torch.flip(order, dims=[-1]).contiguous()
    rng = np.random.default_rng(5)
    r_prev = dev_bf16(qsa_gen.f32_to_bf16_bits(
        rng.standard_normal(x["v"].shape).astype(np.float32) * 0.02))
    outs = []
    for od in (None, order, rev):
        r = r_prev.clone()
        dr = torch.zeros_like(v)
        full = B.qsa_full_attn_residual(g["qc"], g["qs"], g["kc"], g["ks"], v, g["idx"], g["cnt"],
                                        w.block, r, dr, has_prev, order=od)
        torch.cuda.synchronize()
        outs.append([host_bits(t) for t in (full, r, dr)])
    for got in outs[1:]:
        for a, b, nm in zip(outs[0], got, ("full", "r", "dr")):
            assert np.array_equal(a, b), f"{name} has_prev={has_prev}: {nm} differs"


def _match(ov):
    """Mutual-best pairing (ov = block overlaps, saturated at 255): rounds in
    which every single block picks the single block of largest overlap (ties:
    the lower index) and two blocks that pick each other pair up; leftovers
    pair in block order.  Returns partner[b] (-1: the single block)."""
    n = len(ov)
    ov = np.minimum(ov, 255)
    partner = -np.ones(n, np.int64)
    for _ in range(48):
        alive = partner < 0
        best = -np.ones(n, np.int64)
        for t in np.nonzero(alive)[0]:
            cand = np.nonzero(alive)[0]
            cand = cand[cand != t]
            if len(cand):
                best[t] = cand[int(np.argmax(ov[t, cand]))]  # first maximum: lower index
        made = False
        for t in range(n):
            u = best[t]
            if alive[t] and u > t and best[u] == t:
                partner[t], partner[u] = u, t
                made = True
        if not made:
            break
    pending = -1
    for b in range(n):
        if partner[b] >= 0:
            continue
        if pending < 0:
            pending = b
        else:
            partner[pending], partner[b] = b, pending
            pending = -1
    return partner


def _chain(S):
    """Greedy chain from item 0 to the unused item of largest overlap (rows of
    S are signatures), ties to the lowest index."""
    M = S.astype(np.int64) @ S.T.astype(np.int64)
    n = len(S)
    used = np.zeros(n, bool)
    cur, seq = 0, [0]
    used[0] = True
    for _ in range(n - 1):
        cur = int(np.argmax(np.where(used, -1, M[cur])))  # first maximum: lowest index
        used[cur] = True
        seq.append(cur)
    return seq


def _reference_order(idx, cnt, nb, chunk=256, bits=256):
    """The documented processing order, restated in numpy: per chunk of 256
    blocks, the blocks paired by mutual best partners on the overlaps of
    256-bit signatures (bit j mod 256 for key block j), the pairs (indexed by
    their lower block) ordered by a greedy chain over the signatures of their
    unions, an odd chunk's single block last; chunks of at most two blocks
    keep their order."""
    Bn, H = cnt.shape[:2]
    out = np.zeros((Bn, H, nb), np.int64)
    for b in range(Bn):
        for h in range(H):
            sig = np.zeros((nb, bits), bool)
            for i in range(nb):
                js = np.array([j for j in idx[b, h, i, :cnt[b, h, i]] if 0 <= j < nb],
                              dtype=np.int64)
                sig[i, js % bits] = True
            for c0 in range(0, nb, chunk):
                n = min(chunk, nb - c0)
                if n <= 2:
                    out[b, h, c0:c0 + n] = c0 + np.arange(n)
                    continue
                S = sig[c0:c0 + n].astype(np.int64)
                partner = _match(S @ S.T)
                pairs = [(t, int(partner[t])) for t in range(n) if partner[t] > t]
                seq = []
                for k in _chain(np.array([S[p] | S[q] for p, q in pairs])):
                    seq += list(pairs[k])
                seq += [t for t in range(n) if partner[t] < 0]
                out[b, h, c0:c0 + n] = c0 + np.array(seq)
    return out


@pytest.mark.parametrize("nb", [3, 257, 3000])
def test_order_chunks(nb):
    """The order permutes each chunk of 256 consecutive blocks within itself,
    is the documented re-paired chain, and changes no output bit."""
    D, blk, H = 64, 64, 2
    L = nb * blk - 17  # a ragged last block
    gen = torch.Generator(device="cuda").manual_seed(nb)
    q = torch.randn((1, H, L, D), generator=gen, device="cuda").to(torch.bfloat16)
    k = torch.randn((1, H, L, D), generator=gen, device="cuda").to(torch.bfloat16)
    v = torch.randn((1, H, L, D), generator=gen, device="cuda").to(torch.bfloat16)
    qc, qs, qp = B.qsa_quantize(q, blk)
    kc, ks, kp = B.qsa_quantize(k, blk)
    topk = min(3, nb)
    idx, cnt = B.qsa_select_blocks(qp, qs, kp, ks, L, blk, topk, (0,), min(nb, topk + 1))
    order = B.qsa_order_query_blocks(idx, cnt, L, blk, D)
    torch.cuda.synchronize()
    _assert_permutation(order, nb)
    o = order.cpu().numpy()
    for c0 in range(0, nb, 256):
        seg = o[..., c0:c0 + 256]
        assert np.all(np.sort(seg, axis=-1) == np.arange(c0, min(nb, c0 + 256)))
    ref = _reference_order(idx.cpu().numpy(), cnt.cpu().numpy(), nb)
    assert np.array_equal(o, ref), "order differs from the documented greedy chain"
    a = B.qsa_sparse_attn(qc, qs, kc, ks, v, idx, cnt, blk)
    b = B.qsa_sparse_attn_ordered(qc, qs, kc, ks, v, idx, cnt, order, blk)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("name", list(CFGS))
def test_rotated_quantize_bit_exact(name):
    w, _ = CFGS[name]
    x = qsa_gen.make_qkv(w, 0)
    for t in ("q", "k"):
        c, s, p = B.qsa_quantize_rotated(dev_bf16(x[t]), w.block)
        oc, os_, op = oracle.quantize_rotated(x[t], w.block)
        assert np.array_equal(c.cpu().numpy(), oc), t
        assert np.array_equal(s.cpu().numpy().view(np.uint32), os_.view(np.uint32)), t
        assert np.array_equal(p.cpu().numpy(), op), t


@pytest.mark.parametrize("name", ["tiny", "tail64_d128", "tail128_d128", "d64_b128",
                                  "batch2_h3"])
def test_rotated_pipeline_parity(name):
    """Rotated codes through selection and sparse attention with sm_scale / D:
    kept lists bit-exact, outputs within the output tolerance."""
    w, kw = CFGS[name]
    x = qsa_gen.make_qkv(w, 0)
    topk = kw.get("topk", w.topk)
    band = tuple(kw.get("band", w.band))
    kmax = min(w.n_blocks, topk + len(band))
    qc, sq, pq = oracle.quantize_rotated(x["q"], w.block)
    kc, sk, pk = oracle.quantize_rotated(x["k"], w.block)
    idx, cnt = oracle.select_blocks(oracle.block_scores(pq, sq, pk, sk, w.seq_len, w.block),
                                    topk, band, kmax)
    sm = np.float32(oracle.default_sm_scale(w.head_dim) / np.float32(w.head_dim))
    want = oracle.attention(qc, sq, kc, sk, x["v"], idx, cnt, w.block, sm)

    gq = B.qsa_quantize_rotated(dev_bf16(x["q"]), w.block)
    gk = B.qsa_quantize_rotated(dev_bf16(x["k"]), w.block)
    gidx, gcnt = B.qsa_select_blocks(gq[2], gq[1], gk[2], gk[1], w.seq_len, w.block, topk, band,
                                     kmax)
    assert np.array_equal(gcnt.cpu().numpy(), cnt)
    assert np.array_equal(gidx.cpu().numpy(), idx)
    out = B.qsa_sparse_attn(gq[0], gq[1], gk[0], gk[1], dev_bf16(x["v"]), gidx, gcnt, w.block,
                            sm_scale=float(sm))
    assert_close(host_f64(out), want, what=f"{name} rotated sparse")
