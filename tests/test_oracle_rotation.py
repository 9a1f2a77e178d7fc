"""Pins of the oracle's rotated quantisation (Hadamard rotation before the
per-block int8 quantisation; DVD-Quant, gist.science/es/paper/2505.18663,
technical summary §2B, rotated quantisation).

The transform is pinned against an independent construction of the Sylvester
Hadamard matrix (Kronecker powers of [[1, 1], [1, -1]]) with exact integer
arithmetic, against its algebra (H H = D I, dot products scale by D), against
a closed form (a single-channel spike spreads to +-c on every channel), and
against fp64 within a rounding bound.  The quantisation that follows is the
pinned per-block quantisation; for inputs whose rotation is exact it must
equal quantising the exact product.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from tests.exact import round_f32, round_half_even


def sylvester(D):
    h = np.array([[1]], dtype=np.int64)
    while h.shape[0] < D:
        h = np.kron(np.array([[1, 1], [1, -1]], dtype=np.int64), h)
    return h


@pytest.mark.parametrize("D", [2, 8, 64, 128])
def test_fwht_equals_sylvester_product_exactly(D):
    rng = np.random.default_rng(D)
    x = rng.integers(-1000, 1000, size=(5, 3, D))
    got = oracle.fwht(x.astype(np.float32))
    want = x @ sylvester(D)  # int64, exact
    assert np.array_equal(got.astype(np.int64), want)
    assert np.all(np.abs(want) < 2 ** 24)  # every partial sum exact in fp32


@pytest.mark.parametrize("D", [64, 128])
def test_fwht_algebra(D):
    rng = np.random.default_rng(7)
    x = rng.integers(-300, 300, size=(4, D)).astype(np.float32)
    # H_D H_D = D I
    assert np.array_equal(oracle.fwht(oracle.fwht(x)), np.float32(D) * x)
    # dot products of rotated rows scale by D
    q, k = x[0], x[1]
    assert float(oracle.fwht(q) @ oracle.fwht(k)) == D * float(q @ k)


@pytest.mark.parametrize("j", [0, 5, 127])
def test_spike_spreads_to_every_channel(j):
    D, c = 128, np.float32(-3.5)
    x = np.zeros((1, D), np.float32)
    x[0, j] = c
    y = oracle.fwht(x)
    assert np.all(np.abs(y) == abs(c))
    assert np.array_equal(np.sign(y[0]), np.sign(c) * sylvester(D)[j])


def test_fwht_close_to_fp64_for_bf16_inputs():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((64, 128)).astype(np.float32) * 4
    x = oracle.bf16_to_f64(oracle.f64_to_bf16(x)).astype(np.float32)  # bf16 values
    got = oracle.fwht(x).astype(np.float64)
    want = x.astype(np.float64) @ sylvester(128)
    # 7 stages, each one fp32 rounding of a partial sum bounded by sum |x|
    bound = 7 * 2.0 ** -24 * np.abs(x).astype(np.float64).sum(axis=1, keepdims=True)
    assert np.all(np.abs(got - want) <= bound)


def test_rotated_quantisation_of_exactly_rotatable_rows():
    """Integer rows rotate exactly in fp32, so the result must be the per-block
    quantisation of the exact product x H, computed here with exact rationals:
    scale = fl32(amax / 127), code = round-half-even(fl32(y / scale))."""
    rng = np.random.default_rng(11)
    B, H, L, D, block = 1, 2, 150, 64, 64
    xi = rng.integers(-200, 200, size=(B, H, L, D))
    bits = oracle.f64_to_bf16(xi.astype(np.float64))  # small integers are exact in bf16
    codes, scales, pooled = oracle.quantize_rotated(bits, block)
    exact = xi @ sylvester(D)  # int64, |.| < 2^14
    for h in range(H):
        for i, (t0, t1) in enumerate(oracle.block_bounds(L, block)):
            y = exact[0, h, t0:t1]
            s = round_f32(Fraction(int(np.abs(y).max()), 127))
            assert scales[0, h, i] == np.float32(s)
            want = np.array([[max(-127, min(127, round_half_even(Fraction(
                round_f32(Fraction(int(v)) / Fraction(s)))))) for v in row] for row in y])
            assert np.array_equal(codes[0, h, t0:t1], want)
            assert np.array_equal(pooled[0, h, i], want.sum(axis=0))


def test_rotation_spreads_planted_outlier_channels():
    """On rows with a few x10 channels (the workload's outliers) the rotated
    block amax is far below the unrotated one relative to the row norm, so
    the int8 grid is finer: fewer small values collapse to code 0."""
    rng = np.random.default_rng(5)
    x = rng.standard_normal((1, 1, 64, 128)).astype(np.float32)
    x[..., [3, 40, 99]] *= 10
    bits = oracle.f64_to_bf16(x.astype(np.float64))
    c0, s0, _ = oracle.quantize(bits, 64)
    c1, s1, _ = oracle.quantize_rotated(bits, 64)
    assert np.mean(c1 == 0) < np.mean(c0 == 0)
    # relative error of the dequantised rows against the exact rotation
    xr = oracle.bf16_to_f64(bits)[0, 0]
    e0 = np.linalg.norm(c0[0, 0] * np.float64(s0[0, 0, 0]) - xr) / np.linalg.norm(xr)
    yr = xr @ sylvester(128)
    e1 = np.linalg.norm(c1[0, 0] * np.float64(s1[0, 0, 0]) - yr) / np.linalg.norm(yr)
    assert e1 < e0


def test_rotated_attention_is_closer_to_exact_attention():
    """With the workload's outlier channels (x10), attention on rotated codes
    (sm_scale / D) is closer to exact fp64 softmax attention of the bf16
    inputs than attention on unrotated codes: the effect the rotation is for.
    Full kept lists, so the selection plays no part."""
    import qsa_gen
    w = qsa_gen.get_workload("tiny").with_(grid=(1, 6, 30), block=64, head_dim=128,
                                           outlier_channels=3, outlier_gain=10.0)
    x = qsa_gen.make_qkv(w, 0)
    B_, H_, L, D = x["q"].shape
    nb = (L + w.block - 1) // w.block
    idx, cnt = oracle.full_kept_lists(B_, H_, nb)
    sm = oracle.default_sm_scale(D)
    q, k, v = (oracle.bf16_to_f64(x[t]) for t in "qkv")
    z = np.einsum("bhld,bhmd->bhlm", q, k) * np.float64(sm)
    p = np.exp(z - z.max(-1, keepdims=True))
    exact = np.einsum("bhlm,bhmd->bhld", p / p.sum(-1, keepdims=True), v)
    qc, sq, _ = oracle.quantize(x["q"], w.block)
    kc, sk, _ = oracle.quantize(x["k"], w.block)
    plain = oracle.attention(qc, sq, kc, sk, x["v"], idx, cnt, w.block, sm)
    qc, sq, _ = oracle.quantize_rotated(x["q"], w.block)
    kc, sk, _ = oracle.quantize_rotated(x["k"], w.block)
    rot = oracle.attention(qc, sq, kc, sk, x["v"], idx, cnt, w.block, np.float32(sm / D))
    e_plain = np.linalg.norm(plain - exact) / np.linalg.norm(exact)
    e_rot = np.linalg.norm(rot - exact) / np.linalg.norm(exact)
    assert e_rot < 0.5 * e_plain, (e_rot, e_plain)
