"""Pins of the oracle's step 1: per-block symmetric int8 quantisation.

The pages fix only "8-bit activations" (QuantSparse, gist.science/es/paper/
2509.23681, Resumen técnico §1 and §4); the scale/rounding reading is the
oracle's R2.  These tests check the oracle against exact rational arithmetic
(IEEE rounding written out from its definition), closed forms and invariants.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import qsa_gen
from tests.exact import round_f32, round_half_even


def _bits(x):
    return qsa_gen.f32_to_bf16_bits(np.asarray(x, np.float32))


def _expected_code(x: float, amax: float) -> tuple:
    s = round_f32(Fraction(amax) / 127)
    if s == 0:
        return 0, 0.0
    q = round_f32(Fraction(x) / Fraction(s))
    return max(-127, min(127, round_half_even(Fraction(q)))), s


def test_constant_block_closed_form():
    # A block of one constant c: amax = |c|, codes = 127 * sign(c), scale = fl32(|c|/127).
    for c in (1.0, -0.5, 2.0, 0.25, 3.140625, -1e-3, 7.5e4):
        cb = float(qsa_gen.bf16_bits_to_f32(_bits([c]))[0])
        x = np.full((1, 1, 64, 16), cb, np.float32)
        codes, scales, pooled = oracle.quantize(_bits(x), 64)
        assert np.all(codes == (127 if cb > 0 else -127))
        assert scales[0, 0, 0] == np.float32(round_f32(Fraction(abs(cb)) / 127))
        assert np.all(pooled == 64 * (127 if cb > 0 else -127))


def test_half_integer_ties_round_to_even():
    # amax = 127 gives scale exactly 1.0, so x/scale = x and ties are visible.
    xs = np.array([127.0, 2.5, 3.5, -2.5, -3.5, 0.5, 1.5, 126.5, -126.5, 0.0], np.float32)
    codes, scales, _ = oracle.quantize(_bits(xs.reshape(1, 1, 1, -1)), 64)
    assert scales[0, 0, 0] == np.float32(1.0)
    assert codes.reshape(-1).tolist() == [127, 2, 4, -2, -4, 0, 2, 126, -126, 0]


def test_quantize_map_against_exact_rounding():
    # Random (x, amax) bf16 pairs over a wide exponent range, each block one token
    # holding amax in channel 0; the code of every x must equal the exact
    # round-half-even of the correctly rounded fp32 quotient.
    rng = np.random.default_rng(1234)
    nblk, D = 300, 33
    amax = np.abs(rng.standard_normal(nblk)) * np.exp2(rng.integers(-30, 30, nblk))
    amax = qsa_gen.bf16_bits_to_f32(_bits(amax))
    x = rng.uniform(-1, 1, (nblk, D - 1)) * amax[:, None]
    x = qsa_gen.bf16_bits_to_f32(_bits(x))
    x = np.clip(x, -amax[:, None], amax[:, None])
    blk = np.concatenate([amax[:, None], x], axis=1).astype(np.float32)
    # one block per token: block size 1 keeps each token's amax separate
    codes, scales, pooled = oracle.quantize(_bits(blk[None, None]), 1)
    for i in range(nblk):
        for d in range(D):
            c, s = _expected_code(float(blk[i, d]), float(blk[i, 0]))
            assert codes[0, 0, i, d] == c, (i, d, blk[i, d], blk[i, 0])
        assert scales[0, 0, i] == np.float32(s)
        assert pooled[0, 0, i].tolist() == [int(v) for v in codes[0, 0, i]]


def test_tiny_scale_subnormal_path():
    # amax a bf16 subnormal: fp32 scale is subnormal too; the map must still follow
    # exact rounding (no flush to zero).
    tiny = np.float32(2.0 ** -130)
    xs = np.array([tiny, tiny / 2, -tiny / 4, tiny * 0.75], np.float32)
    codes, scales, _ = oracle.quantize(_bits(xs.reshape(1, 1, 1, -1)), 64)
    blk = qsa_gen.bf16_bits_to_f32(_bits(xs))
    for d in range(4):
        c, s = _expected_code(float(blk[d]), float(blk[0]))
        assert codes[0, 0, 0, d] == c
    assert scales[0, 0, 0] == np.float32(round_f32(Fraction(float(blk[0])) / 127))
    assert scales[0, 0, 0] > 0


def test_zero_block_has_zero_scale_and_codes():
    x = np.zeros((1, 1, 128, 8), np.float32)
    x[0, 0, 64:] = 1.0
    codes, scales, pooled = oracle.quantize(_bits(x), 64)
    assert scales[0, 0, 0] == 0 and np.all(codes[0, 0, :64] == 0) and np.all(pooled[0, 0, 0] == 0)
    assert np.all(codes[0, 0, 64:] == 127)


@pytest.mark.parametrize("L,block", [(100, 64), (128, 64), (300, 128), (16, 64)])
def test_invariants_and_tail_blocks(L, block):
    w = qsa_gen.get_workload("tiny").with_(grid=(1, 1, L), block=block, head_dim=64)
    x = qsa_gen.make_qkv(w)["q"]
    codes, scales, pooled = oracle.quantize(x, block)
    xf = qsa_gen.bf16_bits_to_f32(x).astype(np.float64)
    for i, (t0, t1) in enumerate(oracle.block_bounds(L, block)):
        c = codes[0, 0, t0:t1].astype(np.int64)
        s = float(scales[0, 0, i])
        assert np.abs(c).max() == 127                       # amax maps to 127
        assert np.all(np.abs(c) <= 127)
        # reconstruction: |x - code * s| <= s * (1/2 + 127 * 2**-24)
        err = np.abs(xf[0, 0, t0:t1] - c * s)
        assert np.all(err <= s * (0.5 + 127 * 2.0 ** -24))
        # pooled sums over valid tokens only, exact (Python ints)
        for d in range(0, 64, 7):
            assert pooled[0, 0, i, d] == sum(int(v) for v in c[:, d])
        # a tail block is quantised exactly as if it stood alone
        alone = oracle.quantize(x[:, :, t0:t1], block)
        assert np.array_equal(alone[0], codes[:, :, t0:t1])
        assert alone[1][0, 0, 0] == scales[0, 0, i]
