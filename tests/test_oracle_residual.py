"""Pins of the oracle's step 4: second-order sparse attention reparameterisation.

QuantSparse (gist.science/es/paper/2509.23681, Resumen técnico §2B;
gist.science/ko/paper/2509.23681 §2.2): the first-order residual is full minus
sparse attention, the second-order residual its change between consecutive
residuals, and a cache of both corrects sparse steps.  Pinned by closed forms
(density 1 gives zero residuals; unchanged inputs leave only the bf16 rounding
of r in the second-order residual), exactly representable hand values, a
linearly drifting residual, and bf16 rounding checked
against exact rational rounding and torch's conversion.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import qsa_gen
from tests.exact import round_bf16


def _outputs(w, step, dense=False):
    x = qsa_gen.make_qkv(w, step)
    qc, sq, pq = oracle.quantize(x["q"], w.block)
    kc, sk, pk = oracle.quantize(x["k"], w.block)
    B, H, L, D = qc.shape
    sm = oracle.default_sm_scale(D)
    if dense:
        idx, cnt = oracle.full_kept_lists(B, H, w.n_blocks)
    else:
        sc = oracle.block_scores(pq, sq, pk, sk, L, w.block)
        idx, cnt = oracle.select_blocks(sc, w.topk, w.band, w.kmax)
    fidx, fcnt = oracle.full_kept_lists(B, H, w.n_blocks)
    o_sp = oracle.attention(qc, sq, kc, sk, x["v"], idx, cnt, w.block, sm)
    o_full = oracle.attention(qc, sq, kc, sk, x["v"], fidx, fcnt, w.block, sm)
    return o_full, o_sp


def test_f64_to_bf16_against_exact_rounding():
    rng = np.random.default_rng(5)
    vals = np.concatenate([
        rng.standard_normal(2000) * np.exp2(rng.integers(-140, 130, 2000)),
        np.array([0.0, -0.0, 1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 2.0 ** -133, 2.0 ** -134,
                  3 * 2.0 ** -135, 2.0 ** -126 * (1 - 2 ** -9), 3.3895313892515355e38,
                  3.3961775292304e38, -1.5 * 2.0 ** -133]),
    ])
    got = oracle.f64_to_bf16(vals)
    for v, g in zip(vals, got):
        want = round_bf16(Fraction(float(v)))
        gf = float(oracle.bf16_to_f64(np.array([g], np.uint16))[0])
        if np.isinf(want):
            assert np.isinf(gf) and np.sign(gf) == np.sign(want), v
        else:
            assert gf == want, (v, gf, want)
    # values exact in fp32: torch's conversion (a library routine) agrees bit for bit
    with np.errstate(over="ignore"):
        v32 = vals.astype(np.float32)
    mask = np.isfinite(v32) & (v32.astype(np.float64) == vals)
    tb = torch.from_numpy(v32[mask]).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(tb, got[mask])


def test_refresh_and_sparse_step_hand_values():
    # exactly representable values: rho = 0.75 - 0.25 = 0.5; r_prev = 0.375 -> dr = 0.125
    st = oracle.ResidualState((1, 1, 1, 2))
    o_full = np.array([[[[0.75, -1.0]]]])
    o_sp = np.array([[[[0.25, -1.5]]]])
    out = oracle.refresh_step(st, o_full, o_sp)
    assert np.array_equal(out, o_full)
    assert oracle.bf16_to_f64(st.r).reshape(-1).tolist() == [0.5, 0.5]
    assert np.all(st.dr == 0)                       # first refresh: dr = 0
    st.r = qsa_gen.f32_to_bf16_bits(np.array([[[[0.375, 0.5]]]], np.float32))
    oracle.refresh_step(st, o_full, o_sp)
    assert oracle.bf16_to_f64(st.dr).reshape(-1).tolist() == [0.125, 0.0]
    assert oracle.bf16_to_f64(st.r).reshape(-1).tolist() == [0.5, 0.5]
    s2 = oracle.sparse_step(st, np.array([[[[1.0, 2.0]]]]))
    assert s2.reshape(-1).tolist() == [1.0 + 0.5 + 0.125, 2.0 + 0.5]
    s1 = oracle.sparse_step(st, np.array([[[[1.0, 2.0]]]]), order=1)
    assert s1.reshape(-1).tolist() == [1.5, 2.5]


def test_sparse_step_needs_a_refresh():
    st = oracle.ResidualState((1, 1, 4, 4))
    with pytest.raises(RuntimeError):
        oracle.sparse_step(st, np.zeros((1, 1, 4, 4)))


def test_density_one_gives_zero_residuals():
    w = qsa_gen.get_workload("tiny")
    o_full, o_sp = _outputs(w, 0, dense=True)
    np.testing.assert_array_equal(o_full, o_sp)
    st = oracle.ResidualState(o_full.shape)
    oracle.refresh_step(st, o_full, o_sp)
    assert np.all(oracle.bf16_to_f64(st.r) == 0) and np.all(st.dr == 0)
    np.testing.assert_array_equal(oracle.sparse_step(st, o_sp), o_sp)


def test_unchanged_inputs_leave_only_rounding_in_second_order_residual():
    # The cache holds r in bf16, so with unchanged inputs the next refresh sees
    # dr = bf16(rho - bf16(rho)): only the rounding error of r, at most half a
    # bf16 ulp of rho; r + dr then reproduces rho to about 16 bits.
    w = qsa_gen.get_workload("tiny")
    o_full, o_sp = _outputs(w, 0)
    assert np.abs(o_full - o_sp).max() > 1e-3           # sparsity changes the output
    st = oracle.ResidualState(o_full.shape)
    oracle.refresh_step(st, o_full, o_sp)
    r1 = st.r.copy()
    oracle.refresh_step(st, o_full, o_sp)               # same inputs at the next refresh
    rho = o_full - o_sp
    assert np.array_equal(st.r, r1)
    dr = oracle.bf16_to_f64(st.dr)
    assert np.all(np.abs(dr) <= np.abs(rho) * 2.0 ** -8 + 2.0 ** -134)
    out = oracle.sparse_step(st, o_sp)
    assert np.all(np.abs(out - o_full) <= np.abs(rho) * 2.0 ** -15 + 2.0 ** -133)
    out1 = oracle.sparse_step(st, o_sp, order=1)
    assert np.abs(out1 - o_full).max() > np.abs(out - o_full).max()


def test_second_order_tracks_linear_drift_of_residual():
    # If the residual changes by the same amount between refreshes, r + dr
    # extrapolates it exactly (up to bf16 rounding): the second-order reading.
    st = oracle.ResidualState((1, 1, 1, 3))
    o_sp = np.zeros((1, 1, 1, 3))
    for t in range(3):
        oracle.refresh_step(st, np.array([[[[0.5 + 0.25 * t, -1.0 - 0.125 * t, 2.0]]]]), o_sp)
    nxt = oracle.sparse_step(st, o_sp)
    np.testing.assert_array_equal(nxt.reshape(-1), [0.5 + 0.25 * 3, -1.0 - 0.125 * 3, 2.0])
