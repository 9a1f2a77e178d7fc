"""Pins of the oracle's SVD projection of the second-order residual.

QuantSparse (gist.science/es/paper/2509.23681, technical summary §2B;
gist.science/ko/paper/2509.23681, §2.2): the second-order residual is
projected onto its dominant principal components.  The oracle takes, per
(batch, head), the best rank-r approximation X V_r V_r^T from the
eigenvectors of X^T X.  It is pinned here against a different route to the
same object -- the truncated singular value decomposition of X
(Eckart-Young) -- and against hand examples, closed forms and invariants.
"""
import numpy as np
import pytest

import oracle


def _bits(x):
    return oracle.f64_to_bf16(np.asarray(x, np.float64))


def _planted(L, D, rank, seed, top=(8.0, 4.0), floor=0.5):
    """X = U diag(s) W^T with a clear gap after ``rank`` singular values."""
    rng = np.random.default_rng(seed)
    k = min(L, D)
    U, _ = np.linalg.qr(rng.standard_normal((L, k)))
    W, _ = np.linalg.qr(rng.standard_normal((D, D)))
    s = np.concatenate([np.linspace(top[0], top[1], rank), np.linspace(floor, 0.0, k - rank)])
    return (U * s) @ W[:, :k].T


def test_hand_example_rank_one():
    # rows (1,1), (1,1), (1,-1): X^T X = [[3,1],[1,3]] has eigenvalues 4 along
    # (1,1)/sqrt2 and 2 along (1,-1)/sqrt2; rank 1 keeps each row's (1,1) part
    x = np.array([[[[1, 1], [1, 1], [1, -1]]]], np.float64)
    got, vals = oracle.project_residual(_bits(x), 1)
    assert np.allclose(got[0, 0], [[1, 1], [1, 1], [0, 0]], atol=1e-14)
    assert np.allclose(vals[0, 0], [4.0], atol=1e-13)


def test_hand_example_axis_aligned():
    x = np.zeros((1, 1, 4, 3))
    x[0, 0, 0, 0], x[0, 0, 1, 1], x[0, 0, 2, 2] = 3.0, -2.0, 0.5
    got, vals = oracle.project_residual(_bits(x), 2)
    want = x.copy()
    want[0, 0, 2, 2] = 0.0  # the smallest direction (e_2, singular value 0.5) is dropped
    assert np.allclose(got, want, atol=1e-14)
    assert np.allclose(vals[0, 0], [9.0, 4.0], atol=1e-13)


@pytest.mark.parametrize("L,D,rank", [(200, 64, 8), (333, 128, 32), (96, 128, 1)])
def test_projection_equals_truncated_svd(L, D, rank):
    x = np.stack([_planted(L, D, rank, s) for s in range(2)])[None] * 0.01
    bits = _bits(x)
    got, vals = oracle.project_residual(bits, rank)
    xv = oracle.bf16_to_f64(bits)
    for h in range(2):
        U, S, Wt = np.linalg.svd(xv[0, h], full_matrices=False)
        want = (U[:, :rank] * S[:rank]) @ Wt[:rank]
        assert np.max(np.abs(got[0, h] - want)) <= 1e-12 * np.abs(xv).max()
        assert np.allclose(vals[0, h], S[:rank] ** 2, rtol=1e-10)


def test_eckart_young_energy_and_orthogonality():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((1, 1, 150, 64)) * 0.02  # no gap: the energy is still unique
    bits = _bits(x)
    X = oracle.bf16_to_f64(bits)[0, 0]
    got, vals = oracle.project_residual(bits, 16)
    S = np.linalg.svd(X, compute_uv=False)
    P = got[0, 0]
    assert np.isclose(np.sum((X - P) ** 2), np.sum(S[16:] ** 2), rtol=1e-9)
    assert np.isclose(np.sum(P ** 2), np.sum(S[:16] ** 2), rtol=1e-9)
    assert abs(np.sum((X - P) * P)) <= 1e-12 * np.sum(X ** 2)
    assert np.all(np.diff(vals[0, 0]) <= 0)


def test_full_rank_identity_low_rank_exact_idempotent():
    rng = np.random.default_rng(9)
    x = rng.standard_normal((1, 2, 80, 32)) * 0.1
    bits = _bits(x)
    xv = oracle.bf16_to_f64(bits)
    full, _ = oracle.project_residual(bits, 32)
    assert np.allclose(full, xv, atol=1e-13)
    # an exactly rank-3 input is reproduced by any rank >= 3
    low = rng.integers(-4, 5, size=(1, 1, 80, 3)) @ rng.integers(-4, 5, size=(1, 1, 3, 32))
    lb = _bits(low.astype(np.float64))
    assert np.allclose(oracle.project_residual(lb, 3)[0], low, atol=1e-11)
    assert np.allclose(oracle.project_residual(lb, 7)[0], low, atol=1e-11)
    p1, _ = oracle.project_residual(bits, 5)
    # projecting the projection changes nothing (up to the bf16 re-rounding)
    p2, _ = oracle.project_residual(_bits(p1), 5)
    assert np.max(np.abs(p2 - p1)) <= 2 ** -8 * np.abs(p1).max()


def test_zero_residual_and_rank_bounds():
    z = np.zeros((1, 1, 64, 16), np.uint16)
    got, vals = oracle.project_residual(z, 4)
    assert not got.any() and not vals.any()
    with pytest.raises(ValueError):
        oracle.project_residual(z, 0)
    with pytest.raises(ValueError):
        oracle.project_residual(z, 17)


def test_refresh_step_projects_only_the_second_order_residual():
    rng = np.random.default_rng(2)
    shape = (1, 1, 100, 32)
    st_p, st_n = oracle.ResidualState(shape), oracle.ResidualState(shape)
    outs = [(rng.standard_normal(shape), rng.standard_normal(shape) * 0.9) for _ in range(2)]
    for o_full, o_sp in outs:
        oracle.refresh_step(st_p, o_full, o_sp, rank=4)
        oracle.refresh_step(st_n, o_full, o_sp)
    assert np.array_equal(st_p.r, st_n.r)  # the first-order residual is untouched
    want = oracle.f64_to_bf16(oracle.project_residual(st_n.dr, 4)[0])
    assert np.array_equal(st_p.dr, want)
    assert not np.array_equal(st_p.dr, st_n.dr)
    # the first refresh has no second-order residual to project
    st = oracle.ResidualState(shape)
    oracle.refresh_step(st, *outs[0], rank=4)
    assert not st.dr.any()
