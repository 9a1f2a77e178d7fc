"""GPU parity of qsa_project_residual (rank-r projection of the second-order
residual) against the oracle's project_residual.

What is unique is compared with the oracle: the eigenvalues (always), the
projected residual (when the rank-th and next eigenvalues are well
separated, as in the planted-gap inputs) and the captured energy (always:
the sum of the top-r eigenvalues, Eckart-Young).  What is not unique (the
basis, and the projection when the spectrum has no gap at the rank) is
checked for validity: orthonormal columns and an output equal to X V V^T with
the returned basis.

Tolerances (fp32 Gram and Jacobi against the fp64 oracle):
  eigenvalues        |lam - lam_oracle| <= 1e-4 lam_max   (Weyl: the Gram
                     matrix's fp32 summation error, ~sqrt(L) 2^-24 ||G||)
  basis              |V^T V - I| <= 1e-4
  planted-gap output |got - want| <= half a bf16 ulp of the larger of the two
                     + 3e-4 max|X|  (subspace error <= Gram error / gap)
"""
import numpy as np
import pytest
import torch

import oracle
from quantized_sparse_attention_amd import binding as B
from tests.gpu_util import dev_bf16, host_f64

pytestmark = pytest.mark.gpu


def _half_ulp(x):
    e = np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** -126)))
    return 2.0 ** (e - 8)


def _planted(Bn, H, L, D, rank, seed, scale=0.01):
    """bf16 bits of X = U diag(s) W^T per (b, h): `rank` singular values in
    [4, 8], the rest <= 0.5 (a clear gap at the rank)."""
    rng = np.random.default_rng(seed)
    out = np.empty((Bn, H, L, D))
    k = min(L, D)
    for b in range(Bn):
        for h in range(H):
            U, _ = np.linalg.qr(rng.standard_normal((L, k)))
            W, _ = np.linalg.qr(rng.standard_normal((D, D)))
            s = np.concatenate([np.linspace(8.0, 4.0, min(rank, k)),
                                np.linspace(0.5, 0.0, k - min(rank, k))])
            out[b, h] = (U * s) @ W[:, :k].T * np.sqrt(L) * scale
    return oracle.f64_to_bf16(out)


def _run(bits, rank):
    t = dev_bf16(bits)
    basis, vals = B.qsa_project_residual(t, rank)
    torch.cuda.synchronize()
    return host_f64(t), basis.cpu().numpy().astype(np.float64), vals.cpu().numpy()


def _check_basis_and_self_consistency(x, got, basis):
    Bn, H = x.shape[:2]
    r = basis.shape[-1]
    for b in range(Bn):
        for h in range(H):
            V = basis[b, h]
            assert np.max(np.abs(V.T @ V - np.eye(r))) <= 1e-4, (b, h)
            # the output is X V V^T with the returned basis, rounded to bf16
            want = (x[b, h] @ V) @ V.T
            err = np.abs(got[b, h] - want)
            bound = _half_ulp(np.maximum(np.abs(want), np.abs(got[b, h]))) * 1.01 + \
                1e-5 * np.abs(x[b, h]).max()
            assert np.all(err <= bound), (b, h, float((err - bound).max()))


def _check_eigvals(vals, want):
    lam_max = np.abs(want).max(axis=-1, keepdims=True)
    assert np.all(np.abs(vals - want) <= 1e-4 * lam_max + 1e-30)


CASES = [  # B, H, L, D, rank
    (1, 3, 1000, 128, 8),
    (1, 2, 1000, 128, 32),
    (2, 2, 333, 64, 16),
    (1, 2, 5000, 128, 64),
    (1, 1, 70, 64, 1),
    (1, 1, 4100, 64, 64),  # rank = D: the identity projection
]


@pytest.mark.parametrize("Bn,H,L,D,rank", CASES)
def test_projection_planted_gap_matches_oracle(Bn, H, L, D, rank):
    bits = _planted(Bn, H, L, D, rank, seed=L + rank)
    got, basis, vals = _run(bits, rank)
    want, wvals = oracle.project_residual(bits, rank)
    x = oracle.bf16_to_f64(bits)
    _check_eigvals(vals, wvals)
    _check_basis_and_self_consistency(x, got, basis)
    bound = _half_ulp(np.maximum(np.abs(want), np.abs(got))) * 1.01 + \
        3e-4 * np.abs(x).max(axis=(-2, -1), keepdims=True)
    err = np.abs(got - want)
    assert np.all(err <= bound), float((err - bound).max())
    if rank == D:
        assert np.array_equal(got, x) or np.all(np.abs(got - x) <= bound)


@pytest.mark.parametrize("L,D,rank", [(777, 128, 16), (640, 64, 8)])
def test_projection_without_gap_energy_and_validity(L, D, rank):
    rng = np.random.default_rng(L)
    bits = oracle.f64_to_bf16(rng.standard_normal((1, 2, L, D)) * 0.03)
    got, basis, vals = _run(bits, rank)
    _, wvals = oracle.project_residual(bits, rank)
    x = oracle.bf16_to_f64(bits)
    _check_eigvals(vals, wvals)
    _check_basis_and_self_consistency(x, got, basis)
    # captured energy: the optimum sum of the top eigenvalues (Eckart-Young)
    energy = np.sum(got ** 2, axis=(-2, -1))
    opt = wvals.sum(axis=-1)
    assert np.all(np.abs(energy - opt) <= 1e-3 * opt), (energy, opt)


def test_zero_residual_projects_to_zero():
    bits = np.zeros((1, 2, 200, 128), np.uint16)
    got, basis, vals = _run(bits, 4)
    assert not got.any()
    assert not vals.any()
    for h in range(2):
        assert np.allclose(basis[0, h].T @ basis[0, h], np.eye(4))


def test_workspace_reuse_and_deterministic():
    bits = _planted(1, 2, 3000, 128, 16, seed=3)
    work = torch.empty(B.qsa_project_work_bytes(1, 2, 3000, 128, 16), dtype=torch.uint8,
                       device="cuda")
    outs = []
    for _ in range(2):
        t = dev_bf16(bits)
        basis, vals = B.qsa_project_residual(t, 16, work=work)
        torch.cuda.synchronize()
        outs.append((t.view(torch.int16).cpu().numpy(), basis.cpu().numpy(), vals.cpu().numpy()))
    for a, b in zip(*outs):
        assert np.array_equal(a, b)


def test_projection_fullsize_wan14b_720p_sampled_heads():
    """The launch configuration of a Wan2.1-14B 720p layer (B=1, H=40,
    L=75600, D=128, rank 32): planted-gap residuals on three heads compared
    with the oracle, seeded Gaussian residuals on the others."""
    Bn, H, L, D, rank = 1, 40, 75600, 128, 32
    heads = [0, H // 2, H - 1]
    print(f"\n[projection fullsize] B={Bn} H={H} L={L} D={D} rank={rank}", flush=True)
    g = torch.Generator(device="cuda").manual_seed(7)
    t = (torch.randn((Bn, H, L, D), generator=g, device="cuda") * 0.02).to(torch.bfloat16)
    planted = _planted(1, len(heads), L, D, rank, seed=11, scale=0.002)
    for n, h in enumerate(heads):
        t[0, h] = dev_bf16(planted[0, n])
    basis, vals = B.qsa_project_residual(t, rank)
    torch.cuda.synchronize()
    got = host_f64(t[:, heads])
    want, wvals = oracle.project_residual(planted, rank)
    x = oracle.bf16_to_f64(planted)
    _check_eigvals(vals[:, heads].cpu().numpy(), wvals)
    bound = _half_ulp(np.maximum(np.abs(want), np.abs(got))) * 1.01 + \
        3e-4 * np.abs(x).max(axis=(-2, -1), keepdims=True)
    err = np.abs(got - want)
    print(f"[projection fullsize] max err / bound = {float((err / bound).max()):.3f}", flush=True)
    assert np.all(err <= bound)
    assert bool(torch.isfinite(t.float()).all())
    V = basis.double()
    eye = torch.eye(rank, dtype=torch.float64, device="cuda")
    assert float((V.transpose(-1, -2) @ V - eye).abs().max()) <= 1e-4
