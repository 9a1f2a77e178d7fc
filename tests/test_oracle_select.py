"""Pins of the oracle's step 2: pooled block saliency and top-k + band selection.

Saliency reading R4 (mean-pooled dequantised block dot product) follows the
average-pooling and top-k ideas of MSAD (QuantSparse, gist.science/es/paper/
2509.23681, Resumen técnico §2A; gist.science/ko/paper/2509.23681 §2.1).
Scores are pinned by exact rational arithmetic on Python integers, the
selection by a brute-force full sort, and both by hand-worked examples.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import qsa_gen
from tests.exact import round_f64

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_examples.json")


def _rand_pooled(rng, B, H, nb, D, block):
    lim = 127 * block
    return rng.integers(-lim, lim + 1, (B, H, nb, D)).astype(np.int64)


def _rand_scales(rng, B, H, nb):
    return (np.abs(rng.standard_normal((B, H, nb))) * 0.05).astype(np.float32)


def test_scores_against_exact_rationals():
    rng = np.random.default_rng(7)
    B, H, nb, D, block, L = 1, 2, 5, 16, 64, 300  # last block has 44 tokens
    pq, pk = _rand_pooled(rng, B, H, nb, D, block), _rand_pooled(rng, B, H, nb, D, block)
    sq, sk = _rand_scales(rng, B, H, nb), _rand_scales(rng, B, H, nb)
    got = oracle.block_scores(pq, sq, pk, sk, L, block)
    n = [min(block, L - i * block) for i in range(nb)]
    for h in range(H):
        for i in range(nb):
            for j in range(nb):
                S = sum(int(a) * int(b) for a, b in zip(pq[0, h, i], pk[0, h, j]))
                a = Fraction(float(sq[0, h, i])) * Fraction(float(sk[0, h, j]))
                b = round_f64(Fraction(S) * a)
                want = round_f64(Fraction(b) / (n[i] * n[j]))
                assert got[0, h, i, j] == want


def test_score_extreme_magnitudes_exact():
    # |S| near its maximum (64*127)^2 * 128 for block 64, D 128: beyond int32.
    D, block = 128, 64
    pq = np.full((1, 1, 2, D), 127 * 64, np.int64)
    pk = np.full((1, 1, 2, D), -127 * 64, np.int64)
    sq = np.array([[[3.0e-2, 1.0e-38]]], np.float32)
    sk = np.array([[[7.0e-3, 2.5e-40]]], np.float32)
    got = oracle.block_scores(pq, sq, pk, sk, 128, block)
    for i in range(2):
        for j in range(2):
            S = -(127 * 64) ** 2 * D
            assert abs(S) > 2 ** 31
            b = round_f64(Fraction(S) * Fraction(float(sq[0, 0, i])) * Fraction(float(sk[0, 0, j])))
            assert got[0, 0, i, j] == round_f64(Fraction(b) / (64 * 64))


def test_score_symmetry():
    rng = np.random.default_rng(3)
    pq, pk = _rand_pooled(rng, 1, 1, 9, 32, 64), _rand_pooled(rng, 1, 1, 9, 32, 64)
    sq, sk = _rand_scales(rng, 1, 1, 9), _rand_scales(rng, 1, 1, 9)
    s1 = oracle.block_scores(pq, sq, pk, sk, 9 * 64 - 5, 64)
    s2 = oracle.block_scores(pk, sk, pq, sq, 9 * 64 - 5, 64)
    assert np.array_equal(s1, np.swapaxes(s2, -1, -2))


def _brute_kept(scores_row, i, k, band, nb):
    order = sorted(range(nb), key=lambda j: (-scores_row[j], j))
    kept = set(order[: min(k, nb)]) | {i + o for o in band if 0 <= i + o < nb}
    return sorted(kept)


@pytest.mark.parametrize("nb,k,band", [(7, 3, (0,)), (12, 1, ()), (12, 12, (0,)),
                                       (20, 5, (-3, 0, 3)), (33, 0, (0, 1)), (5, 9, (0,))])
def test_selection_against_brute_force_sort(nb, k, band):
    rng = np.random.default_rng(nb * 100 + k)
    # coarse scores force many exact ties; include signed zeros
    sc = rng.integers(-3, 4, (1, 2, nb, nb)).astype(np.float64)
    sc[sc == 0] = np.where(rng.random(np.count_nonzero(sc == 0)) < 0.5, 0.0, -0.0)
    kmax = min(nb, k + len(band)) + 2
    idx, cnt = oracle.select_blocks(sc, k, band, kmax)
    for h in range(2):
        for i in range(nb):
            want = _brute_kept(sc[0, h, i], i, k, band, nb)
            assert cnt[0, h, i] == len(want)
            assert idx[0, h, i, : len(want)].tolist() == want
            assert np.all(idx[0, h, i, len(want):] == -1)


def test_selection_of_a_row_subset_against_brute_force_sort():
    # rows= selects given query blocks out of a wider score matrix; the band
    # follows the real row index
    nb, k, band = 40, 4, (-2, 0, 5)
    rng = np.random.default_rng(77)
    sc = rng.integers(-3, 4, (1, 1, nb, nb)).astype(np.float64)
    rows = [0, 1, 17, 36, 39]
    kmax = k + len(band)
    idx, cnt = oracle.select_blocks(sc[:, :, rows], k, band, kmax, rows=rows)
    assert idx.shape == (1, 1, len(rows), kmax)
    for n, i in enumerate(rows):
        want = _brute_kept(sc[0, 0, i], i, k, band, nb)
        assert cnt[0, 0, n] == len(want)
        assert idx[0, 0, n, : len(want)].tolist() == want


def test_selection_invariants():
    rng = np.random.default_rng(11)
    nb, k, band = 40, 6, (-1, 0, 1)
    sc = rng.standard_normal((1, 1, nb, nb)).round(1)
    idx, cnt = oracle.select_blocks(sc, k, band, k + 3)
    for i in range(nb):
        kept = idx[0, 0, i, : cnt[0, 0, i]].tolist()
        assert kept == sorted(set(kept))
        b = {i + o for o in band if 0 <= i + o < nb}
        assert b <= set(kept)
        assert k <= len(kept) <= k + len(b)
        kth = sorted(sc[0, 0, i], reverse=True)[k - 1]
        tied_kept = [jj for jj in kept if jj not in b and sc[0, 0, i, jj] == kth]
        for j in range(nb):
            if j in kept:
                continue
            assert sc[0, 0, i, j] <= kth
            if sc[0, 0, i, j] == kth:   # an excluded tie sits above every kept tie
                assert all(jj < j for jj in tied_kept)


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def _const_blocks(vals, block, D):
    x = np.concatenate([np.full((block, D), v, np.float32) for v in vals])
    return qsa_gen.f32_to_bf16_bits(x)[None, None]


@pytest.mark.parametrize("name", ["H1", "H2_noband", "H2_band0"])
def test_hand_examples_selection(name):
    g = _golden()[name]
    blk, D = g["block"], g["head_dim"]
    q = _const_blocks(g["q_blocks"], blk, D)
    k = _const_blocks(g["k_blocks"], blk, D)
    L = q.shape[2]
    qc, sq, pq = oracle.quantize(q, blk)
    kc, sk, pk = oracle.quantize(k, blk)
    sc = oracle.block_scores(pq, sq, pk, sk, L, blk)
    np.testing.assert_allclose(sc[0, 0], np.array(g["scores"]), rtol=1e-5)
    nb = len(g["q_blocks"])
    idx, cnt = oracle.select_blocks(sc, g["topk"], tuple(g["band"]), nb)
    got = [idx[0, 0, i, : cnt[0, 0, i]].tolist() for i in range(nb)]
    assert got == g["kept"]
