"""Pins of the oracle's step 3: block-sparse attention on int8 codes.

Sparsified attention keeps a fraction of the connections (QuantSparse,
gist.science/es/paper/2509.23681, Resumen técnico §1 and §4).  The oracle is
pinned against a library routine (torch's scaled_dot_product_attention in
fp64 on the CPU, with an explicit boolean mask built from the kept lists),
closed forms (uniform softmax over identical keys), the hand-worked examples,
and the softmax normalisation invariant.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import qsa_gen
from tests.exact import round_f32

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_examples.json")


def _pipeline(w, step=0, topk=None, band=None):
    x = qsa_gen.make_qkv(w, step)
    qc, sq, pq = oracle.quantize(x["q"], w.block)
    kc, sk, pk = oracle.quantize(x["k"], w.block)
    sc = oracle.block_scores(pq, sq, pk, sk, w.seq_len, w.block)
    topk = w.topk if topk is None else topk
    band = w.band if band is None else band
    kmax = min(w.n_blocks, topk + len(band))
    idx, cnt = oracle.select_blocks(sc, topk, band, kmax)
    return x, qc, sq, kc, sk, idx, cnt


def _sdpa_reference(x, qc, sq, kc, sk, idx, cnt, block, sm):
    """torch SDPA in fp64 on dequantised codes with the kept lists as a mask."""
    B, H, L, D = qc.shape
    nb = -(-L // block)
    tok_blk = np.arange(L) // block
    qd = qc.astype(np.float64) * np.repeat(sq.astype(np.float64), block, axis=-1)[..., :L, None]
    kd = kc.astype(np.float64) * np.repeat(sk.astype(np.float64), block, axis=-1)[..., :L, None]
    v = oracle.bf16_to_f64(x["v"])
    mask = np.zeros((B, H, L, L), bool)
    for b in range(B):
        for h in range(H):
            for i in range(nb):
                kept = np.zeros(nb, bool)
                for j in idx[b, h, i, : cnt[b, h, i]]:
                    if 0 <= j < nb:  # the valid entries, as a set
                        kept[j] = True
                mask[b, h, i * block: (i + 1) * block] = kept[tok_blk][None, :]
    out = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(qd), torch.from_numpy(kd), torch.from_numpy(v),
        attn_mask=torch.from_numpy(mask), scale=float(sm))
    return out.numpy()


@pytest.mark.parametrize("grid,block,D,topk,band", [
    ((2, 8, 8), 64, 64, 1, (0,)),        # tiny: 2 blocks
    ((1, 10, 30), 64, 64, 2, (0,)),      # L = 300: tail block of 44 tokens
    ((1, 1, 333), 128, 128, 1, (-1, 0)), # block 128, tail of 77
    ((3, 7, 11), 64, 128, 3, ()),        # no band
])
def test_sparse_attention_equals_masked_sdpa(grid, block, D, topk, band):
    w = qsa_gen.get_workload("tiny").with_(grid=grid, block=block, head_dim=D)
    x, qc, sq, kc, sk, idx, cnt = _pipeline(w, topk=topk, band=band)
    sm = oracle.default_sm_scale(D)
    got = oracle.attention(qc, sq, kc, sk, x["v"], idx, cnt, block, sm)
    ref = _sdpa_reference(x, qc, sq, kc, sk, idx, cnt, block, sm)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_density_one_equals_dense_attention():
    w = qsa_gen.get_workload("tiny").with_(grid=(1, 12, 25), block=64, head_dim=64)
    x, qc, sq, kc, sk, _, _ = _pipeline(w)
    B, H, L, D = qc.shape
    idx, cnt = oracle.full_kept_lists(B, H, w.n_blocks)
    sm = oracle.default_sm_scale(D)
    got = oracle.attention(qc, sq, kc, sk, x["v"], idx, cnt, w.block, sm)
    # dense softmax attention over dequantised Q/K written as whole-matrix products
    blk = np.arange(L) // w.block
    qd = qc.astype(np.float64) * sq.astype(np.float64)[..., blk, None]
    kd = kc.astype(np.float64) * sk.astype(np.float64)[..., blk, None]
    z = float(sm) * np.einsum("bhld,bhmd->bhlm", qd, kd)
    p = np.exp(z - z.max(-1, keepdims=True))
    p /= p.sum(-1, keepdims=True)
    want = p @ oracle.bf16_to_f64(x["v"])
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)
    # and equals torch's fused routine without a mask
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(qd), torch.from_numpy(kd), torch.from_numpy(oracle.bf16_to_f64(x["v"])),
        scale=float(sm)).numpy()
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_softmax_rows_sum_to_one():
    w = qsa_gen.get_workload("tiny").with_(grid=(1, 5, 40), block=64, head_dim=64)
    x, qc, sq, kc, sk, idx, cnt = _pipeline(w, topk=2)
    for i in range(w.n_blocks):
        blocks = idx[0, 0, i, : cnt[0, 0, i]].tolist()
        p, keys = oracle.attention_block_probs(qc, sq, kc, sk, 0, 0, i, blocks, w.block,
                                               w.seq_len, oracle.default_sm_scale(64))
        assert np.all(p >= 0)
        np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-14)
        assert len(keys) == sum(min(64, w.seq_len - j * 64) for j in blocks)


def _v_pattern(L, D):
    t = np.arange(L)[:, None]
    d = np.arange(D)[None, :]
    return ((((7 * t + 3 * d) % 17) - 8) / 8.0).astype(np.float32)


def _const_blocks(vals, block, D):
    x = np.concatenate([np.full((block, D), v, np.float32) for v in vals])
    return qsa_gen.f32_to_bf16_bits(x)[None, None]


@pytest.mark.parametrize("name", ["H1", "H2_noband", "H2_band0"])
def test_hand_examples_outputs(name):
    with open(GOLDEN) as f:
        g = json.load(f)[name]
    blk, D = g["block"], g["head_dim"]
    nb = len(g["q_blocks"])
    L = nb * blk
    q = _const_blocks(g["q_blocks"], blk, D)
    k = _const_blocks(g["k_blocks"], blk, D)
    vf = _v_pattern(L, D)
    v = qsa_gen.f32_to_bf16_bits(vf)[None, None]
    qc, sq, pq = oracle.quantize(q, blk)
    kc, sk, pk = oracle.quantize(k, blk)
    sc = oracle.block_scores(pq, sq, pk, sk, L, blk)
    idx, cnt = oracle.select_blocks(sc, g["topk"], tuple(g["band"]), nb)
    sm = oracle.default_sm_scale(D)
    out = oracle.attention(qc, sq, kc, sk, v, idx, cnt, blk, sm)[0, 0]
    means = [vf[j * blk:(j + 1) * blk].astype(np.float64).mean(axis=0) for j in range(nb)]
    for i, kept in enumerate(g["kept"]):
        if len(kept) == 1:
            want = means[kept[0]]
        elif name == "H2_band0" and kept == [1, 2]:
            want = (means[1] + means[2]) / 2
        else:  # H2_band0 block 0: keys of block 0 (codes -127) and block 1 (codes +127)
            s = Fraction(round_f32(Fraction(1) / 127))
            z = float(Fraction(float(sm)) * s * s * 64 * 127 * 127)
            w1 = 1.0 / (1.0 + math.exp(-2 * z))
            want = w1 * means[1] + (1 - w1) * means[0]
        np.testing.assert_allclose(out[i * blk:(i + 1) * blk], np.broadcast_to(want, (blk, D)),
                                   rtol=1e-13, atol=1e-13)


def test_empty_kept_list_gives_zeros():
    w = qsa_gen.get_workload("tiny")
    x, qc, sq, kc, sk, idx, cnt = _pipeline(w)
    cnt = cnt.copy()
    cnt[0, 1, 0] = 0
    out = oracle.attention(qc, sq, kc, sk, x["v"], idx, cnt, w.block, oracle.default_sm_scale(64))
    assert np.all(out[0, 1, :64] == 0)
    assert np.any(out[0, 1, 64:] != 0)


def test_kept_list_is_a_set():
    """kept(i) is a set of key blocks (band union top-k): a list with repeats,
    entries outside [0, nb) and any order gives the attention over the set
    of its valid entries (masked SDPA in fp64 as the reference)."""
    w = qsa_gen.get_workload("tiny").with_(grid=(1, 10, 30), block=64, head_dim=64)
    x, qc, sq, kc, sk, idx, cnt = _pipeline(w, topk=2)
    nb = w.n_blocks
    rng = np.random.default_rng(5)
    B, H = qc.shape[:2]
    kmax = 9
    messy = np.full((B, H, nb, kmax), -1, np.int32)
    mcnt = np.zeros((B, H, nb), np.int32)
    for b in range(B):
        for h in range(H):
            for i in range(nb):
                base = list(rng.choice(nb, size=int(rng.integers(1, 4)), replace=False))
                lst = base + [base[0], -3, nb, 10 ** 6]
                rng.shuffle(lst)
                messy[b, h, i, :len(lst)] = lst
                mcnt[b, h, i] = len(lst)
    sm = oracle.default_sm_scale(64)
    got = oracle.attention(qc, sq, kc, sk, x["v"], messy, mcnt, w.block, sm)
    ref = _sdpa_reference(x, qc, sq, kc, sk, messy, mcnt, w.block, sm)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)
    # and it equals the clean ascending list of the same set
    clean = np.full_like(messy, -1)
    ccnt = np.zeros_like(mcnt)
    for b in range(B):
        for h in range(H):
            for i in range(nb):
                st = sorted({int(j) for j in messy[b, h, i, :mcnt[b, h, i]] if 0 <= j < nb})
                clean[b, h, i, :len(st)] = st
                ccnt[b, h, i] = len(st)
    want = oracle.attention(qc, sq, kc, sk, x["v"], clean, ccnt, w.block, sm)
    np.testing.assert_array_equal(got, want)


def test_sampled_blocks_match_full_run():
    w = qsa_gen.get_workload("tiny").with_(grid=(1, 10, 30), block=64, head_dim=64)
    x, qc, sq, kc, sk, idx, cnt = _pipeline(w, topk=2)
    sm = oracle.default_sm_scale(64)
    full = oracle.attention(qc, sq, kc, sk, x["v"], idx, cnt, 64, sm)
    part = oracle.attention(qc, sq, kc, sk, x["v"], idx, cnt, 64, sm, which=[(0, 1, 4), (0, 0, 2)])
    np.testing.assert_array_equal(part[(0, 1, 4)], full[0, 1, 256:300])
    np.testing.assert_array_equal(part[(0, 0, 2)], full[0, 0, 128:192])
