"""Pins of the oracle's SQuad two-pass attention (SQuad,
gist.science/es/paper/2608.16585, technical summary, methodology §1: a local
pass inside windows of w tokens, then a global pass over the tokens at the
same position of every window whose values are the local output).

The oracle composes block-list attention on reordered tensors.  It is pinned
here against the definition written with whole-sequence element masks
(same window / same position) and torch's fused attention routine, against
an explicit index formula for the reordering, a uniform-attention closed
form and the full receptive field the page claims.
"""
import numpy as np
import pytest
import torch

import oracle
import qsa_gen


def _inputs(B, H, n, D, seed):
    """Seeded inputs (the seed selects the generator stream; step 0)."""
    w = qsa_gen.get_workload("tiny").with_(cfg_id=100 + seed, batch=B, heads=H,
                                           grid=(1, n // 64, 64), block=64, head_dim=D)
    return qsa_gen.make_qkv(w, 0)


def test_position_major_index_formula():
    B, H, n, w = 1, 2, 512, 128
    m = n // w
    x = np.arange(B * H * n * 3).reshape(B, H, n, 3)
    y = oracle.to_position_major(x, w)
    for k in range(m):
        for p in range(w):
            assert np.array_equal(y[:, :, p * m + k], x[:, :, k * w + p])
    assert np.array_equal(oracle.from_position_major(y, w), x)


def test_window_lists_hand_example():
    idx, cnt = oracle.window_kept_lists(1, 1, 256, 128, 64)
    assert idx[0, 0].tolist() == [[0, 1], [0, 1], [2, 3], [2, 3]]
    assert cnt[0, 0].tolist() == [2, 2, 2, 2]
    with pytest.raises(ValueError):
        oracle.window_kept_lists(1, 1, 256, 96, 64)


def _dequant(bits, block):
    c, s, _ = oracle.quantize(bits, block)
    blk = np.arange(bits.shape[2]) // block
    return c.astype(np.float64) * s.astype(np.float64)[..., blk, None]


def _masked(q, k, v, mask, sm):
    return torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
        attn_mask=torch.from_numpy(mask), scale=float(sm)).numpy()


@pytest.mark.parametrize("n,w", [(4096, 64), (8192, 64), (8192, 128)])
def test_squad_equals_masked_definition(n, w):
    x = _inputs(1, 2, n, 64, seed=0)
    sm = oracle.default_sm_scale(64)
    got = oracle.squad_attention(x["q"], x["k"], x["v"], w, 64)
    t = np.arange(n)
    m = n // w
    # local pass: same window; operands quantised in the natural order
    local = _masked(_dequant(x["q"], 64), _dequant(x["k"], 64), oracle.bf16_to_f64(x["v"]),
                    (t[:, None] // w) == (t[None, :] // w), sm)
    local = oracle.bf16_to_f64(oracle.f64_to_bf16(local))
    # global pass: same position; Q and K quantised in position-major order,
    # written here with an explicit gather (index p*m + k holds token k*w + p)
    perm = np.array([k * w + p for p in range(w) for k in range(m)])
    inv = np.argsort(perm)
    qg = _dequant(np.ascontiguousarray(x["q"][:, :, perm]), 64)[:, :, inv]
    kg = _dequant(np.ascontiguousarray(x["k"][:, :, perm]), 64)[:, :, inv]
    want = _masked(qg, kg, local, (t[:, None] % w) == (t[None, :] % w), sm)
    np.testing.assert_allclose(got, want, rtol=1e-11, atol=1e-12)


def test_uniform_attention_closed_form():
    """K = 0 makes every logit 0: each pass averages its values."""
    n, w = 4096, 64
    x = _inputs(1, 1, n, 64, seed=1)
    k0 = np.zeros_like(x["k"])
    got = oracle.squad_attention(x["q"], k0, x["v"], w, 64)
    v = oracle.bf16_to_f64(x["v"])[0, 0]
    win_mean = v.reshape(n // w, w, 64).mean(axis=1)                # [windows, D]
    local = oracle.bf16_to_f64(oracle.f64_to_bf16(np.repeat(win_mean, w, axis=0)))
    want = local.reshape(n // w, w, 64).mean(axis=0)                  # [positions, D]
    np.testing.assert_allclose(got[0, 0], np.tile(want, (n // w, 1)), rtol=1e-12, atol=1e-13)


def test_full_receptive_field():
    """One changed value reaches every output (the global pass mixes the
    windows, the local pass the positions).  Small logits keep every weight
    well above the bf16 rounding of the local output."""
    n, w = 4096, 64
    x = _inputs(1, 1, n, 64, seed=2)
    q = oracle.f64_to_bf16(0.05 * oracle.bf16_to_f64(x["q"]))
    base = oracle.squad_attention(q, x["k"], x["v"], w, 64)
    v2 = x["v"].copy()
    v2[0, 0, 777] = oracle.f64_to_bf16(oracle.bf16_to_f64(v2[0, 0, 777]) + 8.0)
    moved = oracle.squad_attention(q, x["k"], v2, w, 64)
    assert np.all(np.any(moved != base, axis=-1))


def test_shape_checks():
    x = _inputs(1, 1, 4096, 64, seed=3)
    with pytest.raises(ValueError):
        oracle.squad_attention(x["q"], x["k"], x["v"], 96, 64)
    with pytest.raises(ValueError):
        oracle.squad_attention(x["q"], x["k"], x["v"], 2048, 64)  # n/w = 2 < block
