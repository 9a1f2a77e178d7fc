"""Checks of the seeded input generator (shapes, determinism, recipe)."""
import numpy as np
import pytest
import torch
from scipy.ndimage import gaussian_filter1d

import qsa_gen


@pytest.mark.parametrize("n", [2, 8, 21, 45, 80])
def test_filter_matrix_matches_scipy_reflect(n):
    g = qsa_gen.gaussian_filter_matrix(n, 4.0)
    x = np.random.default_rng(n).standard_normal((n, 3))
    want = gaussian_filter1d(x, 4.0, axis=0, mode="reflect", truncate=4.0)
    np.testing.assert_allclose(g @ x, want, atol=1e-13)


def test_bf16_rounding_matches_torch():
    x = np.random.default_rng(0).standard_normal(10000).astype(np.float32) * 37
    x[:4] = [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 0.0]
    got = qsa_gen.f32_to_bf16_bits(x)
    tb = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, tb)


def test_deterministic_and_head_subsets():
    w = qsa_gen.get_workload("tiny")
    a = qsa_gen.make_qkv(w)
    b = qsa_gen.make_qkv(w)
    for t in "qkv":
        assert np.array_equal(a[t], b[t])
    one = qsa_gen.make_qkv(w, heads=[1])
    assert np.array_equal(one["k"][:, 0], a["k"][:, 1])


def test_recipe_statistics():
    w = qsa_gen.get_workload("wan13b_480p").with_(grid=(4, 30, 52))
    x = qsa_gen.make_qkv(w, heads=[0])
    q = qsa_gen.bf16_bits_to_f32(x["q"][0, 0]).astype(np.float64)
    v = qsa_gen.bf16_bits_to_f32(x["v"][0, 0]).astype(np.float64)
    sd = q.std(axis=0)
    big = np.sort(sd)[-3:]
    assert np.all(big > 7) and np.sort(sd)[-4] < 2          # 3 outlier channels x10 on Q
    assert np.all(v.std(axis=0) < 2)                          # none on V
    np.testing.assert_allclose(v.std(axis=0), np.sqrt(1 + 0.3 ** 2), rtol=0.1)
    # smooth field: neighbouring tokens along a row are strongly correlated
    c = np.mean([np.corrcoef(v[:-1, d], v[1:, d])[0, 1] for d in range(8)])
    assert c > 0.8


def test_drift_between_steps():
    w = qsa_gen.get_workload("tiny")
    s = qsa_gen.make_qkv_steps(w, 3)
    d = qsa_gen.bf16_bits_to_f32(s[1]["v"]) - qsa_gen.bf16_bits_to_f32(s[0]["v"])
    assert 0.03 < d.std() < 0.08
    assert np.array_equal(s[0]["v"], qsa_gen.make_qkv(w, 0)["v"])
    assert np.array_equal(s[2]["q"], qsa_gen.make_qkv(w, 2)["q"])


def test_workload_parameters():
    w = qsa_gen.get_workload("wan14b_720p")
    assert (w.seq_len, w.n_blocks, w.topk, w.kmax) == (75600, 1182, 178, 179)
    h = qsa_gen.get_workload("hunyuan_720p")
    assert (h.seq_len, h.n_blocks, h.topk, h.band) == (118800, 929, 93, (-28, 0, 28))
    assert qsa_gen.get_workload("wan14b_480p_d15").topk == 77
    assert qsa_gen.get_workload("wan14b_480p_d30").topk == 154
