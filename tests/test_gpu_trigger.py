"""GPU parity of qsa_l1_change and of the layer's adaptive refresh trigger
(DVD-Quant, gist.science/es/paper/2505.18663, technical summary §2C: the
normalised L1 change of consecutive outputs accumulated against a threshold).

The sums are fp64 reductions in a different order from the oracle's, so they
agree to within the reordering error of fp64 summation: at most n * 2^-53 of
the sum of magnitudes for n terms per thread (<= ~1500 at the largest size)
plus the tree depth, i.e. below 1e-12 relative here.  Cases whose terms are
exact multiples of each other must agree exactly.
"""
import numpy as np
import pytest
import torch

import oracle
import qsa_gen
from quantized_sparse_attention_amd import binding as B
from tests.gpu_util import dev_bf16, host_bits

pytestmark = pytest.mark.gpu

REL = 1e-12


def _bits(x):
    return oracle.f64_to_bf16(np.asarray(x, np.float64))


def _sums(a_bits, b_bits):
    s = B.qsa_l1_change(dev_bf16(a_bits), dev_bf16(b_bits))
    torch.cuda.synchronize()
    return s.cpu().numpy()


@pytest.mark.parametrize("shape", [(1, 1, 1, 64), (1, 3, 333, 128), (2, 2, 1000, 64),
                                   (1, 4, 75600 // 16, 128)])
def test_l1_sums_match_oracle(shape):
    rng = np.random.default_rng(shape[2])
    a = rng.standard_normal(shape)
    b = a + 0.1 * rng.standard_normal(shape)
    a_bits, b_bits = _bits(a), _bits(b)
    got = _sums(a_bits, b_bits)
    num, den = oracle.l1_change(a_bits, b_bits)
    assert abs(got[0] - num) <= REL * num and abs(got[1] - den) <= REL * den


def test_l1_exact_cases():
    rng = np.random.default_rng(3)
    a = _bits(rng.standard_normal((1, 2, 500, 128)))
    av = oracle.bf16_to_f64(a)
    s = _sums(a, a)
    assert s[0] == 0.0 and s[1] > 0
    s2 = _sums(a, _bits(2 * av))       # |2a - a| = |a| term by term, same order
    assert s2[0] == s2[1] == s[1]
    s3 = _sums(a, _bits(-av))          # |-a - a| = 2|a|
    assert s3[0] == 2 * s3[1]
    z = np.zeros_like(a)
    s4 = _sums(z, a)
    assert s4[1] == 0.0 and s4[0] == s[1]


def test_l1_deterministic():
    rng = np.random.default_rng(5)
    a, b = (_bits(rng.standard_normal((1, 8, 3000, 128))) for _ in range(2))
    assert np.array_equal(_sums(a, b).view(np.uint64), _sums(a, b).view(np.uint64))


def test_l1_fullsize_wan14b_720p():
    """The launch configuration of a Wan2.1-14B 720p layer output."""
    shape = (1, 40, 75600, 128)
    print(f"\n[l1 fullsize] {shape}", flush=True)
    g = torch.Generator(device="cuda").manual_seed(9)
    a = torch.randn(shape, generator=g, device="cuda").to(torch.bfloat16)
    b = (a.float() + 0.05 * torch.randn(shape, generator=g, device="cuda")).to(torch.bfloat16)
    s = B.qsa_l1_change(a, b).cpu().numpy()
    num, den = oracle.l1_change(host_bits(a), host_bits(b))
    print(f"[l1 fullsize] rel err num {abs(s[0] - num) / num:.2e} den {abs(s[1] - den) / den:.2e}",
          flush=True)
    assert abs(s[0] - num) <= REL * num and abs(s[1] - den) <= REL * den


@pytest.mark.parametrize("delta", [0.02, 0.2])
def test_adaptive_layer_decisions(delta):
    """The layer refreshes exactly when the oracle's trigger, fed the same
    per-step sums, says so; the sums match the oracle's on the GPU outputs."""
    from quantized_sparse_attention_amd import QSAConfig, QuantSparseAttention
    w = qsa_gen.get_workload("tiny").with_(grid=(2, 8, 24), head_dim=64)
    steps = qsa_gen.make_qkv_steps(w, 10)
    layer = QuantSparseAttention(QSAConfig(block=w.block, topk=2, band=(0,),
                                           adaptive_delta=delta))
    trig = oracle.RefreshTrigger(delta)
    prev = None
    kinds = []
    for x in steps:
        refresh = layer.refresh_next or layer.r is None
        assert refresh == trig.refresh_next
        kinds.append("F" if refresh else "S")
        out = layer.step(dev_bf16(x["q"]), dev_bf16(x["k"]), dev_bf16(x["v"]))
        cur = host_bits(out)
        if prev is None:
            assert layer.last_sums is None
            trig.update()
        else:
            num, den = oracle.l1_change(prev, cur)
            gnum, gden = layer.last_sums
            assert abs(gnum - num) <= REL * num and abs(gden - den) <= REL * den
            trig.update(gnum, gden)
        assert layer.refresh_next == trig.refresh_next
        prev = cur
    print(f"\n[adaptive delta={delta}] steps: {''.join(kinds)}", flush=True)
    assert kinds[0] == "F" and kinds[1] == "S"
