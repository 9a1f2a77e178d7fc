"""qsa_l1_change_noalloc against qsa_l1_change, through the C ABI.

The allocation-free variant keeps its partial sums in the library's own
fixed scratch; it must give the same two sums bit for bit as the variant
with a caller workspace (same kernels, same fixed summation order), on
consecutive calls of decreasing size that share that scratch, and the
device's free memory must not change across a call once the scratch's
address has been looked up.
"""
import pytest
import torch

from quantized_sparse_attention_amd import binding as B

pytestmark = pytest.mark.gpu


def _pair(shape, g, dev):
    prev = torch.randn(shape, generator=g, device=dev).to(torch.bfloat16)
    cur = (prev.float() + 0.1 * torch.randn(shape, generator=g, device=dev)).to(torch.bfloat16)
    return prev, cur


def test_l1_change_noalloc_matches_workspace_variant():
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    g = torch.Generator(device=dev)
    g.manual_seed(11)
    # the first call needs more partial sums than the scratch holds (the
    # partial kernel then strides), the second fewer, the third a handful
    shapes = [(1, 8, 4096, 128), (1, 5, 1000, 128), (1, 2, 130, 64)]
    pairs = [_pair(s, g, dev) for s in shapes]
    sums = torch.empty(2, dtype=torch.float64, device=dev)
    work = torch.empty(B.QSA_L1_WORK_BYTES, dtype=torch.uint8, device=dev)
    want_sums = torch.empty(2, dtype=torch.float64, device=dev)
    torch.cuda.synchronize()
    for i, (prev, cur) in enumerate(pairs):
        B.qsa_l1_change(prev, cur, want_sums, work)
        torch.cuda.synchronize()
        want = want_sums.clone()
        free0 = torch.cuda.mem_get_info()[0]
        B.qsa_l1_change_noalloc(prev, cur, sums)
        torch.cuda.synchronize()
        free1 = torch.cuda.mem_get_info()[0]
        assert torch.equal(sums, want), (shapes[i], sums.tolist(), want.tolist())
        if i > 0:  # the scratch's address is looked up on the first call
            assert free1 == free0, f"free device memory changed across a call: {free0} -> {free1}"
    # and the sums are those of the definition (fp64 reference on the device)
    prev, cur = pairs[-1]
    ref_num = (cur.double() - prev.double()).abs().sum().item()
    ref_den = prev.double().abs().sum().item()
    assert abs(sums[0].item() - ref_num) <= 1e-12 * ref_num
    assert abs(sums[1].item() - ref_den) <= 1e-12 * ref_den
