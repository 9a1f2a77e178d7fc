"""GPU parity of SQuad two-pass attention (SQuad,
gist.science/es/paper/2608.16585, technical summary, methodology §1) through
the C ABI against the oracle's squad_attention.

Bit-exact: the window kept lists, the reorder between window-major and
position-major order, and the operator against its composition from the
public entry points.  Within tolerance: the output.  Each pass has the
attention tolerance; the local output is stored in bf16 on both sides, so
the global pass sees values that differ by the local pass's error plus one
bf16 ulp where a rounding flips, and its output (a convex combination of
them) by at most that much more:

  rel-L2 <= 5e-3,   max-abs <= 2 * 2e-2 + 2^-7 * max|V|.
"""
import numpy as np
import pytest
import torch

import oracle
import qsa_gen
from quantized_sparse_attention_amd import binding as B
from tests.gpu_util import MAX_ABS, REL_L2, dev_bf16, host_f64, rel_l2

pytestmark = pytest.mark.gpu


def _inputs(Bn, H, n, D, seed, block=64):
    """Seeded inputs (the seed selects the generator stream; step 0)."""
    w = qsa_gen.get_workload("tiny").with_(cfg_id=100 + seed, batch=Bn, heads=H,
                                           grid=(1, n // 64, 64), block=block, head_dim=D)
    return qsa_gen.make_qkv(w, 0)


def _bound(v_bits):
    return 2 * MAX_ABS + 2.0 ** -7 * np.abs(oracle.bf16_to_f64(v_bits)).max()


@pytest.mark.parametrize("n,window,block,kmax", [(4096, 64, 64, 1), (4096, 512, 64, 8),
                                                 (8192, 256, 128, 4), (4096, 128, 64, 5)])
def test_window_lists_bit_exact(n, window, block, kmax):
    idx, cnt = B.qsa_window_kept(2, 3, n, block, window, kmax=kmax)
    want_idx, want_cnt = oracle.window_kept_lists(2, 3, n, window, block)
    got = idx.cpu().numpy()
    per = window // block
    assert np.array_equal(got[..., :per], want_idx)
    assert np.all(got[..., per:] == -1)
    assert np.array_equal(cnt.cpu().numpy(), want_cnt)


@pytest.mark.parametrize("n,window,D", [(4096, 64, 64), (8192, 128, 128), (6000, 40, 128),
                                        (4096, 4096, 64)])
def test_reorder_bit_exact(n, window, D):
    rng = np.random.default_rng(n + window)
    x = oracle.f64_to_bf16(rng.standard_normal((2, 2, n, D)))
    y = B.qsa_reorder_windows(dev_bf16(x), window)
    want = oracle.to_position_major(x, window)
    got = y.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, want)
    back = B.qsa_reorder_windows(y, window, inverse=True)
    assert np.array_equal(back.view(torch.int16).cpu().numpy().view(np.uint16), x)


@pytest.mark.parametrize("Bn,H,n,D,window,block", [(1, 2, 4096, 64, 64, 64),
                                                    (1, 2, 8192, 128, 128, 64),
                                                    (2, 1, 8192, 64, 64, 64),
                                                    (1, 1, 16384, 128, 128, 128)])
def test_squad_attention_parity(Bn, H, n, D, window, block):
    x = _inputs(Bn, H, n, D, seed=window // 64, block=block)
    out = B.qsa_squad_attention(dev_bf16(x["q"]), dev_bf16(x["k"]), dev_bf16(x["v"]), window,
                                block)
    torch.cuda.synchronize()
    got = host_f64(out)
    want = oracle.squad_attention(x["q"], x["k"], x["v"], window, block)
    r = rel_l2(got, want)
    m = float(np.abs(got - want).max())
    print(f"\n[squad] n={n} w={window} block={block}: rel_l2={r:.2e} max_abs={m:.2e}", flush=True)
    assert r <= REL_L2 and m <= _bound(x["v"])


@pytest.mark.parametrize("Bn,H,n,D,window,block", [(1, 2, 4096, 64, 64, 64),
                                                    (1, 2, 8192, 128, 128, 64),
                                                    (2, 1, 8192, 64, 64, 64),
                                                    (1, 1, 16384, 128, 128, 128)])
def test_squad_equals_its_composition_from_entry_points(Bn, H, n, D, window, block):
    """The operator (one K quantisation per pass, each pass quantising its own
    query rows, row maps in the attention epilogue, no reorder passes) gives,
    bit for bit, what the same two passes give when composed from the public
    entry points: qsa_quantize of Q and K, qsa_window_kept lists and
    qsa_sparse_attn for the local pass; qsa_reorder_windows of Q, K and the
    local output to position-major order, qsa_quantize again, the group lists
    and qsa_sparse_attn for the global pass; the inverse reorder."""
    x = _inputs(Bn, H, n, D, seed=11 + window // 64, block=block)
    q, k, v = (dev_bf16(x[t]) for t in "qkv")
    got = B.qsa_squad_attention(q, k, v, window, block)
    qc, qs, _ = B.qsa_quantize(q, block)
    kc, ks, _ = B.qsa_quantize(k, block)
    idx, cnt = B.qsa_window_kept(Bn, H, n, block, window)
    o_local = B.qsa_sparse_attn(qc, qs, kc, ks, v, idx, cnt, block)
    pm = [B.qsa_reorder_windows(t, window) for t in (q, k, o_local)]
    qc, qs, _ = B.qsa_quantize(pm[0], block)
    kc, ks, _ = B.qsa_quantize(pm[1], block)
    idx, cnt = B.qsa_window_kept(Bn, H, n, block, n // window)
    o_global = B.qsa_sparse_attn(qc, qs, kc, ks, pm[2], idx, cnt, block)
    want = B.qsa_reorder_windows(o_global, window, inverse=True)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), want.view(torch.int16))


# More work items (b*h, group of query blocks) than the device holds
# workgroups at once, with more heads than the other parity cases: every head
# sampled at its ends and middle, and heads 0 and 1 (neighbouring items across
# a head boundary), against the oracle over those whole heads.
@pytest.mark.parametrize("Bn,H,n,D,window,block", [(1, 60, 4096, 64, 64, 64),
                                                    (1, 30, 8192, 128, 128, 64),
                                                    (2, 7, 16384, 128, 128, 128)])
def test_squad_many_heads(Bn, H, n, D, window, block):
    print(f"\n[squad many heads] B={Bn} H={H} n={n} D={D} w={window} block={block}", flush=True)
    x = _inputs(Bn, H, n, D, seed=7 + D // 64, block=block)
    out = B.qsa_squad_attention(dev_bf16(x["q"]), dev_bf16(x["k"]), dev_bf16(x["v"]), window,
                                block)
    torch.cuda.synchronize()
    heads = [0, 1, H // 2, H - 1]
    got = host_f64(out)[:, heads]
    want = oracle.squad_attention(*(x[t][:, heads] for t in "qkv"), window, block)
    r = rel_l2(got, want)
    m = float(np.abs(got - want).max())
    print(f"[squad many heads] heads {heads}: rel_l2={r:.2e} max_abs={m:.2e}", flush=True)
    assert r <= REL_L2 and m <= _bound(x["v"][:, heads])


def test_squad_fullsize_sampled():
    """A 65,536-token sequence (w = sqrt(n) = 256) of 24 heads x 128, the
    head shape of the Wan video DiTs: sampled query blocks of two heads
    against the oracle's local pass over the whole heads and global pass on
    the sampled blocks."""
    Bn, H, n, D, window, block = 1, 24, 65536, 128, 256, 64
    print(f"\n[squad fullsize] B={Bn} H={H} n={n} D={D} w={window}", flush=True)
    w = qsa_gen.get_workload("tiny").with_(batch=Bn, heads=H, grid=(1, 256, 256), block=block,
                                           head_dim=D)
    x = qsa_gen.make_qkv_torch(w, torch.device("cuda:0"))[0]
    out = B.qsa_squad_attention(x["q"], x["k"], x["v"], window, block)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out.float()).all())
    heads = [0, H - 1]
    bits = {t: x[t][:, heads].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
            for t in "qkv"}
    got = host_f64(out[:, heads])
    sm = oracle.default_sm_scale(D)
    # oracle local pass over the two heads
    qc, sq, _ = oracle.quantize(bits["q"], block)
    kc, sk, _ = oracle.quantize(bits["k"], block)
    idx, cnt = oracle.window_kept_lists(Bn, 2, n, window, block)
    o_local = oracle.f64_to_bf16(oracle.attention(qc, sq, kc, sk, bits["v"], idx, cnt, block,
                                                  sm))
    # oracle global pass on sampled position-major blocks
    m = n // window
    qc, sq, _ = oracle.quantize(oracle.to_position_major(bits["q"], window), block)
    kc, sk, _ = oracle.quantize(oracle.to_position_major(bits["k"], window), block)
    idx, cnt = oracle.window_kept_lists(Bn, 2, n, m, block)
    vp = oracle.to_position_major(o_local, window)
    nbk = n // block
    sample = [0, 1, nbk // 2, nbk - 1, 333, 777]
    res = oracle.attention(qc, sq, kc, sk, vp, idx, cnt, block, sm,
                           which=[(0, h, i) for h in range(2) for i in sample])
    gp = oracle.to_position_major(got, window)
    errs, refs = [], []
    for (b, h, i), o in res.items():
        g = gp[b, h, i * block:(i + 1) * block]
        errs.append(g - o)
        refs.append(o)
    err, ref = np.concatenate(errs), np.concatenate(refs)
    r = float(np.linalg.norm(err) / np.linalg.norm(ref))
    mx = float(np.abs(err).max())
    print(f"[squad fullsize] sampled rel_l2={r:.2e} max_abs={mx:.2e}", flush=True)
    assert r <= REL_L2 and mx <= _bound(bits["v"])
