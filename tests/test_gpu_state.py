"""GPU tests of the residual cache's life cycle and of the bounds of every write.

* Resume: a layer's state is saved after F S, restored into a fresh layer,
  and S F S continues; every output and the caches must be bit-identical to
  an uninterrupted run (the cache of QuantSparse, gist.science/es/paper/
  2509.23681, technical summary §2B, is state carried across denoising
  steps, so a restart must reproduce it exactly).  A snapshot must not change
  when the layer it came from steps on.
* Reorder modes: the processing order of the query blocks, taken at refresh
  steps only, at every step, or not at all, changes no output bit.
* Guard bytes: every output buffer of every entry point is allocated inside a
  larger buffer whose bytes before and after it hold a canary pattern, with a
  ragged sequence length and one head (so a write past row L would land in
  the trailing guard); after each call the guards must be intact, and rows of
  the outputs beyond what a call writes must not be touched.
"""
import numpy as np
import pytest
import torch

import qsa_gen
from quantized_sparse_attention_amd import QSAConfig, QuantSparseAttention
from quantized_sparse_attention_amd import binding as B
from tests.gpu_util import dev_bf16

pytestmark = pytest.mark.gpu

TINY = qsa_gen.get_workload("tiny")


def _bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy()


@pytest.mark.parametrize("adaptive", [False, True])
def test_resume_mid_schedule_is_bit_identical(adaptive):
    w = TINY.with_(grid=(2, 12, 40), head_dim=128, noise_std=0.3, outlier_channels=3,
                   outlier_gain=10.0)  # 960 tokens, 15 blocks
    n = 5
    steps = qsa_gen.make_qkv_steps(w, n)
    xs = [{t: dev_bf16(st[t]) for t in "qkv"} for st in steps]
    kinds = [True, False, False, True, False]  # F S | S F S
    cfg = dict(block=w.block, topk=3, band=(0,))
    if adaptive:
        cfg["adaptive_delta"] = 0.02  # the trigger decides refreshes from the output change

    def refresh(s):
        return None if adaptive else kinds[s]

    ref = QuantSparseAttention(QSAConfig(**cfg))
    want = [_bits(ref.step(**xs[s], refresh=refresh(s))) for s in range(n)]
    want_r, want_dr = _bits(ref.r), _bits(ref.dr)

    first = QuantSparseAttention(QSAConfig(**cfg))
    for s in range(2):
        assert np.array_equal(_bits(first.step(**xs[s], refresh=refresh(s))), want[s]), s
    snap = first.state_dict()
    snap_bits = {k: _bits(v) for k, v in snap.items() if isinstance(v, torch.Tensor)}
    # the source layer steps on (including a refresh that rewrites r and dr in
    # place): the snapshot must not follow it
    for s in range(2, n):
        first.step(**xs[s], refresh=refresh(s))
    for k, v in snap_bits.items():
        assert np.array_equal(_bits(snap[k]), v), f"snapshot {k} changed"

    resumed = QuantSparseAttention(QSAConfig(**cfg))
    resumed.load_state_dict(snap)
    for s in range(2, n):
        got = _bits(resumed.step(**xs[s], refresh=refresh(s)))
        assert np.array_equal(got, want[s]), f"step {s} differs after resume"
    assert np.array_equal(_bits(resumed.r), want_r) and np.array_equal(_bits(resumed.dr), want_dr)
    # loading kept copies: the snapshot is still as taken
    for k, v in snap_bits.items():
        assert np.array_equal(_bits(snap[k]), v), f"snapshot {k} changed by the resumed run"


def test_reorder_modes_give_the_same_bits():
    """The processing order of the query blocks changes no output bit: a
    layer that orders at refresh steps and reuses that order on the sparse
    steps (the default), one that orders at every step, and one in ascending
    order give identical outputs and caches over F S S F S with drifting
    inputs.  The first keeps its refresh's order through the sparse steps and
    takes the next refresh's lists' order at the next refresh."""
    w = TINY.with_(grid=(2, 12, 40), head_dim=128, noise_std=0.3, outlier_channels=3,
                   outlier_gain=10.0)  # 960 tokens, 15 blocks
    xs = [{t: dev_bf16(st[t]) for t in "qkv"} for st in qsa_gen.make_qkv_steps(w, 5)]
    kinds = [True, False, False, True, False]
    cfg = dict(block=w.block, topk=3, band=(0,))
    layers = {m: QuantSparseAttention(QSAConfig(reorder=m, **cfg)) for m in ("refresh", "step", "off")}
    assert QuantSparseAttention(QSAConfig(reorder=True, **cfg))._reorder_mode() == "refresh"
    assert QuantSparseAttention(QSAConfig(reorder=False, **cfg))._reorder_mode() == "off"
    with pytest.raises(ValueError):
        QuantSparseAttention(QSAConfig(reorder="sometimes", **cfg))._reorder_mode()
    kept = None
    for s, refresh in enumerate(kinds):
        outs = {m: _bits(lay.step(**xs[s], refresh=refresh)) for m, lay in layers.items()}
        for m in ("step", "off"):
            assert np.array_equal(outs[m], outs["refresh"]), f"step {s}: {m} differs"
            assert np.array_equal(_bits(layers[m].r), _bits(layers["refresh"].r)), (s, m)
            assert np.array_equal(_bits(layers[m].dr), _bits(layers["refresh"].dr)), (s, m)
        lay = layers["refresh"]
        if refresh:
            want = B.qsa_order_query_blocks(lay.last.kept_idx, lay.last.kept_cnt, w.seq_len,
                                            w.block, w.head_dim)
            assert torch.equal(lay.order, want), f"step {s}: the refresh's order"
            kept = lay.order.clone()
        else:
            assert torch.equal(lay.order, kept), f"step {s}: the order was not reused"
        assert layers["off"].order is None


# ---------------------------------------------------------------------------
# guard bytes
# ---------------------------------------------------------------------------

PAD = 4096  # guard bytes on each side (a multiple of 256: keeps the 16-byte alignment)
CANARY = 0xA5


class Guarded:
    """A tensor of ``shape``/``dtype`` inside a byte buffer with PAD canary
    bytes on each side; the tensor's own bytes start as ``fill``."""

    def __init__(self, shape, dtype, dev, fill=CANARY):
        esz = torch.empty((), dtype=dtype).element_size()
        n = int(np.prod(shape)) * esz
        self.raw = torch.full((n + 2 * PAD,), CANARY, dtype=torch.uint8, device=dev)
        self.raw[PAD:PAD + n] = fill
        self.t = self.raw[PAD:PAD + n].view(dtype).view(shape)
        self.n = n

    def guards_intact(self):
        g = torch.cat([self.raw[:PAD], self.raw[PAD + self.n:]])
        return bool((g == CANARY).all())


SHAPES = [
    dict(L=343, block=64, D=128, topk=2, band=(0,)),
    dict(L=347, block=64, D=64, topk=2, band=(-1, 0)),
    dict(L=300, block=128, D=128, topk=1, band=(0,)),
]


@pytest.mark.parametrize("cfg", SHAPES, ids=lambda c: f"L{c['L']}_b{c['block']}_d{c['D']}")
def test_writes_stay_inside_their_buffers(cfg):
    dev = torch.device("cuda:0")
    L, bs, D = cfg["L"], cfg["block"], cfg["D"]
    nb = -(-L // bs)
    kmax = min(nb, cfg["topk"] + len(cfg["band"]))
    w = TINY.with_(grid=(1, 1, L), head_dim=D, block=bs, heads=1)
    x = {t: dev_bf16(v) for t, v in qsa_gen.make_qkv(w).items()}
    G = lambda shape, dt, **kw: Guarded(shape, dt, dev, **kw)  # noqa: E731
    shp = (1, 1, L, D)
    checks = []

    def done(name, *bufs):
        torch.cuda.synchronize()
        for b in bufs:
            assert b.guards_intact(), f"{name}: a write left its buffer ({L=}, {bs=}, {D=})"
        checks.append(name)

    qc, kc = G(shp, torch.int8), G(shp, torch.int8)
    qs, ks = G((1, 1, nb), torch.float32), G((1, 1, nb), torch.float32)
    qp, kp = G((1, 1, nb, D), torch.int32), G((1, 1, nb, D), torch.int32)
    B.qsa_quantize(x["q"], bs, qc.t, qs.t, qp.t)
    B.qsa_quantize(x["k"], bs, kc.t, ks.t, kp.t)
    done("qsa_quantize", qc, kc, qs, ks, qp, kp)
    rc, rs, rp = G(shp, torch.int8), G((1, 1, nb), torch.float32), G((1, 1, nb, D), torch.int32)
    B.qsa_quantize_rotated(x["q"], bs, rc.t, rs.t, rp.t)
    done("qsa_quantize_rotated", rc, rs, rp)
    idx, cnt = G((1, 1, nb, kmax), torch.int32), G((1, 1, nb), torch.int32)
    B.qsa_select_blocks(qp.t, qs.t, kp.t, ks.t, L, bs, cfg["topk"], cfg["band"], kmax, idx.t,
                        cnt.t)
    done("qsa_select_blocks", idx, cnt)
    # the workspace variant: its outputs and the workspace itself (one slice,
    # the exact size) stay inside their buffers, and the lists are the same
    slice_b = B.qsa_select_slice_bytes(1, 1, L, D, bs)
    idx2, cnt2 = G((1, 1, nb, kmax), torch.int32), G((1, 1, nb), torch.int32)
    wk = G((slice_b,), torch.uint8)
    B.qsa_select_blocks(qp.t, qs.t, kp.t, ks.t, L, bs, cfg["topk"], cfg["band"], kmax, idx2.t,
                        cnt2.t, work=wk.t)
    done("qsa_select_blocks_work", idx2, cnt2, wk)
    assert torch.equal(idx2.t, idx.t) and torch.equal(cnt2.t, cnt.t)
    order = G((1, 1, nb), torch.int32)
    B.qsa_order_query_blocks(idx.t, cnt.t, L, bs, D, order.t)
    done("qsa_order_query_blocks", order)
    rng = np.random.default_rng(3)
    small = lambda s: dev_bf16(qsa_gen.f32_to_bf16_bits(  # noqa: E731
        rng.standard_normal(shp).astype(np.float32) * s))
    r_in, dr_in = small(0.05), small(0.01)
    for name, fn in (("qsa_sparse_attn", lambda o: B.qsa_sparse_attn(
            qc.t, qs.t, kc.t, ks.t, x["v"], idx.t, cnt.t, bs, r=r_in, dr=dr_in, out=o)),
                     ("qsa_sparse_attn_ordered", lambda o: B.qsa_sparse_attn_ordered(
            qc.t, qs.t, kc.t, ks.t, x["v"], idx.t, cnt.t, order.t, bs, r=r_in, dr=dr_in,
            out=o))):
        out = G(shp, torch.bfloat16)
        fn(out.t)
        done(name, out)
    for od in (None, order.t):
        r, dr, out = G(shp, torch.bfloat16, fill=0), G(shp, torch.bfloat16), G(shp,
                                                                               torch.bfloat16)
        B.qsa_full_attn_residual(qc.t, qs.t, kc.t, ks.t, x["v"], idx.t, cnt.t, bs, r.t, dr.t, 0,
                                 out_full=out.t, order=od)
        done("qsa_full_attn_residual" + ("_ordered" if od is not None else ""), r, dr, out)
        B.qsa_full_attn_residual(qc.t, qs.t, kc.t, ks.t, x["v"], idx.t, cnt.t, bs, r.t, dr.t, 1,
                                 out_full=out.t, order=od)
        done("qsa_full_attn_residual has_prev", r, dr, out)
    out = G(shp, torch.bfloat16)
    B.qsa_apply_residual(x["v"], r_in, dr_in, out=out.t)
    done("qsa_apply_residual", out)
    sums = G((2,), torch.float64)
    B.qsa_l1_change(x["q"], x["k"], sums.t)
    done("qsa_l1_change", sums)
    rank = 4
    dr_p = G(shp, torch.bfloat16, fill=0)
    dr_p.t.copy_(r_in)
    basis, vals = G((1, 1, D, rank), torch.float32), G((1, 1, rank), torch.float32)
    B.qsa_project_residual(dr_p.t, rank, basis.t, vals.t)
    done("qsa_project_residual", dr_p, basis, vals)
    assert len(checks) == 14
