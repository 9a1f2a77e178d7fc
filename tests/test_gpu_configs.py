"""GPU parity at the 480p workloads over a drifting denoising schedule.

The Wan2.1-1.3B 480p workload (12 heads, 15 % kept) and the Wan2.1-14B 480p
workload at densities 1.0, 0.3 and 0.15 (40 heads), all with L = 32760
(21 x 30 x 52 latent tokens, 512 blocks of 64, the last one 56 tokens), run
through the per-layer driver over ten denoising steps F S S S S F S S S S
(a full-attention refresh every fifth step), with the inputs drifting
between steps.  This exercises the second-order residual (QuantSparse,
gist.science/es/paper/2509.23681, technical summary §2B: the first-order
residual full - sparse is cached at a refresh, its change between
consecutive refreshes is the second-order residual, and sparse steps output
sparse + r + dr) at full size, where the second refresh has dr != 0.

On heads {0, H/2, H-1} (heads are independent) and sampled query blocks
(first, second, middle, the ragged last block, two random), at every step:

* codes, scales, pooled sums and kept lists bit-exact against the oracle;
* refresh steps: the output against the oracle's full attention; r against
  the unrounded oracle residual rho = full - sparse; dr (second refresh)
  against rho - r_prev with the kernel's own cached r_prev and against the
  oracle's own dr.  r and dr are cancellations, so each element is held to
  the sum of the errors of the two attention outputs it is formed from
  (measured per element: the refresh output and the sparse kernel's output
  on the same inputs, which takes the refresh kernel's sparse walk) plus
  their bf16 roundings, and the whole block to rel-L2 <= 5e-3 of the full
  output;
* sparse steps: the output against the oracle's sparse attention plus the
  kernel's own cached r and dr at rel-L2 <= 5e-3 and max-abs <= 2e-2 (the
  caches are checked at the refresh that wrote them, and must be unchanged
  by sparse steps); end to end against the oracle's state machine at
  rel-L2 <= 5e-3;
* density 1.0: every kept set is every block, so sparse = full: r = dr = 0
  bit for bit on every head, the refresh output equals the sparse kernel's
  output bit for bit, and so does every sparse step's output.
"""
import numpy as np
import pytest
import torch

import oracle
import qsa_gen
from quantized_sparse_attention_amd import QSAConfig, QuantSparseAttention
from quantized_sparse_attention_amd import binding as B
from tests.gpu_util import MAX_ABS, REL_L2

pytestmark = pytest.mark.gpu

WORKLOADS = ["wan13b_480p", "wan14b_480p_d100", "wan14b_480p_d30", "wan14b_480p_d15"]
SCHEDULE = "FSSSSFSSSS"


def _bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _hulp(x):
    """Half the bf16 spacing at |x| (normal range)."""
    e = np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** -126)))
    return 2.0 ** (e - 8)


@pytest.fixture(scope="module", params=WORKLOADS)
def run(request):
    w = qsa_gen.get_workload(request.param)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    nb, L, bs = w.n_blocks, w.seq_len, w.block
    print(f"\n[configs] {w.name}: H={w.heads} L={L} nb={nb} topk={w.topk} band={w.band} "
          f"schedule={SCHEDULE}", flush=True)
    heads = [0, w.heads // 2, w.heads - 1]
    rng = np.random.default_rng(7)
    extra = [int(v) for v in rng.choice(np.arange(2, nb - 2), size=2, replace=False)]
    blocks = sorted({0, 1, nb // 2, nb - 1, *extra})
    rows = torch.as_tensor(np.concatenate([np.arange(i * bs, min((i + 1) * bs, L))
                                           for i in blocks]), device=dev)
    inputs = qsa_gen.make_qkv_torch(w, dev, step_seeds=list(range(len(SCHEDULE))))
    layer = QuantSparseAttention(QSAConfig(block=bs, topk=w.topk, band=w.band))
    steps = []
    full_density = {"r_zero": True, "refresh_eq_sparse": True, "step_eq_sparse": True}
    for s, kind in enumerate(SCHEDULE):
        x = inputs[s]
        out = layer.step(x["q"], x["k"], x["v"], refresh=(kind == "F"))
        lb = layer.last
        order = B.qsa_order_query_blocks(lb.kept_idx, lb.kept_cnt, L, bs, w.head_dim)
        # the sparse attention alone on the same inputs (the refresh kernel's
        # sparse walk, and the part a sparse step adds the residuals to)
        sp = B.qsa_sparse_attn_ordered(lb.q_codes, lb.q_scales, lb.k_codes, lb.k_scales, x["v"],
                                       lb.kept_idx, lb.kept_cnt, order, bs)
        torch.cuda.synchronize()
        if w.density >= 1.0:
            same = torch.equal(out.view(torch.int16), sp.view(torch.int16))
            if kind == "F":
                full_density["r_zero"] &= bool((layer.r.view(torch.int16) == 0).all())
                full_density["r_zero"] &= bool((layer.dr.view(torch.int16) == 0).all())
                full_density["refresh_eq_sparse"] &= same
            else:
                full_density["step_eq_sparse"] &= same
        st = {
            "kind": kind,
            "x": {t: _bits(x[t][:, heads]) for t in "qkv"},
            "qc": lb.q_codes[:, heads].cpu().numpy(), "qs": lb.q_scales[:, heads].cpu().numpy(),
            "qp": lb.q_pooled[:, heads].cpu().numpy(), "kc": lb.k_codes[:, heads].cpu().numpy(),
            "ks": lb.k_scales[:, heads].cpu().numpy(), "kp": lb.k_pooled[:, heads].cpu().numpy(),
            "idx": lb.kept_idx[:, heads].cpu().numpy(), "cnt": lb.kept_cnt[:, heads].cpu().numpy(),
            "out": oracle.bf16_to_f64(_bits(out[:, heads][:, :, rows])),
            "sp": oracle.bf16_to_f64(_bits(sp[:, heads][:, :, rows])),
            "r_bits": _bits(layer.r[:, heads][:, :, rows]),
            "dr_bits": _bits(layer.dr[:, heads][:, :, rows]),
            "finite": bool(torch.isfinite(out.float()).all()),
        }
        steps.append(st)
        del out, sp, order
    del inputs, layer
    torch.cuda.empty_cache()

    # the oracle over the same sampled blocks, step by step
    sm = oracle.default_sm_scale(w.head_dim)
    which = [(0, hi, i) for hi in range(len(heads)) for i in blocks]
    fi, fc = oracle.full_kept_lists(1, len(heads), nb)
    for st in steps:
        x = st["x"]
        qc, sq, pq = oracle.quantize(x["q"], bs)
        kc, sk, pk = oracle.quantize(x["k"], bs)
        sc = oracle.block_scores(pq, sq, pk, sk, L, bs)
        idx, cnt = oracle.select_blocks(sc, w.topk, w.band, w.kmax)
        st["o_front"] = dict(qc=qc, qs=sq, qp=pq, kc=kc, ks=sk, kp=pk, idx=idx, cnt=cnt)
        o_sp = oracle.attention(qc, sq, kc, sk, x["v"], idx, cnt, bs, sm, which=which)
        st["o_sp"] = np.stack([np.concatenate([o_sp[(0, hi, i)] for i in blocks])
                               for hi in range(len(heads))])[None]
        if st["kind"] == "F":
            o_f = oracle.attention(qc, sq, kc, sk, x["v"], fi, fc, bs, sm, which=which)
            st["o_full"] = np.stack([np.concatenate([o_f[(0, hi, i)] for i in blocks])
                                     for hi in range(len(heads))])[None]
        del st["x"]
    yield w, heads, blocks, steps, full_density


def test_front_end_bit_exact_every_step(run):
    w, heads, blocks, steps, _ = run
    for s, st in enumerate(steps):
        o = st["o_front"]
        assert np.array_equal(st["qc"], o["qc"]) and np.array_equal(st["kc"], o["kc"]), s
        assert np.array_equal(st["qs"].view(np.uint32), o["qs"].view(np.uint32)), s
        assert np.array_equal(st["ks"].view(np.uint32), o["ks"].view(np.uint32)), s
        assert np.array_equal(st["qp"], o["qp"]) and np.array_equal(st["kp"], o["kp"]), s
        assert np.array_equal(st["cnt"], o["cnt"]) and np.array_equal(st["idx"], o["idx"]), s
        assert st["finite"], s


def _rel(err, ref):
    return float(np.linalg.norm(err) / np.linalg.norm(ref))


def test_refresh_steps_against_oracle(run):
    """Refresh output, r and dr at both refreshes of the schedule."""
    w, heads, blocks, steps, _ = run
    r_prev = None  # the kernel's cached r of the previous refresh (f64 of its bf16)
    r_prev_oracle_bits = None
    n_refresh = 0
    for s, st in enumerate(steps):
        if st["kind"] != "F":
            continue
        n_refresh += 1
        o_full, o_sp = st["o_full"], st["o_sp"]
        got, sp = st["out"], st["sp"]
        e_full, e_sp = got - o_full, sp - o_sp
        assert _rel(e_full, o_full) <= REL_L2 and np.max(np.abs(e_full)) <= MAX_ABS, (
            f"step {s} refresh output: rel {_rel(e_full, o_full):.3e} "
            f"max {np.max(np.abs(e_full)):.3e}")
        assert _rel(e_sp, o_sp) <= REL_L2 and np.max(np.abs(e_sp)) <= MAX_ABS, (
            f"step {s} sparse output: rel {_rel(e_sp, o_sp):.3e} max {np.max(np.abs(e_sp)):.3e}")
        # the kernel's unrounded full and sparse outputs are within half a bf16
        # ulp of the bf16 outputs measured here, so the residual it rounds is
        # within this per-element bound of the oracle's residual
        src = np.abs(e_full) + _hulp(got) + np.abs(e_sp) + _hulp(sp) + 2.0 ** -22 * np.abs(got)
        rho = o_full - o_sp
        r = oracle.bf16_to_f64(st["r_bits"])
        err_r = r - rho
        assert _rel(err_r, o_full) <= REL_L2, f"step {s} r: rel {_rel(err_r, o_full):.3e}"
        assert np.all(np.abs(err_r) <= src + _hulp(r)), (
            f"step {s} r: worst excess {np.max(np.abs(err_r) - src - _hulp(r)):.3e}")
        dr = oracle.bf16_to_f64(st["dr_bits"])
        ost = oracle.ResidualState(rho.shape)
        if r_prev is None:
            assert np.all(st["dr_bits"] == 0), "dr must be 0 at the first refresh"
        else:
            # against rho - r_prev with the kernel's own cached r_prev
            want = rho - r_prev
            err = dr - want
            assert _rel(err, o_full) <= REL_L2, f"step {s} dr: rel {_rel(err, o_full):.3e}"
            assert np.all(np.abs(err) <= src + _hulp(dr)), (
                f"step {s} dr: worst excess {np.max(np.abs(err) - src - _hulp(dr)):.3e}")
            # against the oracle's own state machine (its r_prev differs from
            # the kernel's by the previous refresh's bound)
            ost.r, ost.has_prev = r_prev_oracle_bits, True
            oracle.refresh_step(ost, o_full, o_sp)
            d_or = oracle.bf16_to_f64(ost.dr)
            assert _rel(dr - d_or, o_full) <= 2 * REL_L2, f"step {s} dr vs oracle dr"
            if w.density < 1.0:  # (at density 1 there is no residual: r = dr = 0)
                assert np.max(np.abs(dr)) > 0, "the second refresh must see a drifted residual"
        r_prev = r
        r_prev_oracle_bits = oracle.f64_to_bf16(rho)
    assert n_refresh == 2


def test_sparse_steps_against_oracle(run):
    """Sparse-step outputs: the attention part against the oracle plus the
    kernel's own caches, the caches unchanged since their refresh, and end to
    end against the oracle's state machine."""
    w, heads, blocks, steps, _ = run
    ost = None
    cache = None
    for s, st in enumerate(steps):
        if st["kind"] == "F":
            cache = (st["r_bits"], st["dr_bits"])
            rho_st = oracle.ResidualState(st["o_full"].shape)
            if ost is not None:
                rho_st.r, rho_st.has_prev = ost.r, True
            oracle.refresh_step(rho_st, st["o_full"], st["o_sp"])
            ost = rho_st
            continue
        assert np.array_equal(st["r_bits"], cache[0]) and np.array_equal(st["dr_bits"], cache[1]), (
            f"step {s}: a sparse step changed the residual cache")
        got, sp, o_sp = st["out"], st["sp"], st["o_sp"]
        # the attention the step computes is held to the output tolerance
        e_sp = sp - o_sp
        assert _rel(e_sp, o_sp) <= REL_L2 and np.max(np.abs(e_sp)) <= MAX_ABS, (
            f"step {s} sparse attention: rel {_rel(e_sp, o_sp):.3e} "
            f"max {np.max(np.abs(e_sp)):.3e}")
        # the step output adds the cached residuals to that attention and
        # rounds once more: per element within the attention's own error (its
        # unrounded value is within half a bf16 ulp of the bf16 attention
        # output) plus the output's rounding
        r, dr = oracle.bf16_to_f64(cache[0]), oracle.bf16_to_f64(cache[1])
        want = o_sp + r + dr
        e = got - want
        bound = np.abs(e_sp) + _hulp(sp) + _hulp(got) + 2.0 ** -22 * (np.abs(got) + 1.0)
        assert _rel(e, want) <= REL_L2, f"step {s} sparse step (own caches): rel {_rel(e, want):.3e}"
        assert np.all(np.abs(e) <= bound), (
            f"step {s} sparse step (own caches): worst excess {np.max(np.abs(e) - bound):.3e}")
        e2e = oracle.sparse_step(ost, st["o_sp"])
        assert _rel(got - e2e, e2e) <= REL_L2, f"step {s} end to end: {_rel(got - e2e, e2e):.3e}"


def test_full_density_pins(run):
    """Density 1.0: r = dr = 0 exactly, and refresh and sparse steps give the
    sparse attention's bits (on every head)."""
    w, heads, blocks, steps, fd = run
    if w.density < 1.0:
        pytest.skip("only at density 1.0")
    assert fd["r_zero"], "r or dr not zero at density 1.0"
    assert fd["refresh_eq_sparse"], "refresh output differs from the sparse attention"
    assert fd["step_eq_sparse"], "sparse-step output differs from the sparse attention"
    for st in steps:
        assert np.all(st["cnt"] == w.n_blocks)
