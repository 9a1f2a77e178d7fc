"""GPU parity at full size, in the launch configuration the benchmark times.

The Wan-14B 720p workload (B=1, H=40, L=75600, D=128, block 64, 15 % kept)
and the HunyuanVideo 720p workload (B=1, H=24, L=118800, block 128, 10 %
kept, band {-28, 0, 28}) run through the C ABI on every head.  The oracle then
checks what it can compute one by one:

* bit-exact: codes, scales, pooled sums and kept lists on heads
  {0, H/2, H-1} (heads are independent, so a subset pins the rest);
* rel-L2 / max-abs: the sparse attention output, the refresh-step output
  and the output of a sparse step that applies the refresh's residuals, on
  sampled query blocks of those heads (first, second, middle, the ragged last
  block, two random); the residual r against the unrounded full - sparse;
* everywhere: every output is finite and every kept list is ascending, in
  range, contains its band and has top-k + band entries at most; the sparse
  step and a second refresh step (on top of the cached residual) give the
  same bits when the query blocks run in the computed processing order.

The inputs come from the seeded generator on the GPU (qsa_gen.make_qkv_torch);
the oracle reads the same bf16 values copied to the host.
"""
import numpy as np
import pytest
import torch

import oracle
import qsa_gen
from quantized_sparse_attention_amd import binding as B
from tests.gpu_util import REL_L2, MAX_ABS

pytestmark = pytest.mark.gpu

WORKLOADS = ["wan14b_720p", "hunyuan_720p"]


def _bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.fixture(scope="module", params=WORKLOADS)
def run(request):
    w = qsa_gen.get_workload(request.param)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"\n[fullsize] {w.name}: B={w.batch} H={w.heads} L={w.seq_len} D={w.head_dim} "
          f"block={w.block} topk={w.topk} band={w.band}", flush=True)
    x = qsa_gen.make_qkv_torch(w, dev)[0]
    qc, qs, qp = B.qsa_quantize(x["q"], w.block)
    kc, ks, kp = B.qsa_quantize(x["k"], w.block)
    idx, cnt = B.qsa_select_blocks(qp, qs, kp, ks, w.seq_len, w.block, w.topk, w.band, w.kmax)
    sparse = B.qsa_sparse_attn(qc, qs, kc, ks, x["v"], idx, cnt, w.block)
    r = torch.zeros_like(x["v"])
    dr = torch.zeros_like(r)
    full = B.qsa_full_attn_residual(qc, qs, kc, ks, x["v"], idx, cnt, w.block, r, dr, 0)
    # a sparse step on the same inputs applying the cached residuals
    step = B.qsa_sparse_attn(qc, qs, kc, ks, x["v"], idx, cnt, w.block, r=r, dr=dr)
    # the same step with the query blocks in the computed processing order
    order = B.qsa_order_query_blocks(idx, cnt, w.seq_len, w.block, w.head_dim)
    step_o = B.qsa_sparse_attn_ordered(qc, qs, kc, ks, x["v"], idx, cnt, order, w.block, r=r,
                                       dr=dr)
    # a second refresh on top of the residual just cached (has_prev = 1), in
    # ascending order and in the computed order
    outs = []
    for od in (None, order):
        rr = r.clone()
        ddr = torch.empty_like(r)
        ff = B.qsa_full_attn_residual(qc, qs, kc, ks, x["v"], idx, cnt, w.block, rr, ddr, 1,
                                      order=od)
        outs.append((ff, rr, ddr))
    rot = [*B.qsa_quantize_rotated(x["q"], w.block), *B.qsa_quantize_rotated(x["k"], w.block)]
    torch.cuda.synchronize()
    refresh_same = all(torch.equal(a.view(torch.int16), b.view(torch.int16))
                       for a, b in zip(*outs))
    del outs, rr, ddr, ff
    srt, _ = torch.sort(order.long(), dim=-1)
    order_ok = bool((srt == torch.arange(w.n_blocks, device=dev)).all())
    ordered_same = torch.equal(step.view(torch.int16), step_o.view(torch.int16))
    del step_o, order, srt
    heads = [0, w.heads // 2, w.heads - 1]
    host = {t: _bits(x[t][:, heads]) for t in "qkv"}
    g = {
        "qc": qc[:, heads].cpu().numpy(), "qs": qs[:, heads].cpu().numpy(),
        "qp": qp[:, heads].cpu().numpy(), "kc": kc[:, heads].cpu().numpy(),
        "ks": ks[:, heads].cpu().numpy(), "kp": kp[:, heads].cpu().numpy(),
        "idx": idx[:, heads].cpu().numpy(), "cnt": cnt[:, heads].cpu().numpy(),
        "sparse": oracle.bf16_to_f64(_bits(sparse[:, heads])),
        "full": oracle.bf16_to_f64(_bits(full[:, heads])),
        "r": oracle.bf16_to_f64(_bits(r[:, heads])),
        "r_bits": _bits(r[:, heads]),
        "step": oracle.bf16_to_f64(_bits(step[:, heads])),
        "dr_bits": _bits(dr[:, heads]),
        "finite": all(bool(torch.isfinite(t.float()).all()) for t in (sparse, full, r, step)),
        "idx_all": idx, "cnt_all": cnt,
        "order_ok": order_ok, "ordered_same": ordered_same, "refresh_same": refresh_same,
        "rot": [t[:, heads].cpu().numpy() for t in rot],
    }
    del rot
    # the oracle's front end on the head subset
    oqc, osq, opq = oracle.quantize(host["q"], w.block)
    okc, osk, opk = oracle.quantize(host["k"], w.block)
    sc = oracle.block_scores(opq, osq, opk, osk, w.seq_len, w.block)
    oidx, ocnt = oracle.select_blocks(sc, w.topk, w.band, w.kmax)
    o = dict(qc=oqc, sq=osq, pq=opq, kc=okc, sk=osk, pk=opk, idx=oidx, cnt=ocnt,
             rot=[*oracle.quantize_rotated(host["q"], w.block),
                  *oracle.quantize_rotated(host["k"], w.block)])
    del x, qc, kc, qp, kp, sparse, full, r, dr, step
    yield w, heads, host, g, o
    torch.cuda.empty_cache()


def _sample_blocks(w, seed=0):
    nb = w.n_blocks
    rng = np.random.default_rng(seed)
    extra = [int(v) for v in rng.choice(np.arange(2, nb - 2), size=2, replace=False)]
    return sorted({0, 1, nb // 2, nb - 1, *extra})


def _close(got, want, what):
    err = got - want
    rel = np.linalg.norm(err) / np.linalg.norm(want)
    mx = np.max(np.abs(err))
    assert rel <= REL_L2 and mx <= MAX_ABS, f"{what}: rel_l2={rel:.3e} max_abs={mx:.3e}"
    return rel, mx


def _half_ulp_bf16(x):
    """Half the bf16 spacing at |x| (normal range)."""
    e = np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** -126)))
    return 2.0 ** (e - 8)


def test_fullsize_front_end_bit_exact(run):
    w, heads, host, g, o = run
    assert np.array_equal(g["qc"], o["qc"]) and np.array_equal(g["kc"], o["kc"]), "codes"
    assert np.array_equal(g["qs"], o["sq"]) and np.array_equal(g["ks"], o["sk"]), "scales"
    assert np.array_equal(g["qp"], o["pq"]) and np.array_equal(g["kp"], o["pk"]), "pooled"
    assert np.array_equal(g["cnt"], o["cnt"]), "kept counts"
    assert np.array_equal(g["idx"], o["idx"]), "kept lists"


def test_fullsize_rotated_quantize_bit_exact(run):
    w, heads, host, g, o = run
    for name, got, want in zip(("q codes", "q scales", "q pooled", "k codes", "k scales",
                                "k pooled"), g["rot"], o["rot"]):
        assert np.array_equal(got, want), name


def test_fullsize_kept_lists_valid_on_every_head(run):
    w, heads, host, g, o = run
    idx, cnt = g["idx_all"], g["cnt_all"]
    nb = w.n_blocks
    c = cnt.cpu()
    assert int(c.min()) >= min(w.topk, nb) and int(c.max()) <= min(nb, w.topk + len(w.band))
    kmax = idx.shape[-1]
    pos = torch.arange(kmax, device=idx.device)
    valid = pos[None, None, None, :] < cnt[..., None]
    assert bool(((idx >= 0) & (idx < nb))[valid].all())
    assert bool((idx[~valid] == -1).all())
    ascending = (idx[..., 1:] > idx[..., :-1]) | ~valid[..., 1:]
    assert bool(ascending.all())
    i = torch.arange(nb, device=idx.device)[None, None, :]
    for off in w.band:
        j = i + off
        inside = (j >= 0) & (j < nb)
        hit = ((idx == j[..., None]) & valid).any(-1)
        assert bool(hit[inside.expand_as(hit)].all()), f"band offset {off} missing"


def test_fullsize_outputs_finite(run):
    assert run[3]["finite"]


def test_fullsize_ordered_step_identical(run):
    """The processing order is a permutation on every head and changes no output bit."""
    assert run[3]["order_ok"]
    assert run[3]["ordered_same"]


def test_fullsize_ordered_refresh_identical(run):
    """A refresh step with a previous residual (has_prev = 1) writes the same
    full output, r and dr on every head in the computed processing order."""
    assert run[3]["refresh_same"]


def test_fullsize_sparse_sampled(run):
    w, heads, host, g, o = run
    sm = oracle.default_sm_scale(w.head_dim)
    blocks = _sample_blocks(w)
    which = [(0, hi, i) for hi in range(len(heads)) for i in blocks]
    want = oracle.attention(o["qc"], o["sq"], o["kc"], o["sk"], host["v"], o["idx"], o["cnt"],
                            w.block, sm, which=which)
    worst = (0.0, 0.0)
    for (b, hi, i), ref in want.items():
        t0 = i * w.block
        rel, mx = _close(g["sparse"][b, hi, t0:t0 + ref.shape[0]], ref,
                         f"{w.name} sparse head {heads[hi]} block {i}")
        worst = (max(worst[0], rel), max(worst[1], mx))
    print(f"[fullsize] {w.name} sparse: worst rel_l2={worst[0]:.2e} max_abs={worst[1]:.2e} "
          f"over {len(want)} blocks", flush=True)


def test_fullsize_refresh_and_sparse_step_sampled(run):
    """Refresh step (full output, r) and the next sparse step's output.

    The refresh output is held to the output tolerance.  The residual
    r = bf16(full - sparse) is a cancellation of two outputs: it is held to
    rel-L2 <= 5e-3 relative to the full output, and elementwise to the sum of
    the two outputs' error bounds plus its own bf16 rounding.  The sparse
    attention the sparse step computes is held to the output tolerance
    (rel-L2 <= 5e-3, max-abs <= 2e-2); the step output, that attention plus the
    kernel's own cached r and dr rounded to bf16, to rel-L2 <= 5e-3 and per
    element to the attention's measured error plus its roundings; and end to
    end to rel-L2 <= 5e-3 against the oracle's state machine."""
    w, heads, host, g, o = run
    sm = oracle.default_sm_scale(w.head_dim)
    blocks = _sample_blocks(w, seed=1)
    which = [(0, hi, i) for hi in range(len(heads)) for i in blocks]
    fi, fc = oracle.full_kept_lists(1, len(heads), w.n_blocks)
    o_full = oracle.attention(o["qc"], o["sq"], o["kc"], o["sk"], host["v"], fi, fc, w.block,
                              sm, which=which)
    o_sp = oracle.attention(o["qc"], o["sq"], o["kc"], o["sk"], host["v"], o["idx"], o["cnt"],
                            w.block, sm, which=which)
    worst = {"full": (0.0, 0.0), "r": (0.0, 0.0), "step": (0.0, 0.0)}
    for key, ref in o_full.items():
        b, hi, i = key
        t0, t1 = i * w.block, i * w.block + ref.shape[0]
        what = f"{w.name} head {heads[hi]} block {i}"
        rel, mx = _close(g["full"][b, hi, t0:t1], ref, what + " refresh output")
        worst["full"] = (max(worst["full"][0], rel), max(worst["full"][1], mx))
        rho = ref - o_sp[key]
        err = g["r"][b, hi, t0:t1] - rho
        rel_r = np.linalg.norm(err) / np.linalg.norm(ref)
        assert rel_r <= REL_L2, what + f" r: rel {rel_r:.3e}"
        bound = 2 * MAX_ABS + _half_ulp_bf16(rho)
        assert np.all(np.abs(err) <= bound), what + f" r: max {np.max(np.abs(err)):.3e}"
        worst["r"] = (max(worst["r"][0], rel_r), max(worst["r"][1], float(np.max(np.abs(err)))))
        # the sparse step adds the kernel's cached residuals to its sparse
        # attention: held to the output tolerance against the oracle's sparse
        # attention plus those same caches (the caches themselves are held
        # to the oracle's residual just above)
        got_step = g["step"][b, hi, t0:t1]
        want_own = o_sp[key] + g["r"][b, hi, t0:t1] + oracle.bf16_to_f64(
            g["dr_bits"][b, hi, t0:t1])
        # the attention part is held to the output tolerance, and the step
        # output per element to that attention's error plus its own rounding
        sp = g["sparse"][b, hi, t0:t1]
        _close(sp, o_sp[key], what + " sparse attention")
        e = got_step - want_own
        rel = np.linalg.norm(e) / np.linalg.norm(want_own)
        mx = float(np.max(np.abs(e)))
        bound = (np.abs(sp - o_sp[key]) + _half_ulp_bf16(sp) + _half_ulp_bf16(got_step)
                 + 2.0 ** -22 * (np.abs(got_step) + 1.0))
        assert rel <= REL_L2, what + f" sparse-step output (own caches): rel_l2={rel:.3e}"
        assert np.all(np.abs(e) <= bound), (
            what + f" sparse-step output (own caches): worst excess "
            f"{np.max(np.abs(e) - bound):.3e}")
        # end to end against the oracle's state machine: r = bf16(rho), dr = 0
        # at the first refresh
        st = oracle.ResidualState(rho.shape)
        oracle.refresh_step(st, ref, o_sp[key])
        want_step = oracle.sparse_step(st, o_sp[key])
        rel2 = np.linalg.norm(got_step - want_step) / np.linalg.norm(want_step)
        assert rel2 <= REL_L2, what + f" sparse-step output end to end: rel_l2={rel2:.3e}"
        worst["step"] = (max(worst["step"][0], rel), max(worst["step"][1], mx))
    assert np.all(g["dr_bits"] == 0), "dr must be 0 without a previous refresh"
    print(f"[fullsize] {w.name} " + " ".join(
        f"{k}: rel_l2={v[0]:.2e} max_abs={v[1]:.2e}" for k, v in worst.items()), flush=True)
