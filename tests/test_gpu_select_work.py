"""qsa_select_blocks_work against qsa_select_blocks, bit for bit.

The workspace variant computes the same block scores (QuantSparse,
gist.science/es/paper/2509.23681, technical summary §2A: pooled saliency,
top-k) in a separate pass that writes 64-bit order keys to the caller's
scratch, then selects one query block per wave.  Its kept lists and counts
must equal the one-pass kernel's exactly (and so the oracle's, which the
select tests of test_gpu_parity.py check for both entry points):

* the slices of a call are split into passes by the workspace size: one,
  two and four slices per pass of six, and the whole call in one pass;
* no workspace, or less than one slice of it, runs the one-pass kernel;
* each register width of the select pass (rows of up to 1,024, 1,536 and
  2,048 blocks), head_dim 64 and 128, ragged last blocks;
* more than 2,048 blocks falls back to the one-pass kernel;
* the full Wan-14B 720p shape, all 40 heads;
* rows whose scores agree in the high 32 bits of their order keys and differ
  below (the select orders such ties by the low halves), with exact
  duplicates among them (index order), against the oracle on every row.
"""
import numpy as np
import pytest
import torch

import oracle
import qsa_gen
from quantized_sparse_attention_amd import binding as B

pytestmark = pytest.mark.gpu

TINY = qsa_gen.get_workload("tiny")


def _front(w, heads=None):
    x = qsa_gen.make_qkv_torch(w, torch.device("cuda"), heads=heads)[0]
    qc, qs, qp = B.qsa_quantize(x["q"], w.block)
    kc, ks, kp = B.qsa_quantize(x["k"], w.block)
    return qp, qs, kp, ks


def _select(front, w, topk, band, kmax, work=None):
    qp, qs, kp, ks = front
    idx, cnt = B.qsa_select_blocks(qp, qs, kp, ks, w.seq_len, w.block, topk, band, kmax, work=work)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), cnt.cpu().numpy()


def _work(nbytes):
    return torch.empty(max(nbytes, 16), dtype=torch.uint8, device="cuda")


def _same(a, b, what):
    assert np.array_equal(a[1], b[1]), f"{what}: kept counts differ"
    assert np.array_equal(a[0], b[0]), f"{what}: kept lists differ"


def test_passes_split_by_the_workspace():
    # 2 x 3 slices of 1,581 tokens (25 blocks, the last one ragged)
    w = TINY.with_(batch=2, heads=3, grid=(3, 17, 31), head_dim=128, noise_std=0.3,
                   outlier_channels=3, outlier_gain=10.0)
    front = _front(w)
    slice_b = B.qsa_select_slice_bytes(w.batch, w.heads, w.seq_len, w.head_dim, w.block)
    assert slice_b == w.n_blocks * (-(-w.n_blocks // 16) * 16) * 8
    for topk, band in [(4, (0,)), (1, (-1, 0, 1)), (25, (0,)), (0, (0,))]:
        kmax = min(w.n_blocks, topk + len(band))
        want = _select(front, w, topk, band, kmax)
        for per in (1, 2, 4, 6):
            got = _select(front, w, topk, band, kmax, _work(per * slice_b + 8))
            _same(got, want, f"topk={topk} band={band} {per} slices per pass")
        # less than one slice: the one-pass kernel
        _same(_select(front, w, topk, band, kmax, _work(slice_b - 8)), want, "small workspace")


# token grids (the generator filters along each grid axis) whose block counts
# fall in each register width, with ragged last blocks
@pytest.mark.parametrize("grid,D,block,nb", [((7, 89, 102), 128, 64, 993),
                                             ((11, 87, 100), 128, 64, 1496),
                                             ((13, 97, 101), 128, 64, 1991),
                                             ((11, 87, 100), 64, 64, 1496),
                                             ((7, 99, 129), 128, 128, 699)])
def test_register_widths(grid, D, block, nb):
    w = TINY.with_(grid=grid, head_dim=D, block=block, heads=2, noise_std=0.3,
                   outlier_channels=2, outlier_gain=10.0)
    assert w.n_blocks == nb and w.seq_len % block
    front = _front(w)
    topk = (15 * nb + 99) // 100
    want = _select(front, w, topk, (0,), topk + 1)
    got = _select(front, w, topk, (0,), topk + 1,
                  _work(B.qsa_select_slice_bytes(1, 2, w.seq_len, D, block) * 2))
    _same(got, want, f"nb={nb} D={D} block={block}")


def test_long_rows_fall_back():
    w = TINY.with_(grid=(15, 99, 91), head_dim=128, heads=1)  # 2,112 blocks
    assert w.n_blocks > 2048
    front = _front(w)
    want = _select(front, w, 300, (0,), 301)
    got = _select(front, w, 300, (0,), 301,
                  _work(B.qsa_select_slice_bytes(1, 1, w.seq_len, 128, 64)))
    _same(got, want, f"nb={w.n_blocks}")


def test_fullsize_720p_all_heads():
    w = qsa_gen.get_workload("wan14b_720p")
    front = _front(w)
    want = _select(front, w, w.topk, w.band, w.kmax)
    slice_b = B.qsa_select_slice_bytes(w.batch, w.heads, w.seq_len, w.head_dim, w.block)
    got = _select(front, w, w.topk, w.band, w.kmax, _work(8 * slice_b))  # five passes
    _same(got, want, "720p")


@pytest.mark.parametrize("nb", [300, 1300, 2000])
def test_high_half_ties(nb):
    """Pooled sums built so that S_ij = 127 * 8128^2 + pq[i,127] * pk[j,127]
    with pq[i,127] in [1, 8]: a row's scores lie within about 2^-16 of each
    other, so tens of keys share their high 32 bits (sign, exponent, top 20
    mantissa bits) and the order among them is in the low bits.  30-50 % of
    a head's columns take one of max(30, nb/10) shared sums, so the tied sets
    also hold exact duplicates (index order; exact ties at the k-th place
    themselves are the ties-and-ranges tests' case).  Equal scales, full
    blocks (L = 64 nb); all rows of a head share the column order, so eight
    heads give eight boundary cases."""
    rng = np.random.default_rng(nb)
    H, D, bs = 8, 128, 64
    L = nb * bs
    pq = np.full((1, H, nb, D), 8128, np.int32)
    pk = np.full((1, H, nb, D), 8128, np.int32)
    pq[..., 127] = rng.integers(1, 9, size=(1, H, nb))
    last = rng.integers(-8128, 8129, size=(1, H, nb))
    ns = max(30, nb // 10)
    shared = rng.integers(-8128, 8129, size=ns)
    dup = rng.random((1, H, nb)) < rng.uniform(0.3, 0.5, size=(1, H, 1))
    last[dup] = shared[rng.integers(0, ns, size=int(dup.sum()))]
    pk[..., 127] = last
    sq = np.full((1, H, nb), np.float32(1.0) / np.float32(127.0), np.float32)
    sk = sq.copy()
    topk = (15 * nb + 99) // 100
    kmax = topk + 1
    scores = oracle.block_scores(pq, sq, pk, sk, L, bs)
    want_idx, want_cnt = oracle.select_blocks(scores, topk, (0,), kmax)
    # the case is what it claims: at the k-th place, high halves tied with the
    # low halves apart
    srt = np.sort(scores, axis=-1)[..., ::-1]
    a, b = srt[..., topk - 1], srt[..., topk]
    hi_tie = (a.view(np.uint64) >> np.uint64(32)) == (b.view(np.uint64) >> np.uint64(32))
    assert np.mean(hi_tie & (a != b)) > 0.5
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()  # noqa: E731
    front = (dev(pq), dev(sq), dev(pk), dev(sk))
    w = TINY.with_(grid=(1, 1, L), head_dim=D, block=bs, heads=H)
    for work in (None, _work(B.qsa_select_slice_bytes(1, H, L, D, bs) * H)):
        got = _select(front, w, topk, (0,), kmax, work)
        what = "one pass" if work is None else "workspace"
        assert np.array_equal(got[1], want_cnt), f"{what}: counts"
        assert np.array_equal(got[0], want_idx), f"{what}: kept lists"
