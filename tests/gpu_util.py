"""Helpers of the GPU parity tests: host<->device transfer and error metrics."""
import numpy as np
import torch

import oracle
import qsa_gen

# Output tolerance of the bf16 attention outputs against the fp64 oracle.
REL_L2 = 5e-3
MAX_ABS = 2e-2


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def host_f64(t: torch.Tensor) -> np.ndarray:
    return oracle.bf16_to_f64(host_bits(t))


def rel_l2(got, want) -> float:
    want = np.asarray(want, np.float64)
    den = np.linalg.norm(want)
    return float(np.linalg.norm(np.asarray(got, np.float64) - want) / (den if den > 0 else 1.0))


def assert_close(got, want, rel=REL_L2, atol=MAX_ABS, what=""):
    r = rel_l2(got, want)
    m = float(np.max(np.abs(np.asarray(got, np.float64) - want))) if np.size(want) else 0.0
    assert r <= rel and m <= atol, f"{what}: rel_l2={r:.3e} (<= {rel}) max_abs={m:.3e} (<= {atol})"
    return r, m


def oracle_front(x, w, topk=None, band=None, kmax=None):
    """Oracle quantise + select on host bits; returns a dict of arrays."""
    qc, sq, pq = oracle.quantize(x["q"], w.block)
    kc, sk, pk = oracle.quantize(x["k"], w.block)
    sc = oracle.block_scores(pq, sq, pk, sk, w.seq_len, w.block)
    topk = w.topk if topk is None else topk
    band = w.band if band is None else band
    kmax = min(w.n_blocks, topk + len(band)) if kmax is None else kmax
    idx, cnt = oracle.select_blocks(sc, topk, band, kmax)
    return dict(qc=qc, sq=sq, pq=pq, kc=kc, sk=sk, pk=pk, idx=idx, cnt=cnt, topk=topk,
                band=band, kmax=kmax)
