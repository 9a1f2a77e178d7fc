"""Seeded synthetic inputs for the QuantSparse attention hot path.

This module is shared by the HIP path, the CPU oracle, the tests and the
benchmark.  It holds only input synthesis (workload shapes and a seeded
random-field recipe); none of the method's arithmetic lives here.

The pages measure on real video-DiT activations (Wan2.1-1.3B/14B and
HunyuanVideo-13B generations, QuantSparse technical summary §4); neither the
models nor their prompts are available, so these fields stand in for the
attention inputs of those models, at their attention shapes.

Recipe, per (tensor in {Q, K, V}, batch b, head h):

* white N(0, 1) noise on the latent token grid (frames, height, width) for
  each of the D channels, smoothed by a separable 3-D Gaussian filter
  (sigma = 4 tokens, reflect boundary, truncated at 4 sigma) and normalised
  to zero mean and unit standard deviation per channel;
* plus ``noise_std`` * N(0, 1) white noise;
* Q and K only: ``outlier_channels`` channels, drawn per (tensor, b, h),
  are multiplied by ``outlier_gain``;
* tokens in raster order t = (f * height + y) * width + x;
* rounded to bf16 (round to nearest even);
* denoising step s > 0 adds ``drift_std`` * N(0, 1) to the fp32 state of
  step s - 1 before rounding.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "Workload",
    "WORKLOADS",
    "get_workload",
    "gaussian_filter_matrix",
    "f32_to_bf16_bits",
    "bf16_bits_to_f32",
    "make_qkv",
    "make_qkv_steps",
    "make_qkv_torch",
]

TENSOR_IDS = {"q": 0, "k": 1, "v": 2}


@dataclass(frozen=True)
class Workload:
    """Attention shape plus input recipe of one synthetic workload."""

    name: str
    cfg_id: int
    batch: int
    heads: int
    head_dim: int
    grid: tuple  # latent token grid (frames, height, width)
    block: int
    density: float  # fraction of key blocks kept by the top-k (1.0 = dense)
    band: tuple = (0,)  # block offsets always kept besides the top-k
    noise_std: float = 0.3
    outlier_channels: int = 3
    outlier_gain: float = 10.0
    field_sigma: float = 4.0
    drift_std: float = 0.05
    schedule: str = "FSSSS"  # F = full-attention refresh step, S = sparse step
    topk_override: int | None = None

    @property
    def seq_len(self) -> int:
        f, h, w = self.grid
        return f * h * w

    @property
    def n_blocks(self) -> int:
        return -(-self.seq_len // self.block)

    @property
    def topk(self) -> int:
        """Key blocks ranked in per query block: ceil(density * n_blocks)."""
        if self.topk_override is not None:
            return self.topk_override
        if self.density >= 1.0:
            return self.n_blocks
        return int(math.ceil(self.density * self.n_blocks - 1e-9))

    @property
    def kmax(self) -> int:
        """Row stride of the kept-block lists: enough for top-k plus band."""
        return min(self.n_blocks, self.topk + len(self.band))

    def with_(self, **kw) -> "Workload":
        d = dict(self.__dict__)
        d.update(kw)
        return Workload(**d)


# The shapes of the pages' workloads (QuantSparse technical summary §4 names
# Wan2.1 and HunyuanVideo at densities down to 15 %); token grids are the
# latent grids of those models at 480p / 720p.
WORKLOADS = {
    "tiny": Workload("tiny", 0, 1, 2, 64, (2, 8, 8), 64, 0.5, (0,), noise_std=1.0,
                     outlier_channels=1, outlier_gain=8.0, schedule="FSS",
                     topk_override=1),
    "wan13b_480p": Workload("wan13b_480p", 1, 1, 12, 128, (21, 30, 52), 64, 0.15),
    "wan14b_480p_d100": Workload("wan14b_480p_d100", 2, 1, 40, 128, (21, 30, 52), 64, 1.0),
    "wan14b_480p_d30": Workload("wan14b_480p_d30", 2, 1, 40, 128, (21, 30, 52), 64, 0.30),
    "wan14b_480p_d15": Workload("wan14b_480p_d15", 2, 1, 40, 128, (21, 30, 52), 64, 0.15),
    "wan14b_720p": Workload("wan14b_720p", 3, 1, 40, 128, (21, 45, 80), 64, 0.15),
    "hunyuan_720p": Workload("hunyuan_720p", 4, 1, 24, 128, (33, 45, 80), 128, 0.10,
                             band=(-28, 0, 28), noise_std=0.3),
}


def get_workload(name: str) -> Workload:
    return WORKLOADS[name]


# --------------------------------------------------------------------------
# bf16 bit handling for input synthesis
# --------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round finite float32 values to bf16 (nearest, ties to even); uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# --------------------------------------------------------------------------
# smooth random field
# --------------------------------------------------------------------------

def gaussian_filter_matrix(n: int, sigma: float, truncate: float = 4.0) -> np.ndarray:
    """n x n matrix of a 1-D Gaussian smoothing with half-sample reflection.

    Row i holds the weights that output position i gives to each input
    position; out-of-range taps reflect about the edge with period 2n.
    """
    radius = int(truncate * sigma + 0.5)
    offs = np.arange(-radius, radius + 1)
    w = np.exp(-0.5 * (offs / sigma) ** 2)
    w /= w.sum()
    g = np.zeros((n, n), dtype=np.float64)
    for i in range(n):
        p = (i + offs) % (2 * n)
        p = np.where(p >= n, 2 * n - 1 - p, p)
        np.add.at(g[i], p, w)
    return g


def _smooth_field(white: np.ndarray, mats) -> np.ndarray:
    """Apply the separable filter along the three grid axes of (F, H, W, D)."""
    x = white
    for axis, g in enumerate(mats):
        x = np.moveaxis(np.tensordot(g.astype(np.float32), x, axes=([1], [axis])), 0, axis)
    return np.ascontiguousarray(x)


def _seed(w: Workload, tensor: str, b: int, h: int, stream: int) -> np.random.Generator:
    ss = np.random.SeedSequence([w.cfg_id, TENSOR_IDS[tensor], b, h, stream])
    return np.random.Generator(np.random.PCG64(ss))


def _base_state(w: Workload, tensor: str, b: int, h: int, mats) -> np.ndarray:
    """fp32 state of one (tensor, b, h) at step 0, shape [L, D]."""
    f, hh, ww = w.grid
    d = w.head_dim
    rng = _seed(w, tensor, b, h, 0)
    white = rng.standard_normal((f, hh, ww, d), dtype=np.float32)
    fld = _smooth_field(white, mats).reshape(-1, d)
    mu = fld.mean(axis=0, dtype=np.float64)
    sd = fld.std(axis=0, dtype=np.float64)
    sd[sd == 0] = 1.0
    fld = ((fld - mu) / sd).astype(np.float32)
    x = fld + np.float32(w.noise_std) * rng.standard_normal(fld.shape, dtype=np.float32)
    if tensor in ("q", "k") and w.outlier_channels > 0:
        ch = rng.choice(d, size=w.outlier_channels, replace=False)
        x[:, ch] *= np.float32(w.outlier_gain)
    return x


def _drift(w: Workload, tensor: str, b: int, h: int, step: int, shape) -> np.ndarray:
    rng = _seed(w, tensor, b, h, 1000 + step)
    return np.float32(w.drift_std) * rng.standard_normal(shape, dtype=np.float32)


def make_qkv_steps(w: Workload, steps: int, heads=None, batches=None):
    """bf16 bits of (q, k, v) for denoising steps 0..steps-1.

    Returns a list (one entry per step) of dicts {"q", "k", "v"} holding
    uint16 arrays [B', H', L, D] for the requested batches/heads (default all).
    """
    heads = list(range(w.heads)) if heads is None else list(heads)
    batches = list(range(w.batch)) if batches is None else list(batches)
    mats = [gaussian_filter_matrix(n, w.field_sigma) for n in w.grid]
    L, D = w.seq_len, w.head_dim
    out = [{t: np.empty((len(batches), len(heads), L, D), np.uint16) for t in "qkv"}
           for _ in range(steps)]
    for t in "qkv":
        for bi, b in enumerate(batches):
            for hi, h in enumerate(heads):
                x = _base_state(w, t, b, h, mats)
                for s in range(steps):
                    if s > 0:
                        x = x + _drift(w, t, b, h, s, x.shape)
                    out[s][t][bi, hi] = f32_to_bf16_bits(x)
    return out


def make_qkv(w: Workload, step: int = 0, heads=None, batches=None):
    """bf16 bits of (q, k, v) at one denoising step (see make_qkv_steps)."""
    return make_qkv_steps(w, step + 1, heads, batches)[step]


def make_qkv_torch(w: Workload, device, step_seeds=(0,), heads=None):
    """Same recipe drawn with torch's generator on ``device`` (bf16 tensors).

    Used where numpy synthesis of a full-size workload would dominate the run
    (the benchmark).  The random stream differs from make_qkv's; shapes and
    statistics are the same.  Returns a list of dicts, one per entry of
    ``step_seeds`` (entry s > 0 adds s drift increments to the state).
    """
    import torch

    heads = w.heads if heads is None else heads
    f, hh, ww = w.grid
    D = w.head_dim
    mats = [torch.tensor(gaussian_filter_matrix(n, w.field_sigma), dtype=torch.float32,
                         device=device) for n in w.grid]
    gen = torch.Generator(device=device)
    res = [{} for _ in step_seeds]
    for tid, t in enumerate("qkv"):
        states = []
        for b in range(w.batch):
            per_h = []
            for h in range(heads):
                gen.manual_seed(((w.cfg_id * 7 + tid) * 1009 + b) * 100003 + h)
                white = torch.randn((f, hh, ww, D), generator=gen, device=device)
                x = torch.einsum("fg,ghwd->fhwd", mats[0], white)
                x = torch.einsum("hg,fgwd->fhwd", mats[1], x)
                x = torch.einsum("wg,fhgd->fhwd", mats[2], x).reshape(-1, D)
                x = (x - x.mean(0)) / x.std(0, unbiased=False).clamp_min(1e-30)
                x = x + w.noise_std * torch.randn(x.shape, generator=gen, device=device)
                if t in "qk" and w.outlier_channels > 0:
                    ch = torch.randperm(D, generator=gen, device=device)[: w.outlier_channels]
                    x[:, ch] *= w.outlier_gain
                per_h.append(x)
            states.append(torch.stack(per_h))
        x = torch.stack(states)  # [B, H, L, D] fp32
        done = 0
        for si, s in enumerate(step_seeds):
            while done < s:
                done += 1
                x = x + w.drift_std * torch.randn(x.shape, generator=gen, device=device)
            res[si][t] = x.to(torch.bfloat16).contiguous()
        del x, states
    return res
