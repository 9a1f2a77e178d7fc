"""Per-layer step driver of the QuantSparse attention hot path.

Holds one layer's residual cache across denoising steps (QuantSparse,
gist.science/es/paper/2509.23681, technical summary §2B: first- and
second-order residuals cached and reused on sparse steps) and issues the
C-ABI calls of one step on the current torch stream.  All arithmetic runs in
libqsa.so.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch

from . import binding as B


@dataclass
class QSAConfig:
    block: int = 64
    topk: int = 1
    band: tuple = (0,)
    sm_scale: float | None = None
    order: int = 2  # 2: sparse + r + dr; 1: sparse + r (first-order reuse)
    # process the query blocks in an order that groups blocks with
    # overlapping kept sets (same outputs bit for bit, more shared key-tile
    # loads): "refresh" computes it at refresh steps (and whenever the layer
    # has none for the input shape) and reuses it on the sparse steps until
    # the next refresh, as the kept sets drift slowly between refreshes;
    # "step" recomputes it at every step; "off" keeps ascending order.
    # True and False stand for "refresh" and "off".
    reorder: str | bool = "refresh"
    # quantise Hadamard-rotated Q and K rows (DVD-Quant,
    # gist.science/es/paper/2505.18663, technical summary §2B); attention then
    # runs with sm_scale / head_dim
    rotate: bool = False
    # rank of the SVD projection of the second-order residual at refresh steps
    # (technical summary §2B); None keeps the full residual
    rank: int | None = None
    # adaptive refresh: with a threshold, step(..., refresh=None) refreshes
    # once the accumulated normalised L1 change of this layer's consecutive
    # outputs passes it (DVD-Quant, gist.science/es/paper/2505.18663,
    # technical summary §2C); None keeps caller-chosen refresh steps
    adaptive_delta: float | None = None
    # select through qsa_select_blocks_work with a workspace for every
    # (batch, head) slice's score keys (same kept lists; the layer allocates
    # it once per shape, 8 * nb * nb bytes per slice); False: qsa_select_blocks
    select_workspace: bool = True


@dataclass
class StepBuffers:
    """Outputs of one step, kept for inspection (codes, scales, masks)."""
    q_codes: torch.Tensor = None
    q_scales: torch.Tensor = None
    q_pooled: torch.Tensor = None
    k_codes: torch.Tensor = None
    k_scales: torch.Tensor = None
    k_pooled: torch.Tensor = None
    kept_idx: torch.Tensor = None
    kept_cnt: torch.Tensor = None


class QuantSparseAttention:
    """One attention layer: refresh steps update the residual cache, sparse
    steps add it to the block-sparse output."""

    def __init__(self, cfg: QSAConfig):
        self.cfg = cfg
        self.r = None
        self.dr = None
        self.has_prev = False
        self.last = StepBuffers()
        self.work = None      # scratch of the residual projection
        self.basis = None     # its last basis [B,H,D,rank] and eigenvalues
        self.eigvals = None
        # adaptive refresh trigger state
        self.prev_out = None
        self.change = 0.0       # accumulated normalised L1 change
        self.refresh_next = True
        self.order = None       # processing order of the query blocks (reorder)
        self.last_sums = None   # (sum|O_t - O_t-1|, sum|O_t-1|) of the last step
        self.l1_work = None
        self.l1_sums = None
        self.sel_work = None    # score keys of qsa_select_blocks_work

    def reset(self):
        self.r = self.dr = None
        self.has_prev = False
        self.prev_out = None
        self.change = 0.0
        self.refresh_next = True
        self.order = None

    def state_dict(self):
        """A snapshot of the residual cache and trigger state.  Tensors are
        copies: later steps write r, dr and the previous output in place, and
        must not change a snapshot already taken."""
        cp = lambda t: None if t is None else t.clone()  # noqa: E731
        return {"r": cp(self.r), "dr": cp(self.dr), "has_prev": self.has_prev,
                "prev_out": cp(self.prev_out), "change": self.change,
                "refresh_next": self.refresh_next}

    def load_state_dict(self, sd):
        """Restore a snapshot; the layer keeps copies of its tensors, so the
        snapshot stays valid after later steps."""
        cp = lambda t: None if t is None else t.clone()  # noqa: E731
        self.r, self.dr, self.has_prev = cp(sd["r"]), cp(sd["dr"]), bool(sd["has_prev"])
        self.prev_out = cp(sd.get("prev_out"))
        self.change = float(sd.get("change", 0.0))
        self.refresh_next = bool(sd.get("refresh_next", self.r is None))

    def _sm_scale(self, head_dim: int):
        c = self.cfg
        if not c.rotate:
            return c.sm_scale
        sm = B.default_sm_scale(head_dim) if c.sm_scale is None else float(c.sm_scale)
        return sm / head_dim  # exact: head_dim is a power of two

    def _front(self, q, k):
        c = self.cfg
        quant = B.qsa_quantize_rotated if c.rotate else B.qsa_quantize
        qc, qs, qp = quant(q, c.block)
        kc, ks, kp = quant(k, c.block)
        work = None
        if c.select_workspace:
            Bn, H, L, D = q.shape
            n = B.qsa_select_slice_bytes(Bn, H, L, D, c.block) * Bn * H
            if self.sel_work is None or self.sel_work.numel() != n or self.sel_work.device != q.device:
                self.sel_work = torch.empty(n, dtype=torch.uint8, device=q.device)
            work = self.sel_work
        idx, cnt = B.qsa_select_blocks(qp, qs, kp, ks, q.shape[2], c.block, c.topk, c.band,
                                       work=work)
        self.last = StepBuffers(qc, qs, qp, kc, ks, kp, idx, cnt)
        return qc, qs, kc, ks, idx, cnt

    def step(self, q, k, v, refresh: bool | None = None) -> torch.Tensor:
        """One denoising step of this layer.  ``refresh=None`` lets the
        adaptive trigger decide (needs ``adaptive_delta``)."""
        c = self.cfg
        if refresh is None:
            if c.adaptive_delta is None:
                raise ValueError("refresh=None needs QSAConfig.adaptive_delta")
            refresh = self.refresh_next or self.r is None
        out = self._step(q, k, v, refresh)
        if c.adaptive_delta is not None:
            self._account(out)
        return out

    def _account(self, out):
        """Accumulate the normalised L1 change of consecutive outputs and set
        whether the next step refreshes (one small device-to-host copy)."""
        if self.prev_out is None:
            self.prev_out = out.clone()
            self.refresh_next = False
            self.last_sums = None
            return
        if self.l1_work is None:
            self.l1_work = torch.empty(B.QSA_L1_WORK_BYTES, dtype=torch.uint8, device=out.device)
            self.l1_sums = torch.empty(2, dtype=torch.float64, device=out.device)
        num, den = B.qsa_l1_change(self.prev_out, out, self.l1_sums, self.l1_work).tolist()
        self.last_sums = (num, den)
        d = num / den if den > 0 else (0.0 if num == 0 else float("inf"))
        self.change += d
        self.refresh_next = self.change > self.cfg.adaptive_delta
        if self.refresh_next:
            self.change = 0.0
        self.prev_out.copy_(out)

    def _reorder_mode(self) -> str:
        m = self.cfg.reorder
        m = "refresh" if m is True else "off" if m is False else m
        if m not in ("refresh", "step", "off"):
            raise ValueError(f"QSAConfig.reorder must be 'refresh', 'step' or 'off', not {m!r}")
        return m

    def _order(self, idx, cnt, L: int, D: int, refresh: bool):
        """The processing order for this step (None: ascending order)."""
        mode = self._reorder_mode()
        if mode == "off":
            return None
        stale = self.order is None or self.order.shape != cnt.shape
        if mode == "step" or refresh or stale:
            self.order = B.qsa_order_query_blocks(idx, cnt, L, self.cfg.block, D)
        return self.order

    def _step(self, q, k, v, refresh: bool) -> torch.Tensor:
        c = self.cfg
        qc, qs, kc, ks, idx, cnt = self._front(q, k)
        sm = self._sm_scale(q.shape[3])
        order = self._order(idx, cnt, q.shape[2], q.shape[3], refresh)
        if refresh:
            if self.r is None:
                self.r = torch.zeros_like(v)
                self.dr = torch.zeros_like(v)
            out = B.qsa_full_attn_residual(qc, qs, kc, ks, v, idx, cnt, c.block, self.r, self.dr,
                                           self.has_prev, sm, order=order)
            if c.rank is not None and self.has_prev:
                Bn, H, L, D = v.shape
                need = B.qsa_project_work_bytes(Bn, H, L, D, c.rank)
                if self.work is None or self.work.numel() < need:
                    self.work = torch.empty(need, dtype=torch.uint8, device=v.device)
                self.basis, self.eigvals = B.qsa_project_residual(self.dr, c.rank, work=self.work)
            self.has_prev = True
            return out
        if self.r is None:
            raise RuntimeError("sparse step before any full-attention refresh step")
        dr = self.dr if c.order == 2 else None
        if order is not None:
            return B.qsa_sparse_attn_ordered(qc, qs, kc, ks, v, idx, cnt, order, c.block,
                                             sm, r=self.r, dr=dr)
        return B.qsa_sparse_attn(qc, qs, kc, ks, v, idx, cnt, c.block, sm, r=self.r,
                                 dr=dr)
