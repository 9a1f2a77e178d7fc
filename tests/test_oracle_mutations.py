"""Plant plausible mistakes in the oracle (on the CPU) and check a pin catches each.

Each case swaps one oracle step for a subtly wrong variant (a dropped term, a
wrong rounding, a flipped sign, a transposed operand, the wrong tie order)
and runs the pin that should notice it; the pin must fail.
"""
import numpy as np
import pytest

import oracle
from oracle import qsa_oracle as Q
from tests import test_oracle_attention as TA
from tests import test_oracle_quantize as TQ
from tests import test_oracle_residual as TR
from tests import test_oracle_rotation as TH
from tests import test_oracle_projection as TP
from tests import test_oracle_trigger as TT
from tests import test_oracle_squad as TQS
from tests import test_oracle_select as TS


def _floor_quantize(x_bits, block):
    codes, scales, pooled = ORIG_QUANTIZE(x_bits, block)
    x = Q._bf16_to_f32(x_bits)
    for i in range(scales.shape[-1]):
        s = scales[0, 0, i]
        if s > 0:
            sl = slice(i * block, (i + 1) * block)
            codes[0, 0, sl] = np.clip(np.floor(x[0, 0, sl] / s + np.float32(0.5)), -127, 127)
    return codes, scales, pooled


def _scores_no_count(pq, sq, pk, sk, L, block):
    return ORIG_SCORES(pq, sq, pk, sk, L, block) * (block * block) / (block * block) * \
        _counts(L, block)


def _counts(L, block):
    n = np.array([t1 - t0 for t0, t1 in Q.block_bounds(L, block)], np.float64)
    return n[:, None] * n[None, :]


def _select_high_ties(scores, topk, band, kmax):
    nb = scores.shape[-1]
    flipped = scores[..., ::-1]
    idx, cnt = ORIG_SELECT(flipped, topk, [-o for o in band], kmax)
    out = np.full_like(idx, -1)
    for b in range(idx.shape[0]):
        for h in range(idx.shape[1]):
            for i in range(nb):
                lst = sorted(nb - 1 - j for j in idx[b, h, nb - 1 - i, : cnt[b, h, nb - 1 - i]])
                out[b, h, i, : len(lst)] = lst
    return out, cnt[..., ::-1].copy()


def _attention_no_kscale(qc, sq, kc, sk, v, idx, cnt, block, sm, which=None):
    return ORIG_ATTN(qc, sq, kc, np.ones_like(sk) * sk.mean(), v, idx, cnt, block, sm, which)


def _attention_transposed_v(qc, sq, kc, sk, v, idx, cnt, block, sm, which=None):
    vt = v.copy()
    vt[..., :, :] = v[..., ::-1, :]
    return ORIG_ATTN(qc, sq, kc, sk, vt, idx, cnt, block, sm, which)


def _refresh_flipped(state, o_full, o_sparse):
    return ORIG_REFRESH(state, o_sparse, o_full)


def _fwht_swapped_sign(x):
    # pairs become (a + b, b - a): H with its lower-right blocks negated twice over
    y = np.array(x, dtype=np.float32, copy=True)
    D = y.shape[-1]
    h = 1
    while h < D:
        g = y.reshape(y.shape[:-1] + (D // (2 * h), 2, h))
        a, b = g[..., 0, :].copy(), g[..., 1, :].copy()
        g[..., 0, :], g[..., 1, :] = a + b, b - a
        y = g.reshape(y.shape)
        h *= 2
    return y


def _fwht_last_stage_dropped(x):
    y = np.array(x, dtype=np.float32, copy=True)
    D = y.shape[-1]
    h = 1
    while h < D // 2:
        g = y.reshape(y.shape[:-1] + (D // (2 * h), 2, h))
        a, b = g[..., 0, :].copy(), g[..., 1, :].copy()
        g[..., 0, :], g[..., 1, :] = a + b, a - b
        y = g.reshape(y.shape)
        h *= 2
    return y


def _quantize_rotated_unrotated(x_bits, block):
    return ORIG_QUANTIZE(x_bits, block)


def _project_with(pick, scale_basis=False):
    def bad(dr_bits, rank):
        x = Q.bf16_to_f64(dr_bits)
        out = np.empty_like(x)
        vals = np.empty(x.shape[:2] + (rank,))
        for b in range(x.shape[0]):
            for h in range(x.shape[1]):
                w, V = np.linalg.eigh(x[b, h].T @ x[b, h])
                top = pick(w)[:rank]
                Vr = V[:, top] * (np.sqrt(np.maximum(w[top], 0)) if scale_basis else 1.0)
                out[b, h] = (x[b, h] @ Vr) @ Vr.T
                vals[b, h] = w[top]
        return out, vals
    return bad


_project_smallest = _project_with(lambda w: np.argsort(w, kind="stable"))
_project_unnormalised = _project_with(lambda w: np.argsort(-w, kind="stable"), scale_basis=True)


def _refresh_unprojected(state, o_full, o_sparse, rank=None):
    return ORIG_REFRESH(state, o_full, o_sparse)


def _l1_over_current(prev_bits, cur_bits):
    num, _ = ORIG_L1(prev_bits, cur_bits)
    return num, float(np.abs(Q.bf16_to_f64(cur_bits)).sum())


def _squad_variant(values_v=False, group_w=False, unpermute=True):
    def bad(q_bits, k_bits, v_bits, window, block, sm_scale=None):
        B, H, n, D = q_bits.shape
        sm = Q.default_sm_scale(D)
        qc, sq, _ = Q.quantize(q_bits, block)
        kc, sk, _ = Q.quantize(k_bits, block)
        idx, cnt = Q.window_kept_lists(B, H, n, window, block)
        o_local = Q.f64_to_bf16(Q.attention(qc, sq, kc, sk, v_bits, idx, cnt, block, sm))
        m = n // window
        qc, sq, _ = Q.quantize(Q.to_position_major(q_bits, window), block)
        kc, sk, _ = Q.quantize(Q.to_position_major(k_bits, window), block)
        idx, cnt = Q.window_kept_lists(B, H, n, window if group_w else m, block)
        vals = v_bits if values_v else o_local
        o = Q.attention(qc, sq, kc, sk, Q.to_position_major(vals, window), idx, cnt, block, sm)
        return Q.from_position_major(o, window) if unpermute else o
    return bad


def _pm_identity(x, window):
    return np.ascontiguousarray(x)


class _TriggerNoReset(Q.RefreshTrigger):
    def update(self, num=None, den=None):
        if num is None:
            return super().update()
        self.c += num / den if den > 0 else (0.0 if num == 0 else float("inf"))
        self.refresh_next = self.c > self.delta
        return self.refresh_next


class _TriggerAtOrAbove(Q.RefreshTrigger):
    def update(self, num=None, den=None):
        if num is None:
            return super().update()
        self.c += num / den if den > 0 else (0.0 if num == 0 else float("inf"))
        self.refresh_next = self.c >= self.delta
        if self.refresh_next:
            self.c = 0.0
        return self.refresh_next


ORIG_QUANTIZE = Q.quantize
ORIG_SCORES = Q.block_scores
ORIG_SELECT = Q.select_blocks
ORIG_ATTN = Q.attention
ORIG_REFRESH = Q.refresh_step
ORIG_L1 = Q.l1_change

CASES = [
    ("quantize", _floor_quantize, lambda: TQ.test_half_integer_ties_round_to_even()),
    ("block_scores", _scores_no_count, lambda: TS.test_scores_against_exact_rationals()),
    ("select_blocks", _select_high_ties,
     lambda: TS.test_selection_against_brute_force_sort(12, 1, ())),
    ("attention", _attention_no_kscale,
     lambda: TA.test_sparse_attention_equals_masked_sdpa((1, 10, 30), 64, 64, 2, (0,))),
    ("attention", _attention_transposed_v, lambda: TA.test_hand_examples_outputs("H2_band0")),
    ("refresh_step", _refresh_flipped, lambda: TR.test_refresh_and_sparse_step_hand_values()),
    ("fwht", _fwht_swapped_sign, lambda: TH.test_fwht_equals_sylvester_product_exactly(8)),
    ("fwht", _fwht_last_stage_dropped, lambda: TH.test_fwht_algebra(64)),
    ("fwht", _fwht_last_stage_dropped, lambda: TH.test_rotated_quantisation_of_exactly_rotatable_rows()),
    ("quantize_rotated", _quantize_rotated_unrotated,
     lambda: TH.test_rotated_quantisation_of_exactly_rotatable_rows()),
    ("project_residual", _project_smallest, lambda: TP.test_hand_example_rank_one()),
    ("project_residual", _project_smallest,
     lambda: TP.test_projection_equals_truncated_svd(200, 64, 8)),
    ("project_residual", _project_unnormalised, lambda: TP.test_hand_example_axis_aligned()),
    ("project_residual", _project_unnormalised,
     lambda: TP.test_eckart_young_energy_and_orthogonality()),
    ("refresh_step", _refresh_unprojected,
     lambda: TP.test_refresh_step_projects_only_the_second_order_residual()),
    ("l1_change", _l1_over_current, lambda: TT.test_l1_change_closed_forms()),
    ("RefreshTrigger", _TriggerNoReset, lambda: TT.test_trigger_hand_sequence()),
    ("RefreshTrigger", _TriggerAtOrAbove, lambda: TT.test_trigger_hand_sequence()),
    ("squad_attention", _squad_variant(values_v=True),
     lambda: TQS.test_squad_equals_masked_definition(4096, 64)),
    ("squad_attention", _squad_variant(group_w=True),
     lambda: TQS.test_squad_equals_masked_definition(8192, 64)),
    ("squad_attention", _squad_variant(unpermute=False),
     lambda: TQS.test_squad_equals_masked_definition(4096, 64)),
    ("to_position_major", _pm_identity, lambda: TQS.test_position_major_index_formula()),
]


@pytest.mark.parametrize("name,bad,pin", CASES, ids=[f"{c[0]}-{c[1].__name__}" for c in CASES])
def test_planted_mistake_is_caught(monkeypatch, name, bad, pin):
    monkeypatch.setattr(Q, name, bad)
    monkeypatch.setattr(oracle, name, bad)
    with pytest.raises(AssertionError):
        pin()
