"""Pins of the oracle's adaptive refresh trigger: the normalised L1 change of
consecutive outputs accumulated against a threshold (DVD-Quant,
gist.science/es/paper/2505.18663, technical summary §2C), read as the
trigger of a full-attention refresh step."""
import numpy as np
import pytest

import oracle


def _bits(x):
    return oracle.f64_to_bf16(np.asarray(x, np.float64))


def test_l1_change_closed_forms():
    rng = np.random.default_rng(0)
    x = _bits(rng.standard_normal((1, 2, 50, 64)))
    xv = oracle.bf16_to_f64(x)
    assert oracle.l1_change(x, x) == (0.0, float(np.abs(xv).sum()))
    num, den = oracle.l1_change(x, _bits(2 * xv))   # doubling is exact in bf16
    assert num == den
    num, den = oracle.l1_change(x, _bits(-xv))      # sign flip: twice the norm
    assert num == 2 * den
    num, den = oracle.l1_change(x, np.zeros_like(x))
    assert num == den


def test_l1_change_hand_example():
    prev = _bits([[1.0, -2.0, 0.5, 0.0]])
    cur = _bits([[1.5, -2.0, -0.5, 0.25]])
    assert oracle.l1_change(prev, cur) == (0.5 + 0.0 + 1.0 + 0.25, 3.5)


def test_l1_change_scale_invariance():
    rng = np.random.default_rng(1)
    a, b = (rng.standard_normal((3, 40)) for _ in range(2))
    n1, d1 = oracle.l1_change(_bits(a), _bits(b))
    n2, d2 = oracle.l1_change(_bits(8 * oracle.bf16_to_f64(_bits(a))),
                              _bits(8 * oracle.bf16_to_f64(_bits(b))))
    assert n2 == 8 * n1 and d2 == 8 * d1


def test_trigger_hand_sequence():
    t = oracle.RefreshTrigger(0.1)
    assert t.refresh_next  # the first step always refreshes
    assert t.update() is False  # and the one after it is sparse
    seq = [0.03, 0.04, 0.05, 0.02, 0.2, 0.0, 0.1, 0.001]
    got = [t.update(d, 1.0) for d in seq]
    # c: .03 .07 .12>.1 (reset) .02 .22>.1 (reset) 0 .1 (not > .1) .101>.1
    assert got == [False, False, True, False, True, False, False, True]
    assert t.c == 0.0


def test_trigger_zero_denominator():
    t = oracle.RefreshTrigger(0.5)
    assert t.update(0.0, 0.0) is False
    assert t.update(1e-30, 0.0) is True


@pytest.mark.parametrize("delta", [0.0, 1e9])
def test_trigger_extremes(delta):
    t = oracle.RefreshTrigger(delta)
    got = [t.update(d, 1.0) for d in (0.01, 0.2, 0.3)]
    assert got == ([True] * 3 if delta == 0.0 else [False] * 3)
