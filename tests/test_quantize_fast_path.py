"""CPU pin of the quantiser kernel's division-free code path.

The gfx950 quantiser (csrc/quantize.hip, ``codes8``) does not divide every
element by the block scale.  With s = fl32(amax / 127) and inv = fl32(1 / s)
it takes p = fl32(x * inv) and c = rint(p), and falls back to the IEEE
quotient rint(fl32(x / s)) only when |p - c| > 1/2 - 2^-15 (a quotient within
reach of a half-integer) or when s < 2^-100 (where 1 / s would leave the
normal range).  The
oracle's step 1 (R2: code = clamp(rint(fl32(x / s)), -127, 127), QuantSparse,
gist.science/es/paper/2509.23681, technical summary §1 and §4: 8-bit
activations) always divides.

This test runs that sequence of fp32 operations on the CPU, each written out
with NumPy's IEEE fp32 arithmetic, for every finite bf16 amax as block maximum
and every finite bf16 x whose quotient reaches at least 1/8 in magnitude
(smaller quotients round to 0 on every path), and requires the codes to equal
the oracle's bit for bit.  It also reports how rarely the division is taken.
"""
import numpy as np
import pytest

import oracle
import qsa_gen

F32 = np.float32


def _all_finite_bf16_magnitudes():
    bits = np.arange(0x0001, 0x7F80, dtype=np.uint32).astype(np.uint16)  # +0 excluded
    return qsa_gen.bf16_bits_to_f32(bits)


def _codes_fast_path(x, s):
    """The kernel's code path on fp32 arrays x (values) and s (their block scale, > 0)."""
    x = x.astype(F32)
    s = s.astype(F32)
    fast = s >= F32(2.0 ** -100)
    with np.errstate(divide="ignore", over="ignore"):
        inv = np.where(fast, F32(1.0) / s, F32(0.0)).astype(F32)
    p = (x * inv).astype(F32)
    q = np.rint(p).astype(F32)
    band = ~(np.abs((p - q).astype(F32)) <= F32(0.5 - 2.0 ** -15))
    div = ~fast | band
    with np.errstate(divide="ignore", invalid="ignore"):
        qd = np.rint((x / s).astype(F32)).astype(F32)
    q = np.where(div, qd, q)
    return np.clip(q, -127, 127).astype(np.int8), div


def _blocks_for(amaxes, mags):
    """One block row per amax: [amax, then every bf16 x with |x| in [amax/1024, amax], both
    signs], padded with amax; returns the bf16 bits [1, 1, n_rows, width]."""
    rows = []
    for am in amaxes:
        m = mags[(mags >= am * F32(2.0 ** -10)) & (mags <= am)]
        rows.append(np.concatenate([[am], m, -m]).astype(F32))
    width = max(len(r) for r in rows)
    width += (-width) % 8
    out = np.empty((len(rows), width), F32)
    for i, r in enumerate(rows):
        out[i, : len(r)] = r
        out[i, len(r):] = r[0]
    return qsa_gen.f32_to_bf16_bits(out)[None, None]


@pytest.mark.parametrize("part", range(4))
def test_division_free_codes_match_oracle_on_every_bf16_amax(part):
    mags = _all_finite_bf16_magnitudes()
    amaxes = mags[part::4]  # the four parts together cover every finite bf16 amax
    total = n_div = 0
    for chunk in np.array_split(amaxes, 16):
        bits = _blocks_for(chunk, mags)
        # each block is one token of width D: the scale is fl32(amax/127) of its row
        codes_o, scales_o, _ = oracle.quantize(bits, 1)
        x = qsa_gen.bf16_bits_to_f32(bits)[0, 0]
        s_row = (chunk.astype(F32) / F32(127.0)).astype(F32)
        assert np.array_equal(scales_o[0, 0].view(np.uint32), s_row.view(np.uint32))
        got, div = _codes_fast_path(x, np.broadcast_to(s_row[:, None], x.shape))
        assert np.array_equal(got, codes_o[0, 0]), "division-free codes differ from the oracle"
        total += x.size
        n_div += int(div[s_row >= F32(2.0 ** -100)].sum())
    assert total > 1_000_000
    # the division is the rare path wherever the fast path is enabled
    assert n_div < 1e-2 * total


def test_fast_path_band_catches_planted_half_integer_quotients():
    # Quotients exactly at k + 1/2 (power-of-two scales make them exact) must
    # go to the division and round to even; the multiply-by-inverse alone
    # would be right here too, so also check that the band flags them.
    s = F32(2.0 ** -3)
    ks = np.arange(127, dtype=np.float64)
    x = ((ks + 0.5) * float(s)).astype(F32)
    got, div = _codes_fast_path(x, np.full_like(x, s))
    assert np.all(div)
    assert np.array_equal(got.astype(np.int64), np.round(ks + 0.5).astype(np.int64))  # half to even
