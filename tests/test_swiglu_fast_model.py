"""CPU model of the output-side SwiGLU pass's fast evaluation of h = silu(g) * u.

The kernel computes, on the transcendental unit,
    a = exp2(g C_HI), e = a + a (g C_LO ln 2), d = (1 + e) 2^-64,
    h = ((g * rcp(d)) 2^-64) * u
and keeps that h only where its low 16 bits lie more than a fixed margin of
fp32 steps from the bf16 rounding midpoint; everywhere else it evaluates the
definition g / (1 + exp(-g)) * u with the fixed fp32 exponential (the SwiGLU
of the FFN, h3-rs README, "Speed"; placed on fc1's output side as in the
hybrid model card's "FFN output + SwiGLU" projection).

This test models the fast evaluation in numpy over every finite bf16 gate,
with exp2 and rcp pushed 2 ulps off their exact values in either direction,
and checks that h never lands more than half that margin from the value the
definition gives (the oracle's exponential and one IEEE division).  The
constants and the margin are read from the kernel header, so a change there
is checked here.  The GPU parity tests then confirm bit-exact codes on the
real transcendental unit.
"""

import math
import re
from pathlib import Path

import numpy as np
import pytest

import oracle

HEADER = Path(__file__).resolve().parents[1] / "rotation_quantized_dit_amd" / "csrc" / "fixed_math.h"
f32 = np.float32


def _exact_range():
    """The gate range [lo, hi) that swiglu_fast_exact accepts, from the header."""
    m = re.search(r"return g >= ([0-9.]+)f && g < (0x1p\d+)f;", HEADER.read_text())
    return f32(float(m.group(1))), float.fromhex(m.group(2))


def _header_constants():
    text = HEADER.read_text()
    c_hi = re.search(r"SWIGLU_C_HI\s*=\s*([-+0-9a-fA-Fx.p]+)f;", text).group(1)
    c_lo = re.search(r"SWIGLU_C_LO_LN2\s*=\s*([-+0-9a-fA-Fx.p]+)f;", text).group(1)
    margin = re.search(r"SWIGLU_FAST_MARGIN\s*=\s*(\d+);", text).group(1)
    return f32(float.fromhex(c_hi)), f32(float.fromhex(c_lo)), int(margin)


def _ulp(x):
    x = np.abs(np.asarray(x, dtype=np.float32))
    return (np.nextafter(x, np.float32(np.inf)) - x).astype(np.float64)


def _all_finite_bf16():
    g = (np.arange(0, 1 << 16, dtype=np.uint32) << 16).view(np.float32)
    return g[np.isfinite(g)]


def _definition_quotient(g):
    """g / (1 + exp(-g)) in fp32: the oracle's exponential, one IEEE division."""
    d = np.empty(g.size, dtype=np.float32)
    for i, x in enumerate(g.tolist()):
        d[i] = np.inf if -x > 88.72 else f32(1) + f32(oracle.exp(-x))
    with np.errstate(all="ignore"):
        return (g.astype(np.float64) / d.astype(np.float64)).astype(np.float32)


def _fast_quotient(g, c_hi, c_lo, off_exp, off_rcp):
    """The kernel's scaled quotient with exp2 and rcp off by the given ulps."""
    s = f32(2.0 ** -64)
    with np.errstate(all="ignore"):
        t = (g * c_hi).astype(np.float32)
        a64 = np.exp2(t.astype(np.float64))
        a = (a64 + np.where(np.isfinite(a64),
                            off_exp * _ulp(np.minimum(a64, 3e38)), 0)).astype(np.float32)
        b = (g * c_lo).astype(np.float32)
        e = (a.astype(np.float64) * b.astype(np.float64) + a.astype(np.float64)).astype(np.float32)
        d = ((e.astype(np.float64) + 1.0) * 2.0 ** -64).astype(np.float32)
        r64 = 1.0 / d.astype(np.float64)
        y = (r64 + np.where((r64 > 0) & np.isfinite(r64), off_rcp * _ulp(r64), 0)).astype(np.float32)
        # the 2^-64 scale keeps the reciprocal normal for every finite d
        assert np.all((y == 0) | (np.abs(y) >= 2.0 ** -126))
        return ((g * y).astype(np.float32) * s).astype(np.float32)


def test_header_constants_split_log2e():
    c_hi, c_lo, margin = _header_constants()
    # C_HI carries at most 15 significant bits, so g * C_HI is exact for bf16 g (8 bits)
    mant = int(abs(float(c_hi)) * 2 ** 14)
    assert mant == abs(float(c_hi)) * 2 ** 14 and mant < 2 ** 15
    # exp(-g) = 2^(g C_HI) 2^(g C_LO) with C_HI + C_LO = -log2(e); the header stores C_LO ln 2,
    # so C_HI + C_LO_LN2 / ln 2 must equal -log2(e) to the precision of the fp32 low part
    assert abs(float(c_hi) + float(c_lo) / math.log(2) + 1 / math.log(2)) < 1e-12
    assert margin >= 16


@pytest.mark.parametrize("off", [(2.0, -2.0), (-2.0, 2.0), "random"])
def test_fast_quotient_within_half_margin(off):
    c_hi, c_lo, margin = _header_constants()
    g = _all_finite_bf16()
    q_def = _definition_quotient(g)
    rng = np.random.default_rng(11)
    if off == "random":
        off_e = rng.uniform(-2, 2, g.size)
        off_r = rng.uniform(-2, 2, g.size)
    else:
        off_e = np.full(g.size, off[0])
        off_r = np.full(g.size, off[1])
    q = _fast_quotient(g, c_hi, c_lo, off_e, off_r)
    worst = 0
    for scale in (1e-3, 0.7, 3.0, 50.0):
        u = (rng.standard_normal(g.size) * scale).astype(np.float32)
        u = (u.view(np.uint32) & 0xFFFF0000).view(np.float32)
        with np.errstate(all="ignore"):
            h = (q * u).astype(np.float32)
            h_def = (q_def * u).astype(np.float32)
        # where the fast value is kept at all: finite and below 2^127
        kept = np.isfinite(h) & (np.abs(h) < 2.0 ** 127)
        zero = h_def == 0
        assert np.all(h[kept & zero] == 0)
        assert np.all(np.signbit(h[kept & zero]) == np.signbit(h_def[kept & zero]))
        nz = kept & ~zero
        assert np.all(np.signbit(h[nz]) == np.signbit(h_def[nz]))
        steps = np.abs(h.view(np.int32).astype(np.int64) - h_def.view(np.int32).astype(np.int64))[nz]
        worst = max(worst, int(steps.max()))
        # gates that overflow exp2 (bf16 g <= -89) give -0 * u on both sides
        deep = (g <= -89.0) & np.isfinite(h)
        assert np.all(h[deep] == 0) and np.all(h_def[deep] == 0)
    assert worst <= margin // 2, worst


def test_margin_decides_bf16_rounding():
    """Where h is more than the margin from a bf16 midpoint, any value within
    half the margin rounds to the same bf16 (round to nearest even)."""
    _, _, margin = _header_constants()
    rng = np.random.default_rng(5)
    bits = rng.integers(0x00800000, 0x7F000000, 20000, dtype=np.uint32)
    low = bits & 0xFFFF
    far = ((low - (0x8000 - margin)) & 0xFFFFFFFF) > 2 * margin
    bits = bits[far]

    def to_bf16(b):
        # round to nearest even on the fp32 bit pattern
        lsb = (b >> 16) & 1
        return ((b.astype(np.uint64) + 0x7FFF + lsb) >> 16).astype(np.uint32)

    base = to_bf16(bits)
    for delta in (-(margin // 2), -1, 1, margin // 2):
        moved = (bits.astype(np.int64) + delta).astype(np.uint32)
        assert np.array_equal(to_bf16(moved), base)


@pytest.mark.parametrize("off_exp", [-2.0, 0.0, 2.0])
def test_exact_quotient_range(off_exp):
    """On every bf16 gate that swiglu_fast_exact accepts, the definition's
    1 + exp(-g) rounds to 1 (so its quotient is g) and the fast d is exactly
    2^-64 with exp2 pushed 2 ulps either way (so the fast quotient is
    g 2^64 2^-64 = g); the bf16 gate just below the range has 1 + exp(-g) > 1."""
    c_hi, c_lo, _ = _header_constants()
    lo, hi = _exact_range()
    g = _all_finite_bf16()
    sel = (g >= lo) & (g < hi)
    assert sel.sum() > 1000
    with np.errstate(all="ignore"):
        t = (g * c_hi).astype(np.float32)
        a64 = np.exp2(t.astype(np.float64))
        a = (a64 + np.where(np.isfinite(a64), off_exp * _ulp(np.minimum(a64, 3e38)), 0)).astype(np.float32)
        e = (a.astype(np.float64) * (g * c_lo).astype(np.float64) + a.astype(np.float64)).astype(np.float32)
        d = ((e.astype(np.float64) + 1.0) * 2.0 ** -64).astype(np.float32)
    assert np.all(d[sel] == f32(2.0 ** -64))
    # the largest accepted gate times 2^64 stays finite
    assert np.isfinite(f32(g[sel].max()) * f32(2.0 ** 64))
    one = np.array([f32(1) + f32(oracle.exp(-float(x))) for x in g[sel].tolist()], dtype=np.float32)
    assert np.all(one == 1)
    below = np.nextafter(lo, f32(0))                      # fp32 neighbour, then its bf16 floor
    below = f32((np.array([below], dtype=np.float32).view(np.uint32) & 0xFFFF0000).view(np.float32)[0])
    assert below < lo and f32(1) + f32(oracle.exp(-float(below))) > 1
