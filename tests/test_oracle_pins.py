"""Pins of the CPU oracle against what the definitions fix (CPU only).

Every check compares the oracle with something other than itself: the closed
form of the Sylvester Hadamard matrix, exact integer arithmetic, fp64 dense
linear algebra with a stated rounding bound, numpy's int64 matmul, torch's
bf16 cast, Python's correctly rounded fp64 exp, or a value fixed by the
mathematics of a constructed input.  A plausible slip in the oracle (a wrong
stage order or sign, a dropped 1/16, a transposed operand, round-half-up
instead of half-even, a swapped gate/up half, scales applied to the wrong
axis) fails at least one of them.
"""
import math

import numpy as np
import pytest

import oracle
from tests import hadamard as hd
import workloads

U = 2.0 ** -24
GAMMA8 = 8 * U / (1 - 8 * U)


# ------------------------------------------------------------------ Hadamard

def test_sylvester_definition():
    """H.H = 256 I and H = H^T for the closed-form Sylvester matrix (C1)."""
    H = hd.H()
    assert np.array_equal(H, H.T)
    assert np.array_equal(H @ H, 256 * np.eye(256, dtype=np.int64))
    # Sylvester recursion H_2n = [[H, H], [H, -H]] holds on every level
    for n in (2, 4, 8, 16, 32, 64, 128):
        a = hd.sylvester(n)
        b = hd.sylvester(2 * n)
        assert np.array_equal(b, np.block([[a, a], [a, -a]]))


def test_fwht_basis_columns():
    """fwht(e_j) is column j of H/16, exactly, for every j (C2)."""
    H = hd.H()
    for j in range(256):
        e = np.zeros(256, np.float32)
        e[j] = 1.0
        got = oracle.fwht256(e)
        assert np.array_equal(got.astype(np.float64), H[:, j] / 16.0), j


def test_fwht_exact_integer_regime():
    """For integers |x| <= 2^15 every partial sum is an integer below 2^24, so the
    fp32 butterfly must equal the dense integer product H.x / 16 bit for bit (C3)."""
    rng = np.random.default_rng(11)
    H = hd.H()
    for _ in range(200):
        x = rng.integers(-2 ** 15, 2 ** 15 + 1, 256)
        got = oracle.fwht256(x.astype(np.float32)).astype(np.float64)
        want = (H @ x).astype(np.float64) / 16.0
        assert np.array_equal(got, want)


@pytest.mark.parametrize("kind", ["normal", "outliers", "laplace", "wide"])
def test_fwht_rounding_bound(kind):
    """Depth-8 pairwise summation bound: |fwht(x)_i - (H x / 16)_i| <=
    gamma_8 * sum_j |x_j| / 16, with the reference in fp64 (C4)."""
    rng = np.random.default_rng(12)
    H = hd.H().astype(np.float64)
    for _ in range(100):
        if kind == "normal":
            x = rng.standard_normal(256).astype(np.float32)
        elif kind == "outliers":
            x = rng.standard_normal(256).astype(np.float32)
            x[rng.choice(256, 3, replace=False)] *= 50
        elif kind == "laplace":
            x = rng.laplace(size=256).astype(np.float32)
        else:
            x = (rng.standard_normal(256) * np.exp2(rng.integers(-20, 20, 256))).astype(np.float32)
        got = oracle.fwht256(x).astype(np.float64)
        want = H @ x.astype(np.float64) / 16.0
        bound = GAMMA8 * np.abs(x.astype(np.float64)).sum() / 16.0
        assert np.all(np.abs(got - want) <= bound)


def test_norm_preservation_and_involution():
    """H/16 is orthogonal and involutive: ||fwht(x)|| = ||x|| and
    fwht(fwht(x)) = x, up to the fp32 rounding of 8 stages (C5)."""
    rng = np.random.default_rng(13)
    for _ in range(100):
        x = rng.standard_normal(256).astype(np.float32)
        y = oracle.fwht256(x)
        nx = np.linalg.norm(x.astype(np.float64))
        assert abs(np.linalg.norm(y.astype(np.float64)) - nx) <= 16 * GAMMA8 * nx
        z = oracle.fwht256(y).astype(np.float64)
        bound = 2 * GAMMA8 * np.abs(x.astype(np.float64)).sum() / 16.0 * 16
        assert np.max(np.abs(z - x)) <= bound
    # the exact regime: a second pass returns integer inputs exactly
    x = np.random.default_rng(14).integers(-2000, 2000, 256).astype(np.float32)
    assert np.array_equal(oracle.fwht256(oracle.fwht256(x)), x)


def test_rotation_is_groupwise_and_contiguous():
    """Each contiguous 256-block of a row is rotated on its own: perturbing one
    block changes only that block's outputs (reading: groups of the conv with
    kernel = stride = 256)."""
    rng = np.random.default_rng(15)
    x = rng.standard_normal((3, 1024)).astype(np.float32)
    r = oracle.rotate_rows(x)
    x2 = x.copy()
    x2[1, 300] += 1.0
    r2 = oracle.rotate_rows(x2)
    diff = np.nonzero(np.any(r != r2, axis=0))[0]
    assert diff.min() >= 256 and diff.max() < 512
    assert np.array_equal(r[0], r2[0]) and np.array_equal(r[2], r2[2])
    # and matches the dense fp64 block-diagonal rotation within the bound
    want = hd.rotate_fp64(x)
    for g in range(4):
        bound = GAMMA8 * np.abs(x[:, g * 256:(g + 1) * 256].astype(np.float64)).sum(1) / 16
        assert np.all(np.abs(r[:, g * 256:(g + 1) * 256] - want[:, g * 256:(g + 1) * 256])
                      <= bound[:, None])


def test_rotation_invariance_of_the_product():
    """(x H)(W H)^T = x W^T: the oracle's fp32 rotation of both operands keeps the
    fp64 product within the propagated butterfly bound, on all of the tiny workload (C6)."""
    d = workloads.make_linear("tiny")
    x = hd.bf16_bits_to_f64(d["x"])
    w = d["w"].astype(np.float64)
    xr = oracle.rotate_rows(x.astype(np.float32)).astype(np.float64)
    wr = oracle.rotate_rows(d["w"]).astype(np.float64)
    exact = x @ w.T
    got = xr @ wr.T

    def err(a):
        e = np.empty_like(a)
        for g in range(0, a.shape[1], 256):
            e[:, g:g + 256] = GAMMA8 * np.abs(a[:, g:g + 256]).sum(1, keepdims=True) / 16
        return e
    ex, ew = err(x), err(w)
    bound = ex @ np.abs(wr).T + np.abs(xr) @ ew.T + ex @ ew.T
    bound = bound * (1 + 1e-6) + 1e-12 * (np.abs(x) @ np.abs(w).T)
    assert np.all(np.abs(got - exact) <= bound)


# ------------------------------------------------------------------ quantizer

def _check_quant_invariants(v, q, s):
    v64 = v.astype(np.float64)
    assert q.dtype == np.int8
    assert q.min() >= -127 and q.max() <= 127
    for r in range(v.shape[0]):
        amax = np.abs(v64[r]).max()
        if amax == 0:
            assert s[r] == 0 and not q[r].any()
            continue
        # s is amax / 127 correctly rounded (within half an ulp of the exact quotient)
        assert abs(float(s[r]) - amax / 127) <= 0.5 * float(np.spacing(np.float32(s[r])))
        am = np.argmax(np.abs(v64[r]))
        assert abs(int(q[r, am])) == 127 and np.sign(q[r, am]) == np.sign(v64[r, am])
        # round-trip bound |v - q s| <= s/2 + |v| 2^-24 (division rounding), fp64 slack
        s64 = float(s[r])
        lhs = np.abs(v64[r] - q[r].astype(np.float64) * s64)
        assert np.all(lhs <= s64 / 2 + np.abs(v64[r]) * 2.0 ** -24 + 1e-12 * s64)


def test_quantizer_invariants():
    """Codes in [-127, 127], |q| = 127 at the row's argmax, the round-trip
    bound, and an all-zero row giving s = 0 and zero codes (C7, S9)."""
    rng = np.random.default_rng(16)
    v = rng.standard_normal((40, 512)).astype(np.float32)
    v[3] = 0.0
    v[5] *= 1e-30
    v[7, 17] = 1e6
    v[9] = np.float32(2.0) ** rng.integers(-60, 60, 512)
    q, s = oracle.quantize_rows(v)
    _check_quant_invariants(v, q, s)
    d = workloads.make_linear("tiny")
    qx, sx = oracle.rotate_quant_act(d["x"])
    xr = oracle.rotate_rows(oracle.bf16_to_f32(d["x"]))
    _check_quant_invariants(xr, qx, sx)
    qw, sw = oracle.quantize_weight(d["w"])
    _check_quant_invariants(oracle.rotate_rows(d["w"]), qw, sw)


def _tie_row(k, scale, rng, values):
    """A bf16-exact activation row whose rotation is sparse: group g holds
    v_g * (column j_g of H/16), so the rotated row is v_g at position j_g.
    Returns x (fp64), the rotated row (exact), and the expected codes."""
    H = hd.H().astype(np.float64)
    x = np.zeros(k)
    rot = np.zeros(k)
    for g, val in enumerate(values):
        j = int(rng.integers(0, 256))
        x[g * 256:(g + 1) * 256] = val * scale * H[:, j] / 16.0
        rot[g * 256 + j] = val * scale
    return x, rot


def test_tie_breaking_half_even_activation_path():
    """Rotated values that are exact half-integers of the scale must round half
    to even: 2.5 -> 2, 3.5 -> 4, -2.5 -> -2, -0.5 -> 0, 126.5 -> 126 (C8, S8).
    The amax entry is 127 * 2^e so s = 2^e exactly; all inputs are bf16-exact."""
    rng = np.random.default_rng(17)
    values = [127.0, 2.5, 3.5, -2.5, -0.5, 0.5, 1.5, -1.5, 126.5, -126.5, 4.5, -3.5, 0.0, 5.5, 6.5, -7.5]
    k = 256 * len(values)
    rows, expect, scales = [], [], []
    for e in (0, -3, 5, -10):
        x, rot = _tie_row(k, 2.0 ** e, rng, values)
        assert hd.is_bf16_exact(x)
        rows.append(x)
        expect.append(np.rint(rot / 2.0 ** e))  # numpy rint: exact halves to even
        scales.append(2.0 ** e)
    xb = workloads.to_bf16_bits(np.array(rows, np.float32))
    q, s = oracle.rotate_quant_act(xb)
    assert np.array_equal(s.astype(np.float64), np.array(scales))
    assert np.array_equal(q.astype(np.float64), np.array(expect))
    want = {2.5: 2, 3.5: 4, -2.5: -2, -0.5: 0, 126.5: 126, 0.5: 0, 1.5: 2, -1.5: -2, 4.5: 4}
    for v, c in want.items():
        assert int(np.rint(v)) == c


def test_tie_breaking_weight_path_dense():
    """Weight path (fp32 input): W = H v / 16 with dense half-integer v and
    amax 127 is exact in fp32, its rotation returns v exactly, and the codes are
    v rounded half to even (C8)."""
    rng = np.random.default_rng(18)
    H = hd.H()
    v = rng.integers(-254, 255, (6, 512)).astype(np.float64) / 2.0  # halves in [-127, 127]
    v[:, 5] = 127.0
    w = np.zeros_like(v)
    for g in range(2):
        w[:, g * 256:(g + 1) * 256] = v[:, g * 256:(g + 1) * 256] @ H / 16.0
    assert np.array_equal(w.astype(np.float32).astype(np.float64), w)
    q, s = oracle.quantize_weight(w.astype(np.float32))
    assert np.all(s == 1.0)
    assert np.array_equal(q.astype(np.float64), np.rint(v))
    assert np.any(np.abs(v - np.trunc(v)) == 0.5)


def test_dense_bruteforce_tiny():
    """Rotate and quantize in fp64 from the dense matrix; the oracle's codes must
    equal it except where v/s sits within 1e-5 of a half-integer, and the
    oracle's scales agree to fp32 rounding (C11)."""
    rng = np.random.default_rng(19)
    for trial in range(6):
        m, k = 16, 256 * (1 + trial % 3)
        x = rng.standard_normal((m, k)).astype(np.float32)
        x[:, rng.choice(k, 2, replace=False)] *= 40
        xb = workloads.to_bf16_bits(x)
        q, s = oracle.rotate_quant_act(xb)
        v = hd.rotate_fp64(hd.bf16_bits_to_f64(xb))
        s64 = np.abs(v).max(1) / 127
        assert np.all(np.abs(s - s64) <= 2 * U * s64)
        t = v / s64[:, None]
        q64 = np.clip(np.rint(t), -127, 127)
        mism = q.astype(np.float64) != q64
        near = np.abs(np.abs(t - np.trunc(t)) - 0.5) < 1e-5
        assert np.all(near[mism]), (trial, np.argwhere(mism & ~near)[:5])


# ------------------------------------------------------------------ contraction

def test_gemm_s32_matches_int64_matmul():
    """The int32 triple loop equals numpy's int64 matmul on random codes (C9)."""
    rng = np.random.default_rng(20)
    for (m, n, k) in [(1, 1, 256), (7, 13, 512), (33, 17, 1024), (64, 256, 512)]:
        a = rng.integers(-127, 128, (m, k)).astype(np.int8)
        b = rng.integers(-127, 128, (n, k)).astype(np.int8)
        want = a.astype(np.int64) @ b.astype(np.int64).T
        got = oracle.gemm_s32(a, b)
        assert got.dtype == np.int32 and np.array_equal(got.astype(np.int64), want)
    # not symmetric in its operands: a transposed operand would fail here
    a = rng.integers(-127, 128, (3, 256)).astype(np.int8)
    b = rng.integers(-127, 128, (5, 256)).astype(np.int8)
    assert oracle.gemm_s32(a, b).shape == (3, 5)


def test_gemm_closed_form_extremes():
    """All codes +127 at K = 14336 give 127^2 * 14336 = 231,225,344 exactly, and
    mixed signs give the negative (C9); 127^2 * 133120 still fits int32."""
    k = 14336
    a = np.full((2, k), 127, np.int8)
    b = np.full((3, k), 127, np.int8)
    b[1] = -127
    got = oracle.gemm_s32(a, b)
    assert got[0, 0] == 231225344 and got[1, 1] == -231225344
    assert 127 * 127 * 133120 < 2 ** 31 <= 127 * 127 * 133376


def test_closed_form_single_code():
    """x = c * (column j of H/16) in one group, W = d * (column j of H/16): both
    quantize to a single code of +-127 at j, acc = +-16129, and the output is the
    exact product c * d up to the fp32 scales and bf16 rounding (C10)."""
    H = hd.H().astype(np.float64)
    for (c, d, j, g) in [(3.0, 0.5, 7, 0), (-2.0, 0.25, 200, 1), (48.0, -0.0625, 0, 1), (1.5, 1.5, 255, 0)]:
        x = np.zeros((1, 512))
        w = np.zeros((1, 512))
        x[0, g * 256:(g + 1) * 256] = c * H[:, j] / 16
        w[0, g * 256:(g + 1) * 256] = d * H[:, j] / 16
        assert hd.is_bf16_exact(x)
        xb = workloads.to_bf16_bits(x.astype(np.float32))
        qx, sx = oracle.rotate_quant_act(xb)
        qw, sw = oracle.quantize_weight(w.astype(np.float32))
        assert np.count_nonzero(qx) == 1 and qx[0, g * 256 + j] == 127 * np.sign(c)
        assert np.count_nonzero(qw) == 1 and qw[0, g * 256 + j] == 127 * np.sign(d)
        acc = oracle.gemm_s32(qx, qw)
        assert acc[0, 0] == 16129 * np.sign(c * d)
        y = hd.bf16_bits_to_f64(oracle.dequant_bf16(acc, sx, sw))[0, 0]
        assert abs(y - c * d) <= abs(c * d) * (2.0 ** -8 + 4 * U)


# ------------------------------------------------------------------ epilogues

def test_dequant_against_fp64():
    """fp32 dequant (acc * s_x) * s_w is within 3 roundings of the exact
    product, and its bf16 is within one bf16 ulp; scales apply per row (s_x)
    and per column (s_w), not the other way round (O8)."""
    rng = np.random.default_rng(21)
    acc = rng.integers(-2 ** 28, 2 ** 28, (9, 11)).astype(np.int32)
    sx = rng.uniform(0.001, 2, 9).astype(np.float32)
    sw = rng.uniform(0.0001, 0.01, 11).astype(np.float32)
    f = oracle.dequant_f32(acc, sx, sw).astype(np.float64)
    exact = acc.astype(np.float64) * sx.astype(np.float64)[:, None] * sw.astype(np.float64)[None, :]
    assert np.all(np.abs(f - exact) <= 3.01 * U * np.abs(exact))
    y = hd.bf16_bits_to_f64(oracle.dequant_bf16(acc, sx, sw))
    assert np.all(np.abs(y - exact) <= np.abs(exact) * (2.0 ** -8 + 4 * U))


def test_exp_against_exact():
    """The fixed fp32 exponential is within 1 ulp of the exact e^x over
    [-86, 88.7], exact at 0, +inf above the fp32 range, 0 below -86."""
    xs = np.concatenate([np.linspace(-86, 88.7, 40001), np.linspace(-1, 1, 4001)]).astype(np.float32)
    worst = 0.0
    for x in xs:
        e = oracle.exp(float(x))
        t = math.exp(float(x))
        worst = max(worst, abs(e - t) / float(np.spacing(np.float32(t))))
    assert worst <= 1.0, worst
    assert oracle.exp(0.0) == 1.0
    assert oracle.exp(89.0) == math.inf and oracle.exp(-90.0) == 0.0


def test_silu_special_values_and_accuracy():
    """silu(0) = 0, silu(g) -> -0 for very negative g, silu(g) = g for large g,
    and elsewhere within 3 * 2^-23 relative of the exact g * sigmoid(g) (exp
    within 1 ulp, then three RNE roundings: the add, the division, and none
    else)."""
    assert oracle.silu(0.0) == 0.0
    v = oracle.silu(-100.0)
    assert v == 0.0 and math.copysign(1.0, v) < 0
    assert oracle.silu(100.0) == 100.0
    for g in np.linspace(-60, 60, 6001).astype(np.float32):
        g = float(g)
        t = g / (1 + math.exp(-g))
        if t == 0:
            continue
        assert abs(oracle.silu(g) - t) <= 3 * 2.0 ** -23 * abs(t), g


def test_bf16_rounding_matches_torch():
    """The oracle's fp32 -> bf16 rounding equals torch's cast (round half to
    even) on random values, exact ties, overflow and signed zeros (O10)."""
    rng = np.random.default_rng(22)
    f = (rng.standard_normal(20000) * np.exp2(rng.integers(-100, 100, 20000))).astype(np.float32)
    ties = np.array([0x3F808000, 0x3F818000, 0xBF808000, 0x3F80FFFF, 0x7F7FFFFF, 0x00000000,
                     0x80000000, 0x00018000, 0x7F800000], np.uint32).view(np.float32)
    f = np.concatenate([f, ties])
    assert np.array_equal(oracle.f32_to_bf16(f), workloads.to_bf16_bits(f))
    b = oracle.f32_to_bf16(np.array([np.nan], np.float32))[0]
    assert (b & 0x7F80) == 0x7F80 and (b & 0x7F) != 0


def test_swiglu_epilogue_layout_and_value():
    """SwiGLU takes the gate from the first half of the columns and the up
    projection from the second; y = bf16(silu(g) * u) within one bf16 ulp of
    the exact value (O9, S13)."""
    rng = np.random.default_rng(23)
    i = 24
    acc = rng.integers(-3_000_000, 3_000_000, (5, 2 * i)).astype(np.int32)
    sx = rng.uniform(0.01, 0.1, 5).astype(np.float32)
    sw = rng.uniform(1e-5, 1e-4, 2 * i).astype(np.float32)
    y = hd.bf16_bits_to_f64(oracle.swiglu_bf16(acc, sx, sw))
    g = acc[:, :i] * sx.astype(np.float64)[:, None] * sw[:i].astype(np.float64)
    u = acc[:, i:] * sx.astype(np.float64)[:, None] * sw[i:].astype(np.float64)
    exact = g / (1 + np.exp(-g)) * u
    assert np.all(np.abs(y - exact) <= np.abs(exact) * (2.0 ** -8 + 16 * U) + 1e-30)
    swapped = u / (1 + np.exp(-u)) * g
    assert not np.allclose(y, swapped, rtol=1e-2)


def test_swiglu_ref_layout_and_value():
    """The fp64 reference of the fused epilogue takes g from the first half of
    the columns and u from the second, each the fp32 dequant (a value within
    two fp32 roundings of acc s_x s_w), and returns silu(g) u unrounded: against
    an fp64 evaluation on the exact products it differs by at most the fp32
    dequant's rounding; |g u| comes back as the magnitude."""
    rng = np.random.default_rng(29)
    i = 40
    acc = rng.integers(-3_000_000, 3_000_000, (6, 2 * i)).astype(np.int32)
    sx = rng.uniform(0.01, 0.1, 6).astype(np.float32)
    sw = rng.uniform(1e-5, 1e-4, 2 * i).astype(np.float32)
    ref, mag = oracle.swiglu_ref(acc, sx, sw)
    g = acc[:, :i] * sx.astype(np.float64)[:, None] * sw[:i].astype(np.float64)
    u = acc[:, i:] * sx.astype(np.float64)[:, None] * sw[i:].astype(np.float64)
    exact = g / (1 + np.exp(-g)) * u
    # g and u carry relative errors <= 2U each (two fp32 roundings); a relative
    # error e in g moves silu(g) by |1 + g (1 - sigma(g))| e relatively, so
    # the propagated bound is (|1 + g (1 - sigma(g))| + 1) 2U (+ a margin)
    sig = 1 / (1 + np.exp(-g))
    amp = np.abs(1 + g * (1 - sig)) + 1
    assert np.all(np.abs(ref - exact) <= 2.2 * U * amp * np.abs(exact) + 1e-300)
    assert np.allclose(mag, np.abs(g * u), rtol=8 * U)
    swapped = u / (1 + np.exp(-u)) * g
    assert not np.allclose(ref, swapped, rtol=1e-2)


def test_swiglu_ref_closed_forms():
    """sigma(ln 3) = 3/4 and sigma(-ln 3) = 1/4, so silu(+-ln 3) = +-ln 3 * 3/4,
    -ln 3 / 4; silu(g) - silu(-g) = g for any g; e^-g vanishes for large g
    (silu(g) = g) and overflows for very negative g (silu(g) = -0)."""
    ln3 = np.float32(math.log(3.0))
    acc = np.array([[1, -1, 1, 0, 7, 5, 1, 1, 1, 1, 1, 1]], np.int32)
    sx = np.ones(1, np.float32)
    sw = np.array([ln3, ln3, 100.0, 1.0, -200.0, 3.0, 1.0, 1.0, 2.5, 1.0, 1.0, 1.0], np.float32)   # g | u
    ref, mag = oracle.swiglu_ref(acc, sx, sw)
    g = float(ln3)
    d = g - math.log(3.0)            # fp32 rounding of ln 3, |d| < 2^-24 ln 3
    # sigma(ln 3 + d) = 3/4 + (3/16) d + O(d^2), sigma(-ln 3 - d) = 1/4 - (3/16) d + O(d^2)
    assert abs(ref[0, 0] - g * (0.75 + 3 / 16 * d)) <= 1e-15
    assert abs(ref[0, 1] - (-g) * (0.25 - 3 / 16 * d)) <= 1e-15
    assert abs((ref[0, 0] - ref[0, 1]) - g) <= 1e-15
    assert ref[0, 2] == 100.0 * 2.5                 # silu(100) = 100 to fp64 precision, u = 2.5
    assert ref[0, 3] == 0.0                         # silu(0) = 0
    assert ref[0, 4] == 0.0 and math.copysign(1.0, ref[0, 4]) < 0   # g = -1400: e^1400 overflows
    assert mag[0, 4] == 1400.0 * 1.0
    assert abs(ref[0, 5] - 15.0 / (1 + math.exp(-15.0))) <= 1e-13


def test_swiglu_ref_agrees_with_fixed_fp32_path():
    """Two independent evaluations: the fp64 reference rounded once to bf16
    and the oracle's fixed fp32 exponential path agree within one bf16 ulp on
    every element, and exactly on all but a small fraction."""
    rng = np.random.default_rng(31)
    i = 512
    acc = rng.integers(-4_000_000, 4_000_000, (16, 2 * i)).astype(np.int32)
    sx = rng.uniform(0.005, 0.05, 16).astype(np.float32)
    sw = rng.uniform(1e-5, 2e-4, 2 * i).astype(np.float32)
    ref, _ = oracle.swiglu_ref(acc, sx, sw)
    fixed = hd.bf16_bits_to_f64(oracle.swiglu_bf16(acc, sx, sw))
    ref_b = hd.bf16_bits_to_f64(workloads.to_bf16_bits(ref.astype(np.float32)))
    assert np.all(np.abs(fixed - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-30)
    assert np.mean(fixed != ref_b) < 0.01


# ------------------------------------------------------------------ method level

def _rel_fro(y_bits, exact):
    y = hd.bf16_bits_to_f64(y_bits)
    return np.linalg.norm(y - exact) / np.linalg.norm(exact)


@pytest.mark.parametrize("name,rows", [("tiny", None), ("qkv", 48)])
def test_rotation_beats_unrotated_int8(name, rows):
    """The method's claim (RESEARCH.md, "Weight families"): on inputs with
    outlier channels the rotated int8 product is far closer to x W^T than
    per-token int8 without rotation (same oracle with H replaced by I) (C12)."""
    d = workloads.make_linear(name, m=rows)
    x = hd.bf16_bits_to_f64(d["x"])
    exact = x @ d["w"].astype(np.float64).T
    qw, sw = oracle.quantize_weight(d["w"])
    y_rot = oracle.linear_rows(d["x"], qw, sw)
    qx0, sx0 = oracle.quantize_rows(x.astype(np.float32))
    qw0, sw0 = oracle.quantize_rows(d["w"])
    y_plain = oracle.dequant_bf16(oracle.gemm_s32(qx0, qw0), sx0, sw0)
    e_rot, e_plain = _rel_fro(y_rot, exact), _rel_fro(y_plain, exact)
    assert e_rot < 0.5 * e_plain, (e_rot, e_plain)
    assert e_rot < 0.05


def test_determinism_across_thread_counts():
    """Rows are independent, so results are identical for 1 and many threads (C13)."""
    d = workloads.make_linear("tiny")
    before = oracle.get_threads()
    try:
        oracle.set_threads(1)
        a = oracle.quantize_weight(d["w"]), oracle.linear_rows(d["x"], *oracle.quantize_weight(d["w"]))
        oracle.set_threads(8)
        b = oracle.quantize_weight(d["w"]), oracle.linear_rows(d["x"], *oracle.quantize_weight(d["w"]))
    finally:
        oracle.set_threads(before)
    assert np.array_equal(a[0][0], b[0][0]) and np.array_equal(a[0][1], b[0][1])
    assert np.array_equal(a[1], b[1])


def test_row_subset_equals_full():
    """Processing a subset of rows gives exactly those rows of the full result
    (what the full-size parity tests rely on)."""
    d = workloads.make_linear("tiny")
    qw, sw = oracle.quantize_weight(d["w"])
    full = oracle.linear_rows(d["x"], qw, sw)
    rows = np.array([63, 0, 17, 17, 40])
    sub = oracle.linear_rows(d["x"], qw, sw, rows)
    assert np.array_equal(sub, full[rows])


def test_stage_order_is_ascending():
    """The butterfly's stage order decides rounding (reading: spans 1, 2, ..., 128).
    For x = (1, 2^-24, 2^-24, 0, ...) the ascending order gives, by hand,
    16 * out[i] = (1, 1, 1 - 2^-24, 1 - 2^-23)[i & 3]; the descending order
    would give (1, 1 - 2^-24, 1, 1 - 2^-23) and the exact transform
    (1 + 2^-23, 1, 1, 1 - 2^-23)."""
    x = np.zeros(256, np.float32)
    x[0] = 1.0
    x[1] = x[2] = 2.0 ** -24
    got = oracle.fwht256(x).astype(np.float64) * 16
    pattern = np.array([1.0, 1.0, 1.0 - 2.0 ** -24, 1.0 - 2.0 ** -23])
    assert np.array_equal(got, pattern[np.arange(256) & 3])


def _division_cases():
    # (amax, v) pairs, bf16-exact, where rint(v / s) with a correctly rounded
    # quotient differs from rint(v * RN(1/s)); found by a seeded search and
    # checked below with exact rationals.
    return [(56.25, -28.125), (61.0, 30.5), (44.75, 22.375), (9.8125, -4.90625),
            (3.765625, -1.8828125), (43.75, 21.875), (19.5, 9.75), (19.5, -9.75)]


def _expected_code(amax, v):
    from fractions import Fraction
    s = hd.rn_f32(Fraction(amax) / 127)
    q = hd.rint_half_even(hd.rn_f32(Fraction(v) / Fraction(s)))
    recip = hd.rn_f32(1 / Fraction(s))
    q_recip = hd.rint_half_even(hd.rn_f32(Fraction(v) * Fraction(recip)))
    return s, q, q_recip


@pytest.mark.parametrize("path", ["activation", "weight"])
def test_quotient_is_correctly_rounded(path):
    """Codes use a correctly rounded v / s (reading of the absmax quantizer),
    not v times a rounded reciprocal.  Rows are built so that their rotation is
    exactly (amax at one position, v at another); the expected code comes from
    exact rational arithmetic.  Each case is one where the two differ."""
    H = hd.H().astype(np.float64)
    cases = _division_cases()
    rows, want_s, want_q = [], [], []
    for (amax, v) in cases:
        s, q, q_recip = _expected_code(amax, v)
        assert q != q_recip
        row = np.zeros(512)
        row[0:256] = amax * H[:, 3] / 16
        row[256:512] = v * H[:, 77] / 16
        rows.append(row)
        want_s.append(s)
        want_q.append(q)
    rows = np.array(rows)
    if path == "activation":
        assert hd.is_bf16_exact(rows)
        q, s = oracle.rotate_quant_act(workloads.to_bf16_bits(rows.astype(np.float32)))
    else:
        q, s = oracle.quantize_weight(rows.astype(np.float32))
    assert np.array_equal(s.astype(np.float64), np.array(want_s))
    assert np.array_equal(q[:, 3].astype(np.int64), np.full(len(cases), 127))
    assert np.array_equal(q[:, 256 + 77].astype(np.int64), np.array(want_q))
    assert np.count_nonzero(q) == 2 * len(cases)


def _golden(tag):
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "closed_forms.txt")
    out = []
    for line in open(path):
        parts = line.split()
        if parts and parts[0] == tag:
            out.append(parts[1:])
    assert out, tag
    return out


def test_golden_closed_forms():
    """The stored closed-form table (tests/golden/closed_forms.txt) holds for
    the oracle: half-even ties, int32 extremes and the stage-order pattern."""
    rng = np.random.default_rng(24)
    for v, code in _golden("ties"):
        x, rot = _tie_row(512, 1.0, rng, [127.0, float(v)])
        q, s = oracle.rotate_quant_act(workloads.to_bf16_bits(x[None].astype(np.float32)))
        assert s[0] == 1.0
        assert int(q[0, 256 + np.nonzero(rot[256:])[0][0]]) == int(code)
    for k, a, b, want in _golden("gemm"):
        k = int(k)
        qa = np.full((1, k), int(a), np.int8)
        qb = np.full((1, k), int(b), np.int8)
        assert oracle.gemm_s32(qa, qb)[0, 0] == int(want)
    x = np.zeros(256, np.float32)
    x[0] = 1.0
    x[1] = x[2] = 2.0 ** -24
    got = oracle.fwht256(x).astype(np.float64) * 16
    for i, val in _golden("stage"):
        assert np.all(got[np.arange(256) % 4 == int(i)] == float(val))


def test_tiny_digest_unchanged():
    """The oracle's tiny-workload results match the committed digests (a lock
    against unintended changes of its arithmetic or of the input generator)."""
    from tests.golden.make_tiny_digest import digests
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "tiny_oracle_digest.txt")
    want = dict(l.split() for l in open(path) if l.strip() and not l.startswith("#"))
    assert digests() == want


# ------------------------------------------------- SwiGLU on fc1's output side

def _bf16_from_f64(v):
    """Round float64 values once to bf16 (torch's fp64 -> bf16 cast is a single
    round-to-nearest-even from the exact fp64 value), as raw bits."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float64)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def test_swiglu_pairs_against_fp64():
    """h = bf16(silu(g) * u) on fc1's bf16 output: equal to an fp64 evaluation
    rounded once to bf16, except where the fp64 value lies within the fp32
    chain's error (exp <= 1 ulp, then one add, one division and one multiply,
    each RN) of a bf16 half-way point, where the neighbour is allowed.  Gate
    columns [0, i), up columns [i, 2i): a swapped half fails by far."""
    rng = np.random.default_rng(31)
    m, i = 24, 512
    g = rng.standard_normal((m, i)) * np.array([0.5, 4.0, 30.0])[rng.integers(0, 3, (m, i))]
    u = rng.standard_normal((m, i)) * 3.0
    gu = workloads.to_bf16_bits(np.concatenate([g, u], axis=1).astype(np.float32))
    h = oracle.swiglu_pairs_bf16(gu)
    gf = oracle.bf16_to_f32(gu[:, :i]).astype(np.float64)
    uf = oracle.bf16_to_f32(gu[:, i:]).astype(np.float64)
    with np.errstate(over="ignore"):
        sil64 = gf / (1.0 + np.exp(-gf))
    h64 = sil64 * uf
    ref = _bf16_from_f64(h64)
    hv = oracle.bf16_to_f32(h).astype(np.float64)
    # fp32 exp(-g) overflows above 88.72, so the definition's fp32 quotient is
    # exactly +-0 there (fp64 still has a denormal-range value)
    over = -gf > 88.72
    assert over.any() and np.all(hv[over] == 0) and np.all(np.abs(h64[over]) < 2.0 ** -100)
    # where the quotient itself is near or inside the fp32 denormal range it
    # carries fewer bits: its absolute error is at most a few denormal steps
    # (2^-149), scaled by |u|, plus the final bf16 rounding of the product
    tiny = ~over & (np.abs(sil64) < 2.0 ** -120)
    assert tiny.any()
    bound = np.abs(uf) * 2.0 ** -147 + 2.0 ** -8 * np.abs(h64) + 2.0 ** -133
    assert np.all(np.abs(hv[tiny] - h64[tiny]) <= bound[tiny])
    diff = (h != ref) & ~over & ~tiny
    assert diff.mean() < 1e-3, diff.mean()
    # every other mismatch is a near-tie: h64 within 8 fp32 ulps of the bf16 midpoint between the two
    for r, c in zip(*np.nonzero(diff)):
        a = float(oracle.bf16_to_f32(np.array([h[r, c]], np.uint16))[0])
        b = float(oracle.bf16_to_f32(np.array([ref[r, c]], np.uint16))[0])
        assert abs(np.int32(h[r, c]) - np.int32(ref[r, c])) == 1       # adjacent bf16 values
        mid = 0.5 * (a + b)
        assert abs(h64[r, c] - mid) <= 8 * U * abs(mid), (h64[r, c], a, b)
    # the halves matter: silu(u) * g differs almost everywhere
    with np.errstate(over="ignore"):
        swapped = _bf16_from_f64(uf / (1.0 + np.exp(-uf)) * gf)
    assert (swapped != h).mean() > 0.9


def test_swiglu_pairs_special_values():
    """silu(0) u = 0; u = 0 gives 0; g -> -inf gives -0 (1 + e^200 overflows);
    large g gives silu(g) = g exactly (e^-g is 0 below -86), so h = bf16(g u)."""
    g = np.array([0.0, 1.5, -200.0, 200.0, 120.0, -3.0], np.float32)
    u = np.array([5.0, 0.0, 2.0, 2.0, -0.5, 0.0], np.float32)
    gu = workloads.to_bf16_bits(np.concatenate([g, u])[None, :])
    h = oracle.bf16_to_f32(oracle.swiglu_pairs_bf16(gu))[0]
    assert h[0] == 0 and h[1] == 0 and h[5] == 0
    assert h[2] == 0 and np.signbit(h[2])          # (-200 / inf) * 2 = -0
    assert h[3] == 400.0 and h[4] == -60.0


def test_swiglu_rotate_quant_composes():
    """The fused preparation equals rotating and quantizing the bf16 SwiGLU
    output row by row (selected rows included), and a row whose up half is
    zero has scale 0 and all-zero codes."""
    rng = np.random.default_rng(32)
    m, i = 9, 768
    gu = workloads.to_bf16_bits(rng.laplace(size=(m, 2 * i)).astype(np.float32))
    gu[3, i:] = 0
    q, s = oracle.swiglu_rotate_quant_act(gu)
    q2, s2 = oracle.rotate_quant_act(oracle.swiglu_pairs_bf16(gu))
    assert np.array_equal(q, q2) and np.array_equal(s.view(np.uint32), s2.view(np.uint32))
    assert s[3] == 0 and not q[3].any()
    rows = np.array([8, 3, 0])
    qr, sr = oracle.swiglu_rotate_quant_act(gu, rows)
    assert np.array_equal(qr, q[rows]) and np.array_equal(sr, s[rows])


# ------------------------------------------------ weight dequantize / LoRA merge

def test_dequantize_weight_closed_form():
    """W = RN((H q / 16) * s) per 256-group, from the Sylvester matrix in exact
    integer arithmetic and the scale applied in fp64 (exact: under 40 bits),
    then one rounding to fp32: bit-equal to the oracle.  A wrong axis, sign,
    group, normalization or row scale fails."""
    rng = np.random.default_rng(51)
    n, k = 12, 768
    q = rng.integers(-127, 128, size=(n, k), dtype=np.int8)
    q[0] = 127                                 # extremes of the exact range
    q[1] = -127
    s = (rng.random(n) * 0.05 + 1e-4).astype(np.float32)
    s[2] = np.float32(2.0 ** -20)
    H = hd.H().astype(np.int64)
    rot = np.concatenate([q[:, g * 256:(g + 1) * 256].astype(np.int64) @ H for g in range(k // 256)], axis=1)
    ref = ((rot.astype(np.float64) / 16.0) * s[:, None].astype(np.float64)).astype(np.float32)
    w = oracle.dequantize_weight(q, s)
    assert np.array_equal(w.view(np.uint32), ref.view(np.uint32))


def test_dequantize_requantize_round_trip():
    """Quantizing dequantized weights returns the same codes (the rotation
    back and forth moves each value by far less than half a code step) and
    scales within 2 ulps; a merge with zero strength changes no code."""
    rng = np.random.default_rng(52)
    w = (0.02 * rng.standard_normal((40, 1024))).astype(np.float32)
    w[:, rng.choice(1024, 8, replace=False)] *= 20
    q, s = oracle.quantize_weight(w)
    q2, s2 = oracle.quantize_weight(oracle.dequantize_weight(q, s))
    assert np.array_equal(q, q2)
    assert np.abs(s2.view(np.int32).astype(np.int64) - s.view(np.int32)).max() <= 2
    b = rng.standard_normal((40, 8)).astype(np.float32)
    a = rng.standard_normal((8, 1024)).astype(np.float32)
    q3, _ = oracle.merge_lora(q, s, b, a, 0.0)
    assert np.array_equal(q, q3)


def test_lora_add_exact_on_integers():
    """Small-integer factors and weights keep every fp32 step exact, so
    W + scale (B . A) must equal numpy's int64 matmul exactly (B is [n, rank],
    A is [rank, k]; a transposed or swapped operand fails)."""
    rng = np.random.default_rng(53)
    n, k, r = 20, 512, 16
    b = rng.integers(-8, 9, size=(n, r))
    a = rng.integers(-8, 9, size=(r, k))
    w = rng.integers(-1000, 1001, size=(n, k))
    for scale in (1.0, 0.5, -2.0):
        got = oracle.lora_add(w.astype(np.float32), b.astype(np.float32), a.astype(np.float32), scale)
        ref = w + scale * (b @ a)
        assert np.array_equal(got, ref.astype(np.float32)), scale


def test_lora_add_rounding_bound():
    """Random fp32 factors: within the sequential fused-multiply-add summation
    bound gamma_r * sum|b a| (scaled), plus one rounding each for the scale
    multiply and the final add, of the fp64 value."""
    rng = np.random.default_rng(54)
    n, k, r = 16, 256, 64
    b = rng.standard_normal((n, r)).astype(np.float32)
    a = rng.standard_normal((r, k)).astype(np.float32)
    w = rng.standard_normal((n, k)).astype(np.float32)
    scale = np.float32(0.37)
    got = oracle.lora_add(w, b, a, scale).astype(np.float64)
    d64 = b.astype(np.float64) @ a.astype(np.float64)
    ref = w.astype(np.float64) + float(scale) * d64
    gamma = r * U / (1 - r * U)
    bound = (abs(float(scale)) * (gamma * (np.abs(b).astype(np.float64) @ np.abs(a).astype(np.float64))
                                  + 2 * U * np.abs(d64)) + 2 * U * np.abs(ref))
    assert np.all(np.abs(got - ref) <= bound)


# ------------------------------------------------------------------ attention

def _attn(qc, sq, kc, sk, v):
    return oracle.attention_rows(np.asarray(qc, np.int8), np.asarray(sq, np.float32),
                                 np.asarray(kc, np.int8), np.asarray(sk, np.float32),
                                 np.asarray(v, np.float16))


def test_attention_two_keys_closed_form():
    """Hand-derived: d = 4 (so 1/sqrt(d) = 1/2), q = (1, 2, 3, 4) with s_q =
    1/8; k_0 = (4, 3, 2, 1) with s_k = 1/4, k_1 = (-1, 0, 1, 0) with s_k = 1/2.
    Integer dots 20 and 2, logits 20/64 = 0.3125 and 2/32 = 0.0625, so the
    first key's weight is the logistic of 0.25.  A wrong sign, a dropped
    1/sqrt(d), a scale taken from the wrong index or a transposed code matrix
    each changes the weight."""
    v = np.array([[1.0, -2.0, 0.5, 8.0], [3.0, 4.0, -0.25, 0.0]])
    o, a = _attn([[1, 2, 3, 4]], [0.125], [[4, 3, 2, 1], [-1, 0, 1, 0]], [0.25, 0.5], v)
    w0 = 1.0 / (1.0 + math.exp(-0.25))
    ref = w0 * v[0] + (1.0 - w0) * v[1]
    assert np.allclose(o[0], ref, rtol=1e-15, atol=1e-15)
    assert np.allclose(a[0], w0 * np.abs(v[0]) + (1 - w0) * np.abs(v[1]), rtol=1e-15, atol=1e-15)


def test_attention_uniform_keys_and_zero_query():
    """Identical keys (codes and scale), or an all-zero query (s_q = 0): every
    logit is equal, so the output is the plain mean of the values."""
    rng = np.random.default_rng(60)
    s, d = 37, 128
    v = rng.integers(-64, 65, size=(s, d)) / 8.0
    kc_row = rng.integers(-127, 128, size=d)
    kc = np.tile(kc_row, (s, 1))
    qc = rng.integers(-127, 128, size=(3, d))
    o, _ = _attn(qc, [0.01, 0.5, 3.0], kc, np.full(s, 0.02), v)
    assert np.allclose(o, np.tile(v.mean(axis=0), (3, 1)), rtol=1e-14, atol=1e-14)
    kc2 = rng.integers(-127, 128, size=(s, d))
    o2, _ = _attn(qc[:1], [0.0], kc2, rng.uniform(0.01, 0.1, s), v)
    assert np.allclose(o2[0], v.mean(axis=0), rtol=1e-14, atol=1e-14)


def test_attention_large_logits_keep_finite():
    """Logits near 894 (exp would overflow without the max subtraction); two
    keys share the codes and differ in scale, so the weight of the first is
    the logistic of the logit difference, computed here from the definition's
    logits in fp64."""
    d = 128
    q = np.full((1, d), 127)
    kc = np.full((2, d), 127)
    sq, sk = np.float32(0.07), np.array([0.07, 0.0699], np.float32)
    acc = 127 * 127 * d
    l = [acc * float(sq) * float(x) / math.sqrt(d) for x in sk]
    assert l[0] > 800
    v = np.array([np.full(d, 1.0), np.full(d, -1.0)])
    o, _ = _attn(q, [sq], kc, sk, v)
    w0 = 1.0 / (1.0 + math.exp(-(l[0] - l[1])))
    assert np.all(np.isfinite(o))
    assert np.allclose(o[0], w0 - (1 - w0), rtol=1e-12, atol=1e-12)


def test_attention_key_permutation_and_affine_values():
    """Keys are a set: permuting key codes, key scales and value rows together
    leaves the output unchanged; the weights sum to one, so values 2 v + 1
    (exact in fp16 here) give 2 O + 1, and each output lies between the
    smallest and largest value of its column."""
    rng = np.random.default_rng(61)
    nq, s, d = 5, 41, 128
    qc = rng.integers(-127, 128, size=(nq, d))
    kc = rng.integers(-127, 128, size=(s, d))
    sq = rng.uniform(0.001, 0.01, nq)
    sk = rng.uniform(0.001, 0.01, s)
    v = rng.integers(-64, 65, size=(s, d)) / 8.0
    o, _ = _attn(qc, sq, kc, sk, v)
    p = rng.permutation(s)
    o_p, _ = _attn(qc, sq, kc[p], sk[p], v[p])
    assert np.allclose(o_p, o, rtol=1e-13, atol=1e-13)
    o_a, _ = _attn(qc, sq, kc, sk, 2 * v + 1)
    assert np.allclose(o_a, 2 * o + 1, rtol=1e-13, atol=1e-13)
    assert np.all(o >= v.min(axis=0) - 1e-12) and np.all(o <= v.max(axis=0) + 1e-12)
    # the logits are not flat here (else the checks above say little)
    assert np.abs(o - v.mean(axis=0)).max() > 0.1


def test_attention_bruteforce_decimal():
    """Tiny random case against 40-digit decimal arithmetic from the integer
    codes and the exact binary values of the fp32 scales."""
    import decimal
    from fractions import Fraction
    decimal.getcontext().prec = 40
    D = decimal.Decimal
    rng = np.random.default_rng(62)
    nq, s, d = 3, 6, 8
    qc = rng.integers(-127, 128, size=(nq, d))
    kc = rng.integers(-127, 128, size=(s, d))
    sq = rng.uniform(0.005, 0.03, nq).astype(np.float32)
    sk = rng.uniform(0.005, 0.03, s).astype(np.float32)
    v = (rng.standard_normal((s, d))).astype(np.float16)
    o, _ = _attn(qc, sq, kc, sk, v)
    root_d = D(d).sqrt()
    for i in range(nq):
        logits = []
        for j in range(s):
            acc = int(np.dot(qc[i].astype(np.int64), kc[j].astype(np.int64)))
            f = Fraction(acc) * Fraction(float(sq[i])) * Fraction(float(sk[j]))
            logits.append(D(f.numerator) / D(f.denominator) / root_d)
        m = max(logits)
        p = [(x - m).exp() for x in logits]
        z = sum(p)
        for c in range(d):
            ref = sum(p[j] * D(float(v[j, c])) for j in range(s)) / z
            assert abs(o[i, c] - float(ref)) <= 1e-13 * (1 + abs(float(ref))), (i, c)


def test_attention_quant_is_the_per_row_quantizer():
    """Q and K codes: the per-row absmax/127 quantizer on the widened bf16
    values of each token's head slice, bit for bit against an exact-rational
    evaluation of rint(v / s) with s = RN(max|v| / 127)."""
    from fractions import Fraction
    rng = np.random.default_rng(63)
    x = workloads.to_bf16_bits(rng.standard_normal((20, 128)).astype(np.float32) * 3)
    q, s = oracle.attention_quant(x)
    f = oracle.bf16_to_f32(x)
    for r in range(20):
        amax = np.abs(f[r]).max()
        assert s[r] == np.float32(amax) / np.float32(127.0)
        for c in range(128):
            t = Fraction(float(f[r, c])) / Fraction(float(s[r]))
            n = round(t)          # Python rounds exact halves to even
            assert q[r, c] == max(-127, min(127, n)), (r, c)


# ------------------------------------------------------------------ MXFP4

# FP4 E2M1 magnitudes in code order (code = exponent bits 2..1, mantissa bit 0),
# as the OCP Microscaling format lists them.
E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def _nibbles(codes):
    lo, hi = codes & 15, codes >> 4
    return np.stack([lo, hi], axis=-1).reshape(codes.shape[0], -1)


def test_mx_element_values():
    """Every one of the 16 codes decodes (with a unit scale, code 127) to the
    listed magnitude with the sign bit's sign."""
    codes = np.array([[(2 * j) | ((2 * j + 1) << 4) for j in range(8)] + [0] * 8], np.uint8)
    scales = np.array([[127]], np.uint8)
    got = oracle.mx_decode(codes, scales)[0, :16]
    want = [E2M1[c & 7] * (-1 if c & 8 else 1) for c in range(16)]
    assert np.array_equal(got, np.array(want))


def test_mx_packing_hand_example():
    """Hand-derived: a block whose largest magnitude is 6 takes scale 2^0
    (floor(log2 6) - 2 = 0, code 127); 1.0 is code 2, -0.5 is code 9, so the
    first byte is 0x92 (element 0 in the low nibble)."""
    v = np.zeros((1, 32), np.float32)
    v[0, 0], v[0, 1], v[0, 2] = 1.0, -0.5, 6.0
    codes, scales = oracle.mx_quantize(v)
    assert scales[0, 0] == 127
    assert codes[0, 0] == 0x92 and codes[0, 1] == 0x07


def test_mx_rounding_brute_force():
    """With a block maximum of 4 (scale 2^0), every grid value y in (-8, 8)
    (steps of 1/64, which include every midpoint) rounds to the nearest listed
    magnitude; at a midpoint the even code wins; above 6 it saturates."""
    ys = np.arange(-511, 512) / 64.0
    for chunk in range(0, ys.size, 31):
        part = ys[chunk:chunk + 31]
        v = np.zeros((1, 32), np.float32)
        v[0, 0] = 4.0                       # sets the scale to 2^0 (floor(log2 4) - 2 = 0) ...
        v[0, 1:1 + part.size] = part        # ... unless a grid value reaches 8 (|y| < 8 here)
        codes, scales = oracle.mx_quantize(v)
        assert scales[0, 0] == 127
        nib = _nibbles(codes)[0]
        for j, y in enumerate(part):
            c = int(nib[1 + j])
            a = abs(y)
            if a >= 6.0:
                want = 7
            else:
                d = [abs(a - m) for m in E2M1]
                best = min(d)
                cands = [i for i in range(8) if d[i] == best]
                want = cands[0] if len(cands) == 1 else [i for i in cands if i % 2 == 0][0]
            assert (c & 7) == want, (y, c, want)
            assert bool(c & 8) == bool(np.signbit(np.float32(y))), y


def test_mx_scale_exponent_exact():
    """For random blocks over a wide magnitude range, the scale exponent e puts
    the block maximum in [4, 8) * 2^e (checked with exact rationals); an
    all-zero block has code 0; exponents clamp to the E8M0 range."""
    from fractions import Fraction
    rng = np.random.default_rng(70)
    v = (rng.standard_normal((64, 32)) * np.exp2(rng.integers(-40, 40, size=(64, 1)))).astype(np.float32)
    v[5] = 0.0
    codes, scales = oracle.mx_quantize(v)
    for r in range(64):
        amax = np.abs(v[r]).max()
        if amax == 0:
            assert scales[r, 0] == 0
            continue
        e = int(scales[r, 0]) - 127
        q = Fraction(float(amax)) / Fraction(2) ** e
        assert Fraction(4) <= q < Fraction(8), (r, e, float(q))
    tiny = np.full((1, 32), 1e-39, np.float32)      # floor(log2) - 2 = -132 -> clamps to -127
    _, s_t = oracle.mx_quantize(tiny)
    assert s_t[0, 0] == 0


def test_mx_roundtrip_bound():
    """|v - decode(quantize(v))| <= 2^e for unsaturated elements (half the
    widest gap, 2, between listed magnitudes) and <= 2^(e+1) for saturated
    ones (|v| / 2^e < 8); signs agree wherever the decoded value is nonzero."""
    rng = np.random.default_rng(71)
    v = rng.standard_normal((50, 256)).astype(np.float32) * 3
    codes, scales = oracle.mx_quantize(v)
    d = oracle.mx_decode(codes, scales)
    e = np.repeat(scales.astype(np.int64) - 127, 32, axis=1)
    unit = np.exp2(e.astype(np.float64))
    y = v / unit
    err = np.abs(v - d)
    assert np.all(err[np.abs(y) <= 6] <= unit[np.abs(y) <= 6])
    assert np.all(err <= 2 * unit)
    nz = d != 0
    assert np.all(np.sign(d[nz]) == np.sign(v[nz]))


def test_mx_gemm_against_dense():
    """The MX product equals numpy's fp64 product of the decoded matrices
    exactly (every product is a short binary fraction, so every partial sum
    is exact in fp64), with A and B of different shapes (a transposed or
    swapped operand fails); sum |a b| bounds |y|."""
    rng = np.random.default_rng(72)
    a = rng.standard_normal((7, 128)).astype(np.float32)
    b = rng.standard_normal((5, 128)).astype(np.float32) * 10
    ac, asc = oracle.mx_quantize(a)
    bc, bsc = oracle.mx_quantize(b)
    y, absacc = oracle.mx_gemm(ac, asc, bc, bsc)
    ref = oracle.mx_decode(ac, asc) @ oracle.mx_decode(bc, bsc).T
    assert np.array_equal(y, ref)
    assert np.all(np.abs(y) <= absacc)
    assert np.allclose(absacc, np.abs(oracle.mx_decode(ac, asc)) @ np.abs(oracle.mx_decode(bc, bsc)).T)


def test_mx_rotated_composition():
    """Rotated MXFP4: rotating the decoded values back (H/16 is its own
    inverse) returns the input within the block error in the rotated basis
    (the rotation preserves every 256-group's norm), and the product of two
    rotated operands approximates the unrotated product x W^T; on rows with
    an outlier channel the rotated format is closer to x W^T than the plain
    one (the reason to rotate)."""
    rng = np.random.default_rng(73)
    x = rng.standard_normal((24, 512)).astype(np.float32)
    x[:, 7] *= 30
    w = (rng.standard_normal((16, 512)) * 0.02).astype(np.float32)
    xc, xs = oracle.mx_quantize_rotated(x)
    d = oracle.mx_decode(xc, xs)
    back = oracle.rotate_rows(d.astype(np.float32)).astype(np.float64)
    r = oracle.rotate_rows(x).astype(np.float64)
    for g in range(2):
        sl = slice(256 * g, 256 * g + 256)
        assert np.allclose(np.linalg.norm(back[:, sl] - x[:, sl], axis=1),
                           np.linalg.norm(d[:, sl] - r[:, sl], axis=1), rtol=1e-5, atol=1e-6)
    y_rot, _ = oracle.mx_gemm(xc, xs, *oracle.mx_quantize_rotated(w))
    y_plain, _ = oracle.mx_gemm(*oracle.mx_quantize(x), *oracle.mx_quantize(w))
    ref = x.astype(np.float64) @ w.astype(np.float64).T
    e_rot = np.linalg.norm(y_rot - ref) / np.linalg.norm(ref)
    e_plain = np.linalg.norm(y_plain - ref) / np.linalg.norm(ref)
    assert e_rot < 0.2 and e_rot < e_plain, (e_rot, e_plain)
