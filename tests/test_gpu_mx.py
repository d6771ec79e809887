"""GPU parity of the MXFP4 path against the CPU oracle.

Bit-exact: the FP4 codes and E8M0 scales of activations (bf16) and weights
(fp32).  Products: within the fp32 accumulation of the MFMA and the bf16
store, per element |y - y_ref| <= 2^-8 |y_ref| + (k / 32) 2^-23 sum_k |a b|,
with y_ref and the sum from the oracle's exact fp64 evaluation."""
import numpy as np
import pytest

import oracle
import workloads
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def cr():
    import rotation_quantized_dit_amd as cr
    cr.load_library()
    return cr


def natural_scales(chunked):
    """Chunk-major [k/128, rows, 4] scales (the library's layout) -> the
    natural [rows, k/32] (a relayout, no arithmetic)."""
    c = np.asarray(chunked)
    return np.ascontiguousarray(c.transpose(1, 0, 2).reshape(c.shape[1], -1))


def assert_mx_product(y_bits, ref, absacc, k, what):
    g = gu.bf16_f64(y_bits)
    err = np.abs(g - ref)
    tol = 2.0 ** -8 * np.abs(ref) + (k / 32) * 2.0 ** -23 * absacc
    bad = err > tol
    if bad.any():
        i = np.unravel_index(np.argmax(err / np.maximum(tol, 1e-300)), err.shape)
        raise AssertionError("%s: %d of %d outside the bound; worst at %s: gpu %r ref %r tol %r" % (
            what, int(bad.sum()), bad.size, i, g[i], ref[i], tol[i]))
    print("%s: max err / bound = %.3f" % (what, float((err / np.maximum(tol, 1e-300)).max())), flush=True)


def edge_rows(k, rng):
    """Rows that hit every rounding case: all-zero and signed-zero blocks,
    exact midpoints and saturation at several scales, denormals, one huge
    value per block."""
    rows = []
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 7.0, 7.9375])
    for e in (-20, -3, 0, 5, 40):
        r = np.zeros(k, np.float32)
        for b in range(k // 32):
            blk = np.zeros(32, np.float32)
            blk[0] = 4.0                              # scale 2^0 before the shift by e
            blk[1:1 + mids.size] = mids * (1 if b % 2 else -1)
            blk[12:20] = rng.uniform(-6, 6, 8)
            r[32 * b:32 * b + 32] = blk * np.float32(2.0 ** e)
        rows.append(r)
    z = np.zeros(k, np.float32)
    z[32:64] = -0.0
    rows.append(z)
    d = np.full(k, 1e-40, np.float32)
    d[::3] = -3e-39
    rows.append(d)
    return np.stack(rows)


@pytest.mark.parametrize("m,k,rotate", [(1, 128, False), (7, 256, False), (64, 512, False),
                                        (300, 5376, False), (33, 14336, False), (1, 256, True),
                                        (9, 512, True), (300, 5376, True), (33, 14336, True)])
def test_mx_quantize_parity(cr, m, k, rotate):
    import torch
    rng = np.random.default_rng(200 + m)
    x = rng.standard_normal((m, k)).astype(np.float32) * rng.choice([0.01, 1, 30], size=(m, 1)).astype(np.float32)
    x = np.concatenate([x, edge_rows(k, rng)])
    xb = workloads.to_bf16_bits(x)
    qc_d, qs_d = cr.mx_quantize_act(gu.dev_bf16(xb), rotate=rotate)
    wc_d, ws_d = cr.mx_quantize_weight(gu.dev(x), rotate=rotate)
    torch.cuda.synchronize()
    if rotate:
        qc, qs = oracle.mx_quantize_act_rotated(xb)
        wc, ws = oracle.mx_quantize_rotated(x)
    else:
        qc, qs = oracle.mx_quantize_act(xb)
        wc, ws = oracle.mx_quantize(x)
    gu.assert_equal(gu.host(qc_d), qc, "activation codes")
    gu.assert_equal(natural_scales(gu.host(qs_d)), qs, "activation scales")
    gu.assert_equal(gu.host(wc_d), wc, "weight codes")
    gu.assert_equal(natural_scales(gu.host(ws_d)), ws, "weight scales")


@pytest.mark.parametrize("m,n,k,rotate", [(1, 1, 128, False), (5, 37, 128, False), (64, 256, 256, False),
                                          (257, 300, 384, False), (300, 513, 5376, False),
                                          (512, 64, 14336, False), (33, 70, 256, True),
                                          (300, 513, 5376, True)])
def test_mx_gemm_parity(cr, m, n, k, rotate):
    import torch
    rng = np.random.default_rng(300 + m + n)
    x = rng.standard_normal((m, k)).astype(np.float32)
    x[:, rng.choice(k, max(1, k // 100), replace=False)] *= 30
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    xb = workloads.to_bf16_bits(x)
    xd, wd = gu.dev_bf16(xb), gu.dev(w)
    ac, asc = cr.mx_quantize_act(xd, rotate=rotate)
    bc, bsc = cr.mx_quantize_weight(wd, rotate=rotate)
    y = cr.mx_gemm(ac, asc, bc, bsc)
    y2 = cr.mx_linear(xd, bc, bsc, rotate=rotate)
    torch.cuda.synchronize()
    if rotate:
        oac, oas = oracle.mx_quantize_act_rotated(xb)
        obc, obs = oracle.mx_quantize_rotated(w)
    else:
        oac, oas = oracle.mx_quantize_act(xb)
        obc, obs = oracle.mx_quantize(w)
    gu.assert_equal(gu.host(ac), oac, "A codes")
    gu.assert_equal(gu.host(bc), obc, "B codes")
    gu.assert_equal(natural_scales(gu.host(asc)), oas, "A scales")
    gu.assert_equal(natural_scales(gu.host(bsc)), obs, "B scales")
    ref, absacc = oracle.mx_gemm(oac, oas, obc, obs)
    yb = gu.host_bf16(y)
    assert_mx_product(yb, ref, absacc, k, "mx_gemm %dx%dx%d" % (m, n, k))
    gu.assert_equal(gu.host_bf16(y2), yb, "mx_linear vs quantize + mx_gemm")


def test_mx_gemm_deterministic_and_exact_on_small_integers(cr):
    """Codes whose products and sums are exact in fp32 (one scale, few
    blocks): the bf16 output equals the oracle's exact value rounded once;
    two calls give the same bytes."""
    import torch
    rng = np.random.default_rng(7)
    m, n, k = 96, 80, 256
    x = rng.integers(-6, 7, size=(m, k)).astype(np.float32)
    x[:, 0] = 6.0                                   # every block max 6 -> scale 2^0
    x[:, 32::32] = 6.0
    w = rng.integers(-4, 5, size=(n, k)).astype(np.float32)
    w[:, ::32] = 4.0
    xd, wd = gu.dev_bf16(workloads.to_bf16_bits(x)), gu.dev(w)
    ac, asc = cr.mx_quantize_act(xd)
    bc, bsc = cr.mx_quantize_weight(wd)
    y1 = gu.host_bf16(cr.mx_gemm(ac, asc, bc, bsc))
    y2 = gu.host_bf16(cr.mx_gemm(ac, asc, bc, bsc))
    torch.cuda.synchronize()
    ref, _ = oracle.mx_gemm(*oracle.mx_quantize(x), *oracle.mx_quantize(w))
    gu.assert_equal(y1, y2, "two calls")
    gu.assert_equal(y1, workloads.to_bf16_bits(ref.astype(np.float32)), "exact small-integer product")


def test_mx_validation(cr):
    import torch
    x = torch.zeros(4, 200, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(cr.ConvRotError):
        cr.mx_quantize_act(x)                       # k not a multiple of 128
    x2 = torch.zeros(4, 384, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(cr.ConvRotError):
        cr.mx_quantize_act(x2, rotate=True)         # rotation needs whole 256-groups


@pytest.mark.parametrize("name,rotate", [("qkv", False), ("ffn_up", False), ("qkv", True)])
def test_mx_full_size(cr, name, rotate):
    """The QKV (4096 x 5376 -> 16128) and FFN-input (32256 x 5376 -> 28672)
    shapes: every activation and weight code and scale bit for bit, and the
    product on sampled rows (first, last, 64 seeded)."""
    import torch
    c = workloads.WORKLOADS[name]
    print("mx full size %s: generating" % name, flush=True)
    d = workloads.make_linear(name)
    xd, wd = gu.dev_bf16(d["x"]), gu.dev(d["w"])
    ac, asc = cr.mx_quantize_act(xd, rotate=rotate)
    bc, bsc = cr.mx_quantize_weight(wd, rotate=rotate)
    y = cr.mx_linear(xd, bc, bsc, rotate=rotate)
    torch.cuda.synchronize()
    rows = workloads.sample_rows(c.m, seed=c.seed)
    g = dict(ac=gu.host(ac), asc=natural_scales(gu.host(asc)), bc=gu.host(bc), bsc=natural_scales(gu.host(bsc)),
             y=gu.host_bf16(y[torch.from_numpy(rows).cuda()]))
    del xd, wd, ac, asc, bc, bsc, y
    print("mx full size %s: oracle" % name, flush=True)
    if rotate:
        oac, oas = oracle.mx_quantize_act_rotated(d["x"])
        obc, obs = oracle.mx_quantize_rotated(d["w"])
    else:
        oac, oas = oracle.mx_quantize_act(d["x"])
        obc, obs = oracle.mx_quantize(d["w"])
    gu.assert_equal(g["ac"], oac, name + " activation codes")
    gu.assert_equal(g["asc"], oas, name + " activation scales")
    gu.assert_equal(g["bc"], obc, name + " weight codes")
    gu.assert_equal(g["bsc"], obs, name + " weight scales")
    ref, absacc = oracle.mx_gemm(oac[rows], oas[rows], obc, obs)
    assert_mx_product(g["y"], ref, absacc, c.k, name + " sampled rows")


@pytest.mark.parametrize("rotate", [False, True])
def test_mx_max_k(cr, rotate):
    """The largest K the MXFP4 entry points accept (2^20): every code and scale
    of 3 activation and 5 weight rows bit for bit, and the product within its
    bound (the fp32 accumulation term grows with k / 32)."""
    import torch
    k = 1 << 20
    rng = np.random.default_rng(77)
    x = rng.standard_normal((3, k)).astype(np.float32)
    x[:, rng.choice(k, 64, replace=False)] *= 30
    w = (0.02 * rng.standard_normal((5, k))).astype(np.float32)
    xb = workloads.to_bf16_bits(x)
    xd, wd = gu.dev_bf16(xb), gu.dev(w)
    ac, asc = cr.mx_quantize_act(xd, rotate=rotate)
    bc, bsc = cr.mx_quantize_weight(wd, rotate=rotate)
    y = cr.mx_gemm(ac, asc, bc, bsc)
    torch.cuda.synchronize()
    if rotate:
        oac, oas = oracle.mx_quantize_act_rotated(xb)
        obc, obs = oracle.mx_quantize_rotated(w)
    else:
        oac, oas = oracle.mx_quantize_act(xb)
        obc, obs = oracle.mx_quantize(w)
    gu.assert_equal(gu.host(ac), oac, "A codes at k = 2^20")
    gu.assert_equal(natural_scales(gu.host(asc)), oas, "A scales at k = 2^20")
    gu.assert_equal(gu.host(bc), obc, "B codes at k = 2^20")
    gu.assert_equal(natural_scales(gu.host(bsc)), obs, "B scales at k = 2^20")
    ref, absacc = oracle.mx_gemm(oac, oas, obc, obs)
    assert_mx_product(gu.host_bf16(y), ref, absacc, k, "mx_gemm 3x5x2^20")
