"""GPU parity on small and edge-case inputs: the HIP library (through the C
ABI) against the CPU oracle on the same seeded bytes.  Codes, scales and int32
accumulators must match bit for bit; bf16 outputs must meet the 1e-2 relative
bound.  The bf16 dequant epilogue, where both sides evaluate the same rounding
sequence, must also match bit for bit; the fused SwiGLU epilogue, which runs on
the hardware exponential and reciprocal, must lie within one bf16 ulp (2^-8
relative) of the oracle's exact value."""
import numpy as np
import pytest

import oracle
import workloads
from tests import gpu_util as gu
from tests import hadamard as hd

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def cr():
    import rotation_quantized_dit_amd as cr
    cr.load_library()
    return cr


def _f32_bits(a):
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


def run_all_stages(cr, x_bits, w, swiglu=False):
    """Every entry point on one input; returns GPU results and oracle results."""
    import torch
    xd, wd = gu.dev_bf16(x_bits), gu.dev(w)
    qw_d, sw_d = cr.quantize_weight(wd)
    qx_d, sx_d = cr.rotate_quant_act(xd)
    acc_d = cr.gemm_s32(qx_d, qw_d)
    if swiglu:
        y_d = cr.linear_swiglu(xd, qw_d, sw_d)
        y2_d = cr.gemm_swiglu(qx_d, sx_d, qw_d, sw_d)
    else:
        y_d = cr.linear(xd, qw_d, sw_d)
        y2_d = cr.gemm_dequant(qx_d, sx_d, qw_d, sw_d)
    torch.cuda.synchronize()
    g = dict(q_w=gu.host(qw_d), s_w=gu.host(sw_d), q_x=gu.host(qx_d), s_x=gu.host(sx_d),
             acc=gu.host(acc_d), y=gu.host_bf16(y_d), y2=gu.host_bf16(y2_d))
    qw, sw = oracle.quantize_weight(w)
    qx, sx = oracle.rotate_quant_act(x_bits)
    acc = oracle.gemm_s32(qx, qw)
    o = dict(q_w=qw, s_w=sw, q_x=qx, s_x=sx, acc=acc)
    if swiglu:
        o["ref"], o["mag"] = oracle.swiglu_ref(acc, sx, sw)
    else:
        o["y"] = oracle.dequant_bf16(acc, sx, sw)
    return g, o


def check_all(g, o, what):
    gu.assert_equal(g["q_w"], o["q_w"], what + " q_w")
    gu.assert_equal(_f32_bits(g["s_w"]), _f32_bits(o["s_w"]), what + " s_w")
    gu.assert_equal(g["q_x"], o["q_x"], what + " q_x")
    gu.assert_equal(_f32_bits(g["s_x"]), _f32_bits(o["s_x"]), what + " s_x")
    gu.assert_equal(g["acc"], o["acc"], what + " acc")
    if "ref" in o:
        gu.assert_swiglu_bound(g["y"], o["ref"], o["mag"], what + " y")
        gu.assert_equal(g["y2"], g["y"], what + " y (prepared codes) equals y")
    else:
        gu.assert_bf16_parity(g["y"], o["y"], what + " y")
        gu.assert_bf16_parity(g["y2"], o["y"], what + " y (prepared codes)")


def test_tiny_all_stages(cr):
    """The tiny workload (64 x 512 x 256, 4 outlier channels x50) in full."""
    d = workloads.make_linear("tiny")
    g, o = run_all_stages(cr, d["x"], d["w"])
    check_all(g, o, "tiny")


def test_tiny_swiglu(cr):
    """The tiny workload's weight read as a fused gate/up pair (i = 128)."""
    d = workloads.make_linear("tiny")
    g, o = run_all_stages(cr, d["x"], d["w"], swiglu=True)
    check_all(g, o, "tiny swiglu")


@pytest.mark.parametrize("m,n,k", [(1, 1, 256), (37, 100, 256), (300, 300, 768), (257, 513, 512),
                                   (511, 130, 1024), (64, 256, 5376), (385, 257, 1280), (769, 1025, 256)])
def test_ragged_shapes(cr, m, n, k):
    """Ragged token and output counts: tails of partial 384 x 256 tiles and of
    the 16-row / 16-column MFMA blocks inside them, one row or column past a
    tile boundary, and stage counts of one and five rounds of the ring."""
    rng = np.random.default_rng(m * 7 + n * 3 + k)
    x = rng.standard_normal((m, k), dtype=np.float32)
    x[:, rng.choice(k, 3, replace=False)] *= 40
    w = (0.02 * rng.standard_normal((n, k))).astype(np.float32)
    g, o = run_all_stages(cr, workloads.to_bf16_bits(x), w)
    check_all(g, o, "ragged %dx%dx%d" % (m, n, k))


@pytest.mark.parametrize("m,i,k", [(5, 1, 256), (300, 100, 512), (130, 200, 768), (385, 129, 1280)])
def test_ragged_swiglu(cr, m, i, k):
    rng = np.random.default_rng(m + i + k)
    x = rng.laplace(size=(m, k)).astype(np.float32)
    w = (0.05 * rng.standard_normal((2 * i, k))).astype(np.float32)
    g, o = run_all_stages(cr, workloads.to_bf16_bits(x), w, swiglu=True)
    check_all(g, o, "swiglu ragged %dx%dx%d" % (m, i, k))


def test_degenerate_rows(cr):
    """All-zero rows (s = 0, codes 0, y = 0), rows of tiny values (the exact
    division path for every element), a single non-zero, huge values."""
    k, n = 512, 64
    rng = np.random.default_rng(5)
    x = rng.standard_normal((8, k), dtype=np.float32)
    x[0] = 0
    x[1] *= np.float32(1e-33)
    x[2] = 0
    x[2, 77] = 3.0
    x[3] *= np.float32(1e30)
    x[4, :256] = 0
    w = (0.02 * rng.standard_normal((n, k))).astype(np.float32)
    w[0] = 0
    w[1] *= np.float32(1e-35)
    g, o = run_all_stages(cr, workloads.to_bf16_bits(x), w)
    check_all(g, o, "degenerate")
    assert g["s_x"][0] == 0 and not g["q_x"][0].any() and not g["y"][0].any()
    assert g["s_w"][0] == 0 and not g["q_w"][0].any()


def test_bf16_rounding_edges(cr):
    """The dequant epilogue's fp32 -> bf16 rounding on crafted values: one-hot
    weight rows make every output a single product of two int8 codes (many
    have 9+ significant bits, so exact half-way cases occur), and power-of-two
    scales move the products through the fp32 denormal range and past the
    largest finite value.  The oracle rounds half to even with denormals kept."""
    import torch
    rng = np.random.default_rng(23)
    m, n, k = 96, 256, 256
    qx = rng.integers(-127, 128, size=(m, k), dtype=np.int8)
    codes = rng.integers(1, 128, size=n) * rng.choice([-1, 1], size=n)
    qw = np.zeros((n, k), dtype=np.int8)
    qw[np.arange(n), np.arange(n)] = codes
    ex = rng.integers(-150, 30, size=m)
    ex[:4] = [0, -126, -133, 113]             # exact ties, denormal edge, deep denormal, overflow
    sx = np.ldexp(np.float32(1.0), ex).astype(np.float32)
    sw = np.ldexp(np.float32(1.0), rng.integers(-8, 9, size=n)).astype(np.float32)
    y = cr.gemm_dequant(gu.dev(qx), gu.dev(sx), gu.dev(qw), gu.dev(sw))
    torch.cuda.synchronize()
    acc = oracle.gemm_s32(qx, qw)
    ref = oracle.dequant_bf16(acc, sx, sw)
    got = gu.host_bf16(y)
    f = (acc.astype(np.float64) * sx[:, None].astype(np.float64)) * sw[None, :].astype(np.float64)
    assert np.any(np.abs(f) < 2.0 ** -126) and np.any(np.abs(f) > 3.4e38)   # both ranges are hit
    gu.assert_equal(got, ref, "bf16 rounding edges")


def test_tie_rows_half_even(cr):
    """Rows whose rotation is exactly a half-integer multiple of the scale
    (amax 127 s) round half to even on the GPU as in the oracle."""
    H = hd.H().astype(np.float64)
    rng = np.random.default_rng(17)
    values = [127.0, 2.5, 3.5, -2.5, -0.5, 0.5, 1.5, -1.5, 126.5, -126.5, 4.5, -3.5, 0.0, 5.5, 6.5, -7.5]
    rows = []
    for e in (0, -3, 5, -10):
        row = np.zeros(256 * len(values))
        for gi, v in enumerate(values):
            j = int(rng.integers(0, 256))
            row[gi * 256:(gi + 1) * 256] = v * 2.0 ** e * H[:, j] / 16
        rows.append(row)
    x = np.array(rows)
    assert hd.is_bf16_exact(x)
    w = x.astype(np.float32)              # the same rows through the fp32 weight path
    g, o = run_all_stages(cr, workloads.to_bf16_bits(x.astype(np.float32)), w)
    check_all(g, o, "ties")


def test_correctly_rounded_quotients(cr):
    """Cases where rint(v * RN(1/s)) != rint(RN(v / s)) (exact rationals in the
    oracle pins): the GPU takes the exact quotient."""
    H = hd.H().astype(np.float64)
    cases = [(56.25, -28.125), (61.0, 30.5), (44.75, 22.375), (9.8125, -4.90625),
             (3.765625, -1.8828125), (43.75, 21.875), (19.5, 9.75), (19.5, -9.75)]
    rows = []
    for amax, v in cases:
        row = np.zeros(512)
        row[:256] = amax * H[:, 3] / 16
        row[256:] = v * H[:, 77] / 16
        rows.append(row)
    x = np.array(rows).astype(np.float32)
    rng = np.random.default_rng(3)
    w = (0.1 * rng.standard_normal((32, 512))).astype(np.float32)
    w[:8] = x                             # and the weight path
    g, o = run_all_stages(cr, workloads.to_bf16_bits(x), w)
    check_all(g, o, "quotients")


def test_two_pass_long_rows(cr):
    """k = 129 groups (33024) exceeds the register-resident row and takes the
    recomputing second pass."""
    rng = np.random.default_rng(9)
    k = 129 * 256
    x = rng.standard_normal((3, k), dtype=np.float32)
    x[:, 5] *= 60
    w = (0.01 * rng.standard_normal((40, k))).astype(np.float32)
    g, o = run_all_stages(cr, workloads.to_bf16_bits(x), w)
    check_all(g, o, "two-pass k=33024")


def test_int32_extreme_at_max_k(cr):
    """k = 133120, every code +-127: acc = +-127^2 k = +-2,147,092,480 exactly."""
    import torch
    k = 133120
    qx = torch.full((3, k), 127, dtype=torch.int8, device="cuda")
    qx[1] = -127
    qw = torch.full((2, k), 127, dtype=torch.int8, device="cuda")
    acc = gu.host(cr.gemm_s32(qx, qw))
    assert acc[0, 0] == 2147092480 and acc[1, 1] == -2147092480 and acc[2, 0] == 2147092480


def test_max_k_rotate_quant(cr):
    """The largest k the boundary accepts, through rotation and quantization."""
    rng = np.random.default_rng(10)
    k = 133120
    x = rng.standard_normal((2, k), dtype=np.float32)
    xb = workloads.to_bf16_bits(x)
    qx, sx = cr.rotate_quant_act(gu.dev_bf16(xb))
    oq, os_ = oracle.rotate_quant_act(xb)
    gu.assert_equal(gu.host(qx), oq, "q_x max k")
    gu.assert_equal(_f32_bits(gu.host(sx)), _f32_bits(os_), "s_x max k")


def _swiglu_pairs_input(m, i, seed):
    """fc1-output-like bf16 gate/up rows [m, 2i] with special rows: an all-zero
    up half (scale 0), gates below -88.72 (silu underflows to -0), large gates
    (silu(g) = g), and mixed magnitudes elsewhere."""
    rng = np.random.default_rng(seed)
    g = rng.standard_normal((m, i)) * np.array([0.5, 4.0, 30.0])[rng.integers(0, 3, (m, i))]
    u = rng.standard_normal((m, i)) * 3.0
    if m > 0:
        u[0] = 0.0
    if m > 1:
        g[1, ::3] = -200.0
    if m > 2:
        g[2] = 150.0 + rng.random(i)
    return workloads.to_bf16_bits(np.concatenate([g, u], axis=1).astype(np.float32))


@pytest.mark.parametrize("m,i", [(1, 256), (37, 768), (300, 5376), (64, 14336), (3, 33024), (2, 133120)])
def test_swiglu_rotate_quant(cr, m, i):
    """SwiGLU on fc1's bf16 output, then rotate + quantize per token: codes and
    scales bit-exact against the oracle (row kernel for 1..32 groups per pass,
    the recomputing kernel for 129 and 520 groups)."""
    gu_in = _swiglu_pairs_input(m, i, seed=m + i)
    qh, sh = cr.swiglu_rotate_quant_act(gu.dev_bf16(gu_in))
    oq, os_ = oracle.swiglu_rotate_quant_act(gu_in)
    gu.assert_equal(gu.host(qh), oq, "swiglu_rotate_quant q_h %dx%d" % (m, i))
    gu.assert_equal(_f32_bits(gu.host(sh)), _f32_bits(os_), "swiglu_rotate_quant s_h %dx%d" % (m, i))
    if m > 0:
        assert gu.host(sh)[0] == 0 and not gu.host(qh)[0].any()


def test_swiglu_rotate_quant_near_bf16_midpoints(cr):
    """h = bf16(silu(g) u) where the fp32 value lies within a few units in
    the last place of a bf16 rounding midpoint, the cases where any evaluation
    but the definition's could round h the other way.  Each row holds one
    such (g, u) pair and zeros elsewhere, so the rotated row is +-h/16 at every
    position and the row scale |h| / 16 / 127 pins h's bf16 value: scales and
    codes must equal the oracle's bit for bit.  Pairs are picked from a seeded
    pool by an fp64 estimate of h (the expected values are the oracle's);
    g spans both signs well past |g| = 16, down to -88.5, where the
    exponential of -g is near the top of the fp32 range.  Further rows, not
    picked near midpoints: g in [-120, -60] (for g <= -89 the definition's
    exponential overflows and its quotient is -0), and |g| near 2^60..2^70,
    where the fast quotient overflows and the definition is taken.  Last,
    exact ties g u for every bf16 gate in (16, 20): from 16.75 on the
    quotient is g itself and the fast value is taken as it stands."""
    rng = np.random.default_rng(77)
    n = 1 << 24
    sig = rng.choice(np.array([0.3, 2.0, 6.0, 14.0, 40.0, 71.0], dtype=np.float32), n)
    g = oracle.bf16_to_f32(workloads.to_bf16_bits(rng.standard_normal(n, dtype=np.float32) * sig))
    u = oracle.bf16_to_f32(workloads.to_bf16_bits(
        rng.standard_normal(n, dtype=np.float32) * rng.choice(np.array([1e-3, 1.0, 300.0], dtype=np.float32), n)))
    g64 = g.astype(np.float64)
    with np.errstate(over="ignore"):
        h = (g64 / (1.0 + np.exp(-g64)) * u.astype(np.float64)).astype(np.float32)
    low = h.view(np.uint32) & 0xFFFF
    near = (np.abs(low.astype(np.int64) - 0x8000) <= 12) & (h != 0)
    # for g > 16 silu(g) u is often the exact product g u, a bf16 tie; keep
    # every range in the sample
    small = np.nonzero(near & (np.abs(g) <= 16))[0][:4000]
    pos = np.nonzero(near & (g > 16))[0][:1000]
    neg = np.nonzero(near & (g < -16))[0][:1000]
    assert small.size > 1500 and pos.size > 300 and neg.size > 300, (small.size, pos.size, neg.size)
    pick = np.concatenate([small, pos, neg])
    g_pick, u_pick = g[pick], u[pick]
    tail_g = oracle.bf16_to_f32(workloads.to_bf16_bits(rng.uniform(-120.0, -60.0, 1000).astype(np.float32)))
    tail_u = oracle.bf16_to_f32(workloads.to_bf16_bits(rng.standard_normal(1000, dtype=np.float32)))
    huge_g = oracle.bf16_to_f32(workloads.to_bf16_bits(
        (rng.choice([-1.0, 1.0], 100) * np.exp2(rng.uniform(60.0, 70.0, 100))).astype(np.float32)))
    huge_u = oracle.bf16_to_f32(workloads.to_bf16_bits((1e-3 * rng.standard_normal(100)).astype(np.float32)))
    # exact bf16 ties g u with g on the bf16 grid around 16.75, where
    # 1 + exp(-g) first rounds to 1 and the quotient becomes g itself
    edge_g = np.repeat(np.arange(16.125, 20.0, 0.125, dtype=np.float32), 4096)
    edge_u = oracle.bf16_to_f32(workloads.to_bf16_bits(
        rng.standard_normal(edge_g.size, dtype=np.float32) * rng.choice(np.array([1.0, 300.0], dtype=np.float32), edge_g.size)))
    tie = ((edge_g.astype(np.float64) * edge_u).astype(np.float32).view(np.uint32) & 0xFFFF) == 0x8000
    edge = np.nonzero(tie)[0]
    assert edge.size > 500 and np.unique(edge_g[edge]).size == 31, edge.size
    g_pick = np.concatenate([g_pick, tail_g, huge_g, edge_g[edge]])
    u_pick = np.concatenate([u_pick, tail_u, huge_u, edge_u[edge]])
    m, i = g_pick.size, 256
    gu_rows = np.zeros((m, 2 * i), dtype=np.float32)
    cols = rng.integers(0, i, m)
    gu_rows[np.arange(m), cols] = g_pick
    gu_rows[np.arange(m), i + cols] = u_pick
    gu_in = workloads.to_bf16_bits(gu_rows)
    qh, sh = cr.swiglu_rotate_quant_act(gu.dev_bf16(gu_in))
    oq, os_ = oracle.swiglu_rotate_quant_act(gu_in)
    gu.assert_equal(_f32_bits(gu.host(sh)), _f32_bits(os_), "near-midpoint s_h (%d rows)" % m)
    gu.assert_equal(gu.host(qh), oq, "near-midpoint q_h (%d rows)" % m)


def test_output_side_swiglu_chain_small(cr):
    """The whole FFN with SwiGLU on fc1's output side, small: x -> fc1 (bf16
    dequant on 2i columns) -> SwiGLU + rotate + quantize -> down GEMM, against
    the oracle's composition of the same steps, bit for bit at every stage."""
    import torch
    rng = np.random.default_rng(41)
    m, k, i, n = 200, 512, 768, 300
    x = rng.laplace(size=(m, k)).astype(np.float32)
    x[:, rng.choice(k, 5, replace=False)] *= 30
    xb = workloads.to_bf16_bits(x)
    w1 = (0.05 * rng.standard_normal((2 * i, k))).astype(np.float32)
    w2 = (0.03 * rng.standard_normal((n, i))).astype(np.float32)
    q1, s1 = cr.quantize_weight(gu.dev(w1))
    q2, s2 = cr.quantize_weight(gu.dev(w2))
    gu_d = cr.linear(gu.dev_bf16(xb), q1, s1)
    qh, sh = cr.swiglu_rotate_quant_act(gu_d)
    y = cr.gemm_dequant(qh, sh, q2, s2)
    torch.cuda.synchronize()
    oq1, os1 = oracle.quantize_weight(w1)
    oq2, os2 = oracle.quantize_weight(w2)
    ogu = oracle.linear_rows(xb, oq1, os1)
    oqh, osh = oracle.swiglu_rotate_quant_act(ogu)
    oy = oracle.dequant_bf16(oracle.gemm_s32(oqh, oq2), osh, os2)
    gu.assert_bf16_parity(gu.host_bf16(gu_d), ogu, "output-side chain: fc1 gate/up")
    gu.assert_equal(gu.host(qh), oqh, "output-side chain: q_h")
    gu.assert_equal(_f32_bits(gu.host(sh)), _f32_bits(osh), "output-side chain: s_h")
    gu.assert_bf16_parity(gu.host_bf16(y), oy, "output-side chain: y")


@pytest.mark.parametrize("n,k", [(1, 256), (37, 768), (100, 5376), (3, 133120)])
def test_dequantize_weight(cr, n, k):
    """W = RN((H q / 16) * s): bit-exact against the oracle, codes at +-127
    included, on ragged row counts and up to the largest k."""
    rng = np.random.default_rng(n + k)
    q = rng.integers(-127, 128, size=(n, k), dtype=np.int8)
    q[0, :256] = 127
    s = (rng.random(n) * 0.05 + 1e-5).astype(np.float32)
    w = cr.dequantize_weight(gu.dev(q), gu.dev(s))
    gu.assert_equal(_f32_bits(gu.host(w)), _f32_bits(oracle.dequantize_weight(q, s)),
                    "dequantize_weight %dx%d" % (n, k))


@pytest.mark.parametrize("n,k,r", [(5, 256, 0), (9, 512, 1), (37, 768, 7), (100, 1024, 64)])
def test_lora_add(cr, n, k, r):
    """W += scale * (B . A) with the fp32 order of the definition: bit-exact
    against the oracle (rank 0 included; rows not a multiple of 8)."""
    rng = np.random.default_rng(n * 3 + k + r)
    w = rng.standard_normal((n, k)).astype(np.float32)
    b = rng.standard_normal((n, max(r, 1))).astype(np.float32)[:, :r].copy()
    a = rng.standard_normal((max(r, 1), k)).astype(np.float32)[:r].copy()
    wd = gu.dev(w)
    cr.lora_add(wd, gu.dev(b), gu.dev(a), 0.37)
    gu.assert_equal(_f32_bits(gu.host(wd)), _f32_bits(oracle.lora_add(w, b, a, 0.37)),
                    "lora_add %dx%d rank %d" % (n, k, r))


def test_merge_lora_and_in_place(cr):
    """Dequantize + LoRA add + requantize: codes and scales bit-exact against
    the oracle, into fresh buffers and in place; zero strength keeps the codes."""
    import torch
    rng = np.random.default_rng(61)
    n, k, r = 300, 1536, 16
    w = (0.02 * rng.standard_normal((n, k))).astype(np.float32)
    b = (0.01 * rng.standard_normal((n, r))).astype(np.float32)
    a = (0.01 * rng.standard_normal((r, k))).astype(np.float32)
    oq, os_ = oracle.quantize_weight(w)
    mq, ms = oracle.merge_lora(oq, os_, b, a, 0.75)
    qd, sd = gu.dev(oq), gu.dev(os_)
    q2, s2 = cr.merge_lora(qd, sd, gu.dev(b), gu.dev(a), 0.75)
    gu.assert_equal(gu.host(q2), mq, "merge_lora q")
    gu.assert_equal(_f32_bits(gu.host(s2)), _f32_bits(ms), "merge_lora s")
    cr.merge_lora(qd, sd, gu.dev(b), gu.dev(a), 0.75, q_out=qd, s_out=sd)
    torch.cuda.synchronize()
    gu.assert_equal(gu.host(qd), mq, "merge_lora in place q")
    gu.assert_equal(_f32_bits(gu.host(sd)), _f32_bits(ms), "merge_lora in place s")
    q0, _ = cr.merge_lora(gu.dev(oq), gu.dev(os_), gu.dev(b), gu.dev(a), 0.0)
    gu.assert_equal(gu.host(q0), oq, "merge_lora zero strength")


def test_zero_size_calls(cr):
    import torch
    x = torch.empty((0, 256), dtype=torch.bfloat16, device="cuda")
    q, s = cr.rotate_quant_act(x)
    assert q.shape == (0, 256) and s.shape == (0,)
    qw = torch.zeros((4, 256), dtype=torch.int8, device="cuda")
    sw = torch.zeros((4,), dtype=torch.float32, device="cuda")
    y = cr.linear(x, qw, sw)
    assert y.shape == (0, 4)


def test_invalid_arguments_raise(cr):
    import torch
    x = torch.zeros((4, 300), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(cr.ConvRotError) as e:
        cr.rotate_quant_act(x)
    assert e.value.status == 2
    x = torch.zeros((4, 512), dtype=torch.bfloat16, device="cuda")
    qw = torch.zeros((8, 512), dtype=torch.int8, device="cuda")
    sw = torch.zeros((8,), dtype=torch.float32, device="cuda")
    ws = torch.zeros(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(cr.ConvRotError) as e:
        cr.linear(x, qw, sw, workspace=ws)
    assert e.value.status == 4


def test_deterministic_and_row_chunking(cr):
    """Same bytes on repeated calls, and splitting the tokens into chunks (the
    caller's activation-memory knob) changes nothing: rows are independent."""
    import torch
    d = workloads.make_linear("qkv", m=700)
    xd = gu.dev_bf16(d["x"])
    qw, sw = cr.quantize_weight(gu.dev(d["w"][:1000]))
    y1 = cr.linear(xd, qw, sw)
    y2 = cr.linear(xd, qw, sw)
    parts = [cr.linear(xd[a:b].contiguous(), qw, sw) for a, b in [(0, 1), (1, 300), (300, 700)]]
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    assert torch.equal(y1.view(torch.int16), torch.cat(parts).view(torch.int16))
