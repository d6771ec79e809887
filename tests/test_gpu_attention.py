"""GPU parity of the int8 Q.K^T / fp16 P.V attention against the CPU oracle.

Bit-exact: the Q and K codes and scales and the fp16 V layout in the
workspace.  Outputs: within the rounding that the kernel adds to the fp64
definition -- fp16 probabilities (relative 2^-11), fp32 logits and sums
(relative ~1e-4 over 32k keys) and the bf16 store (relative 2^-9) -- bounded
per element by 2^-8 |O| + 2^-9 sum_j p_j |v_j| / sum_j p_j, with the second
term taken from the oracle."""
import numpy as np
import pytest

import oracle
import workloads
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

D = 128


@pytest.fixture(scope="module")
def cr():
    import rotation_quantized_dit_amd as cr
    cr.load_library()
    return cr


def _f32_bits(a):
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


def vt_pos(j):
    """Position of key j inside its 32-key block of the V region (convrot.h)."""
    j = np.asarray(j)
    return (j & ~12) | ((j & 4) << 1) | ((j & 8) >> 1)


def thirds(qkv_bits, heads):
    w = heads * D
    return qkv_bits[:, :w], qkv_bits[:, w:2 * w], qkv_bits[:, 2 * w:]


def run_gpu(cr, qkv_bits, heads, strided=True):
    """Attention on the GPU; returns (out bits [s, heads*128], workspace bytes)."""
    import torch
    qkv = gu.dev_bf16(qkv_bits)
    w = heads * D
    if strided:
        q, k, v = qkv[:, :w], qkv[:, w:2 * w], qkv[:, 2 * w:]
    else:
        q, k, v = (qkv[:, i * w:(i + 1) * w].contiguous() for i in range(3))
    s = qkv_bits.shape[0]
    ws = cr.attention_prep(q, k, v, heads)
    out = cr.attention_prepared(ws, s, heads)
    torch.cuda.synchronize()
    return gu.host_bf16(out), gu.host(ws)


def check_workspace(ws, qkv_bits, heads, ref_codes, what):
    """Q/K codes and scales bit for bit; V region equal to fp16(V) in the
    documented blocked, transposed, permuted layout."""
    from rotation_quantized_dit_amd import attention_workspace
    s = qkv_bits.shape[0]
    s_pad = (s + 63) // 64 * 64
    nbytes, off = attention_workspace(s, heads)
    assert ws.size >= nbytes
    qc, sq, kc, sk = ref_codes
    g_qc = ws[off[0]:off[0] + heads * s * D].view(np.int8).reshape(heads, s, D)
    g_sq = ws[off[1]:off[1] + heads * s * 4].view(np.float32).reshape(heads, s)
    g_kc = ws[off[2]:off[2] + heads * s_pad * D].view(np.int8).reshape(heads, s_pad, D)
    g_sk = ws[off[3]:off[3] + heads * s_pad * 4].view(np.float32).reshape(heads, s_pad)
    g_v = ws[off[4]:off[4] + heads * s_pad * D * 2].view(np.float16).reshape(heads, s_pad // 64, D, 64)
    gu.assert_equal(g_qc, qc, what + " q codes")
    gu.assert_equal(_f32_bits(g_sq), _f32_bits(sq), what + " q scales")
    gu.assert_equal(g_kc[:, :s], kc, what + " k codes")
    gu.assert_equal(g_sk[:, :s].view(np.uint32), _f32_bits(sk), what + " k scales")
    assert not g_kc[:, s:].any() and not g_sk[:, s:].any(), what + " key padding"
    _, _, v = thirds(qkv_bits, heads)
    v16 = np.zeros((heads, s_pad, D), np.float16)
    v16[:, :s] = oracle.to_fp16(oracle.split_heads(v, heads).reshape(-1, D)).reshape(heads, s, D)
    blocks = v16.reshape(heads, s_pad // 64, 64, D).transpose(0, 1, 3, 2)   # [h, b, d, j]
    j = np.arange(64)
    want = np.empty_like(blocks)
    want[..., (j & ~31) | vt_pos(j & 31)] = blocks
    gu.assert_equal(g_v.view(np.uint16), want.view(np.uint16), what + " V layout")


def assert_attn_close(out_bits, ref, absw, heads, rows, what):
    """out_bits [s, heads*128] (GPU) at ``rows`` against the oracle's [heads,
    len(rows), 128] fp64 output and rounding scale."""
    g = gu.bf16_f64(out_bits[rows]).reshape(len(rows), heads, D).transpose(1, 0, 2)
    err = np.abs(g - ref)
    tol = 2.0 ** -8 * np.abs(ref) + 2.0 ** -9 * absw
    bad = err > tol
    if bad.any():
        i = np.unravel_index(np.argmax(err / np.maximum(tol, 1e-300)), err.shape)
        raise AssertionError("%s: %d of %d outside the bound; worst at %s: gpu %r ref %r tol %r" % (
            what, int(bad.sum()), bad.size, i, g[i], ref[i], tol[i]))
    assert np.all(np.isfinite(g)), what
    print("%s: max err / bound = %.3f" % (what, float((err / np.maximum(tol, 1e-300)).max())), flush=True)


CASES = [
    # s, heads, qk_std, k_outlier
    (1, 1, 2.0, 0.0),
    (2, 2, 2.0, 0.0),
    (63, 1, 2.0, 0.0),
    (64, 2, 2.0, 0.0),
    (65, 1, 2.0, 0.0),
    (255, 1, 1.0, 0.0),
    (256, 1, 2.0, 0.0),
    (257, 2, 2.0, 0.0),
    (700, 3, 4.0, 0.0),
    (1000, 2, 2.0, 30.0),
    (2048, 1, 1.0, 0.0),
    (3001, 2, 2.0, 0.0),
]


@pytest.mark.parametrize("s,heads,qk_std,k_outlier", CASES)
def test_attention_parity(cr, s, heads, qk_std, k_outlier):
    a = workloads.make_attention(s, heads, seed=100 + s, qk_std=qk_std, k_outlier=k_outlier)
    what = "attn s=%d h=%d std=%g outl=%g" % (s, heads, qk_std, k_outlier)
    print(what, flush=True)
    out, ws = run_gpu(cr, a["qkv"], heads)
    q, k, v = thirds(a["qkv"], heads)
    ref, absw, codes = oracle.attention(q, k, v, heads)
    check_workspace(ws, a["qkv"], heads, codes, what)
    assert_attn_close(out, ref, absw, heads, np.arange(s), what)


def test_attention_strided_equals_contiguous_and_is_deterministic(cr):
    """Column slices of one QKV matrix give the same bytes as contiguous
    copies, the one-call entry point the same as prep + prepared, and two
    calls the same bytes."""
    import torch
    s, heads = 777, 2
    a = workloads.make_attention(s, heads, seed=7)
    o1, _ = run_gpu(cr, a["qkv"], heads, strided=True)
    o2, _ = run_gpu(cr, a["qkv"], heads, strided=False)
    qkv = gu.dev_bf16(a["qkv"])
    w = heads * D
    o3 = cr.attention(qkv[:, :w], qkv[:, w:2 * w], qkv[:, 2 * w:], heads)
    torch.cuda.synchronize()
    gu.assert_equal(o1, o2, "strided vs contiguous")
    gu.assert_equal(o1, gu.host_bf16(o3), "one call vs two")


def test_attention_degenerate_rows(cr):
    """All-zero query rows (s_q = 0) and a head whose keys are all zero
    (s_k = 0): every logit of those rows is 0, so the output is the plain mean
    of V; the oracle agrees and nothing is NaN."""
    s, heads = 200, 2
    a = workloads.make_attention(s, heads, seed=8)
    qkv = a["qkv"].copy()
    qkv[::7, :heads * D] = 0                       # some zero queries, both heads
    qkv[:, heads * D:heads * D + D] = 0            # head 0: all keys zero
    out, ws = run_gpu(cr, qkv, heads)
    q, k, v = thirds(qkv, heads)
    ref, absw, codes = oracle.attention(q, k, v, heads)
    check_workspace(ws, qkv, heads, codes, "degenerate")
    assert_attn_close(out, ref, absw, heads, np.arange(s), "degenerate")
    mean0 = oracle.to_fp16(oracle.split_heads(v, heads)[0]).astype(np.float64).mean(axis=0)
    g0 = gu.bf16_f64(out[:, :D])
    assert np.allclose(g0, mean0, rtol=2 ** -7, atol=2 ** -9 * np.abs(mean0).max())


def test_attention_validation(cr):
    import torch
    s, heads = 64, 1
    x = torch.zeros(s, 3 * heads * D, dtype=torch.bfloat16, device="cuda")
    w = heads * D
    with pytest.raises(ValueError):
        cr.attention(x[:, :w], x[:, w:2 * w], x[:, 2 * w:], heads=2)
    ws = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(cr.ConvRotError):
        cr.attention(x[:, :w], x[:, w:2 * w], x[:, 2 * w:], heads, workspace=ws)


def test_attention_full_size(cr):
    """The benchmark's configuration, 32256 tokens x 42 heads of 128, one call
    of each entry point: Q/K codes and scales of every token and head bit for
    bit, the V layout of every head, and the output of sampled queries (first,
    last, 24 seeded) of heads 0, 21 and 41 against all 32256 keys."""
    import torch
    s, heads = workloads.VIDEO_TOKENS, workloads.ATTN_HEADS
    print("attention full size: generating %d x %d" % (s, 3 * heads * D), flush=True)
    a = workloads.make_attention()
    qkv = gu.dev_bf16(a["qkv"])
    w = heads * D
    ws = cr.attention_prep(qkv[:, :w], qkv[:, w:2 * w], qkv[:, 2 * w:], heads)
    out = cr.attention_prepared(ws, s, heads)
    torch.cuda.synchronize()
    out_h, ws_h = gu.host_bf16(out), gu.host(ws)
    del qkv, ws, out
    print("attention full size: oracle codes", flush=True)
    q, k, v = thirds(a["qkv"], heads)
    qh, kh = oracle.split_heads(q, heads), oracle.split_heads(k, heads)
    qc, sq = oracle.attention_quant(qh.reshape(-1, D))
    kc, sk = oracle.attention_quant(kh.reshape(-1, D))
    codes = (qc.reshape(heads, s, D), sq.reshape(heads, s), kc.reshape(heads, s, D), sk.reshape(heads, s))
    check_workspace(ws_h, a["qkv"], heads, codes, "full size")
    rows = workloads.sample_rows(s, seed=workloads.ATTN_SEED, count=24)
    vh = oracle.split_heads(v, heads)
    for h in (0, 21, 41):
        print("attention full size: oracle head %d, %d queries" % (h, rows.size), flush=True)
        ref, absw = oracle.attention_rows(codes[0][h][rows], codes[1][h][rows], codes[2][h], codes[3][h],
                                          oracle.to_fp16(vh[h]))
        sub = out_h[:, h * D:(h + 1) * D]
        assert_attn_close(sub, ref[None], absw[None], 1, rows, "full size head %d" % h)
