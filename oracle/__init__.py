"""CPU oracle for the ConvRot int8 quantized linear (test infrastructure).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  The product library never loads it and shares no code with it.

The arithmetic lives in ``convrot_oracle.c`` (plain scalar C, built with gcc
``-O2 -ffp-contract=off -fno-fast-math``); this module builds it on first use,
loads it with ctypes and wraps each function for numpy arrays.  Every wrapper
states the step it computes; the C file cites the passages of the pages each
step follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "convrot_oracle.c")
_LIB = os.path.join(_HERE, "libconvrot_oracle.so")

GROUP = 256

_CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
           "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra"]


def build(force: bool = False) -> str:
    """Compile the oracle with gcc into ``oracle/libconvrot_oracle.so``."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.run(["gcc", *_CFLAGS, _SRC, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        L.orc_set_threads.argtypes = [ctypes.c_int]
        L.orc_get_threads.restype = ctypes.c_int
        L.orc_bf16_to_f32_one.argtypes = [ctypes.c_uint16]
        L.orc_bf16_to_f32_one.restype = ctypes.c_float
        L.orc_f32_to_bf16_one.argtypes = [ctypes.c_float]
        L.orc_f32_to_bf16_one.restype = ctypes.c_uint16
        L.orc_bf16_to_f32.argtypes = [P, P, I64]
        L.orc_f32_to_bf16.argtypes = [P, P, I64]
        L.orc_fwht256.argtypes = [P]
        L.orc_rotate_rows.argtypes = [P, I64, I64]
        L.orc_quantize_row.argtypes = [P, I64, P, P]
        L.orc_quantize_rows.argtypes = [P, I64, I64, P, P]
        L.orc_quantize_weight.argtypes = [P, I64, I64, P, P]
        L.orc_quantize_weight.restype = ctypes.c_int
        L.orc_rotate_quant_act_rows.argtypes = [P, I64, P, I64, P, P]
        L.orc_rotate_quant_act_rows.restype = ctypes.c_int
        L.orc_gemm_s32.argtypes = [P, I64, P, I64, I64, P]
        L.orc_dequant_one.argtypes = [ctypes.c_int32, ctypes.c_float, ctypes.c_float]
        L.orc_dequant_one.restype = ctypes.c_float
        L.orc_dequant_bf16.argtypes = [P, I64, I64, P, P, P]
        L.orc_exp.argtypes = [ctypes.c_float]
        L.orc_exp.restype = ctypes.c_float
        L.orc_silu.argtypes = [ctypes.c_float]
        L.orc_silu.restype = ctypes.c_float
        L.orc_swiglu_bf16.argtypes = [P, I64, I64, P, P, P]
        L.orc_swiglu_ref.argtypes = [P, I64, I64, P, P, P, P]
        L.orc_swiglu_pairs_bf16.argtypes = [P, I64, I64, P]
        L.orc_swiglu_rotate_quant_rows.argtypes = [P, I64, P, I64, P, P]
        L.orc_swiglu_rotate_quant_rows.restype = ctypes.c_int
        L.orc_dequantize_weight.argtypes = [P, P, I64, I64, P]
        L.orc_lora_add.argtypes = [P, I64, I64, P, P, I64, ctypes.c_float]
        L.orc_attention_rows.argtypes = [P, P, I64, P, P, P, I64, I64, P, P]
        L.orc_mx_quantize_rows.argtypes = [P, I64, I64, P, P]
        L.orc_mx_decode.argtypes = [P, P, I64, I64, P]
        L.orc_mx_gemm.argtypes = [P, P, I64, P, P, I64, I64, P, P]
        _lib = L
    return _lib


def _p(a: np.ndarray) -> int:
    assert a.flags.c_contiguous
    return a.ctypes.data


def set_threads(n: int) -> None:
    lib().orc_set_threads(int(n))


def get_threads() -> int:
    return int(lib().orc_get_threads())


# ------------------------------------------------------------------ formats

def bf16_to_f32(h: np.ndarray) -> np.ndarray:
    """Exact widening of raw bf16 bits (uint16) to fp32."""
    h = np.ascontiguousarray(h, dtype=np.uint16)
    out = np.empty(h.shape, np.float32)
    lib().orc_bf16_to_f32(_p(h), _p(out), h.size)
    return out


def f32_to_bf16(f: np.ndarray) -> np.ndarray:
    """fp32 -> raw bf16 bits, round to nearest even."""
    f = np.ascontiguousarray(f, dtype=np.float32)
    out = np.empty(f.shape, np.uint16)
    lib().orc_f32_to_bf16(_p(f), _p(out), f.size)
    return out


# ------------------------------------------------------------------ rotation

def fwht256(v: np.ndarray) -> np.ndarray:
    """Normalized 256-point Walsh-Hadamard transform of one fp32 vector."""
    v = np.array(v, dtype=np.float32, copy=True).reshape(GROUP)
    lib().orc_fwht256(_p(v))
    return v


def rotate_rows(x: np.ndarray) -> np.ndarray:
    """Group-wise rotation of every row of an fp32 [rows, k] array."""
    x = np.array(x, dtype=np.float32, copy=True, order="C")
    rows, k = x.shape
    assert k % GROUP == 0
    lib().orc_rotate_rows(_p(x), rows, k)
    return x


# ------------------------------------------------------------------ quantizer

def quantize_rows(v: np.ndarray):
    """Per-row symmetric int8 of fp32 rows as given (no rotation)."""
    v = np.ascontiguousarray(v, dtype=np.float32)
    rows, k = v.shape
    q = np.empty((rows, k), np.int8)
    s = np.empty(rows, np.float32)
    lib().orc_quantize_rows(_p(v), rows, k, _p(q), _p(s))
    return q, s


def quantize_weight(w: np.ndarray):
    """Rotate each row of fp32 W [n, k] along k and quantize it per row."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    n, k = w.shape
    q = np.empty((n, k), np.int8)
    s = np.empty(n, np.float32)
    rc = lib().orc_quantize_weight(_p(w), n, k, _p(q), _p(s))
    if rc != 0:
        raise ValueError("oracle quantize_weight failed (k=%d)" % k)
    return q, s


def rotate_quant_act(x_bf16: np.ndarray, rows: np.ndarray | None = None):
    """Widen bf16 x [m, k], rotate along k, quantize per token.

    With ``rows`` given, only those rows are processed (in that order)."""
    x_bf16 = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    m, k = x_bf16.shape
    if rows is None:
        nrows, rp = m, None
    else:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        assert rows.size == 0 or (rows.min() >= 0 and rows.max() < m)
        nrows, rp = rows.size, _p(rows)
    q = np.empty((nrows, k), np.int8)
    s = np.empty(nrows, np.float32)
    rc = lib().orc_rotate_quant_act_rows(_p(x_bf16), k, rp, nrows, _p(q), _p(s))
    if rc != 0:
        raise ValueError("oracle rotate_quant_act failed (k=%d)" % k)
    return q, s


# ------------------------------------------------------------------ contraction

def gemm_s32(qx: np.ndarray, qw: np.ndarray) -> np.ndarray:
    """int32 acc[j, c] = sum_k qx[j, k] * qw[c, k] (triple loop)."""
    qx = np.ascontiguousarray(qx, dtype=np.int8)
    qw = np.ascontiguousarray(qw, dtype=np.int8)
    nrows, k = qx.shape
    n, k2 = qw.shape
    assert k == k2
    acc = np.empty((nrows, n), np.int32)
    lib().orc_gemm_s32(_p(qx), nrows, _p(qw), n, k, _p(acc))
    return acc


# ------------------------------------------------------------------ epilogues

def dequant_bf16(acc: np.ndarray, s_x: np.ndarray, s_w: np.ndarray) -> np.ndarray:
    """bf16(((float)acc * s_x[row]) * s_w[col])."""
    acc = np.ascontiguousarray(acc, dtype=np.int32)
    s_x = np.ascontiguousarray(s_x, dtype=np.float32)
    s_w = np.ascontiguousarray(s_w, dtype=np.float32)
    nrows, n = acc.shape
    assert s_x.size == nrows and s_w.size == n
    y = np.empty((nrows, n), np.uint16)
    lib().orc_dequant_bf16(_p(acc), nrows, n, _p(s_x), _p(s_w), _p(y))
    return y


def dequant_f32(acc: np.ndarray, s_x: np.ndarray, s_w: np.ndarray) -> np.ndarray:
    """The fp32 value before bf16 rounding, element by element (small inputs)."""
    L = lib()
    out = np.empty(acc.shape, np.float32)
    for j in range(acc.shape[0]):
        for c in range(acc.shape[1]):
            out[j, c] = L.orc_dequant_one(int(acc[j, c]), float(s_x[j]), float(s_w[c]))
    return out


def exp(x: float) -> float:
    return float(lib().orc_exp(float(x)))


def silu(g: float) -> float:
    return float(lib().orc_silu(float(g)))


def swiglu_bf16(acc: np.ndarray, s_x: np.ndarray, s_w: np.ndarray) -> np.ndarray:
    """bf16(silu(g) * u), g from columns [0, i), u from columns [i, 2i)."""
    acc = np.ascontiguousarray(acc, dtype=np.int32)
    s_x = np.ascontiguousarray(s_x, dtype=np.float32)
    s_w = np.ascontiguousarray(s_w, dtype=np.float32)
    nrows, n2 = acc.shape
    assert n2 % 2 == 0 and s_w.size == n2 and s_x.size == nrows
    i = n2 // 2
    y = np.empty((nrows, i), np.uint16)
    lib().orc_swiglu_bf16(_p(acc), nrows, i, _p(s_x), _p(s_w), _p(y))
    return y


def swiglu_ref(acc: np.ndarray, s_x: np.ndarray, s_w: np.ndarray):
    """The exact fused-epilogue value in fp64, ref = silu(g) * u with g, u the
    fp32 dequantized gate and up values (columns [0, i) and [i, 2i)); returns
    (ref [m, i] float64, |g u| [m, i] float64)."""
    acc = np.ascontiguousarray(acc, dtype=np.int32)
    s_x = np.ascontiguousarray(s_x, dtype=np.float32)
    s_w = np.ascontiguousarray(s_w, dtype=np.float32)
    nrows, n2 = acc.shape
    assert n2 % 2 == 0 and s_w.size == n2 and s_x.size == nrows
    i = n2 // 2
    ref = np.empty((nrows, i), np.float64)
    mag = np.empty((nrows, i), np.float64)
    lib().orc_swiglu_ref(_p(acc), nrows, i, _p(s_x), _p(s_w), _p(ref), _p(mag))
    return ref, mag


def swiglu_pairs_bf16(gu_bf16: np.ndarray) -> np.ndarray:
    """h = bf16(silu(g) * u) from fc1's bf16 output [m, 2i]: g = columns
    [0, i), u = columns [i, 2i), both widened exactly."""
    gu_bf16 = np.ascontiguousarray(gu_bf16, dtype=np.uint16)
    m, n2 = gu_bf16.shape
    assert n2 % 2 == 0
    i = n2 // 2
    h = np.empty((m, i), np.uint16)
    lib().orc_swiglu_pairs_bf16(_p(gu_bf16), m, i, _p(h))
    return h


def swiglu_rotate_quant_act(gu_bf16: np.ndarray, rows: np.ndarray | None = None):
    """SwiGLU on fc1's bf16 output [m, 2i], then rotate along i and quantize
    per token: the down projection's codes and scales with SwiGLU moved out
    of fc1's epilogue.  With ``rows``, only those rows (in that order)."""
    gu_bf16 = np.ascontiguousarray(gu_bf16, dtype=np.uint16)
    m, n2 = gu_bf16.shape
    assert n2 % 2 == 0
    i = n2 // 2
    if rows is None:
        nrows, rp = m, None
    else:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        assert rows.size == 0 or (rows.min() >= 0 and rows.max() < m)
        nrows, rp = rows.size, _p(rows)
    q = np.empty((nrows, i), np.int8)
    s = np.empty(nrows, np.float32)
    rc = lib().orc_swiglu_rotate_quant_rows(_p(gu_bf16), i, rp, nrows, _p(q), _p(s))
    if rc != 0:
        raise ValueError("oracle swiglu_rotate_quant_act failed (i=%d)" % i)
    return q, s


def dequantize_weight(q_w: np.ndarray, s_w: np.ndarray) -> np.ndarray:
    """fp32 W [n, k] = (q . s) . H/16 per row: the unrotated weights."""
    q_w = np.ascontiguousarray(q_w, dtype=np.int8)
    s_w = np.ascontiguousarray(s_w, dtype=np.float32)
    n, k = q_w.shape
    assert s_w.size == n and k % 256 == 0
    w = np.empty((n, k), np.float32)
    lib().orc_dequantize_weight(_p(q_w), _p(s_w), n, k, _p(w))
    return w


def lora_add(w: np.ndarray, b: np.ndarray, a: np.ndarray, scale: float) -> np.ndarray:
    """W + scale * (B . A) with the fp32 order of the definition (returns a copy)."""
    w = np.array(w, dtype=np.float32, copy=True, order="C")
    b = np.ascontiguousarray(b, dtype=np.float32)
    a = np.ascontiguousarray(a, dtype=np.float32)
    n, k = w.shape
    rank = b.shape[1]
    assert b.shape == (n, rank) and a.shape == (rank, k)
    lib().orc_lora_add(_p(w), n, k, _p(b), _p(a), rank, float(scale))
    return w


def merge_lora(q_w, s_w, b, a, scale):
    """Dequantize, add the low-rank delta, requantize: new (q_w, s_w)."""
    return quantize_weight(lora_add(dequantize_weight(q_w, s_w), b, a, scale))


# ------------------------------------------------------------------ compositions

def linear_rows(x_bf16, q_w, s_w, rows=None):
    """y rows of the ConvRot linear: rotate+quantize x, int32 GEMM, dequant."""
    qx, sx = rotate_quant_act(x_bf16, rows)
    acc = gemm_s32(qx, q_w)
    return dequant_bf16(acc, sx, s_w)


def linear_swiglu_rows(x_bf16, q_w, s_w, rows=None):
    """y rows of the ConvRot fc1 with fused SwiGLU (q_w holds 2i rows), with
    the oracle's fixed fp32 exponential, rounded to bf16."""
    qx, sx = rotate_quant_act(x_bf16, rows)
    acc = gemm_s32(qx, q_w)
    return swiglu_bf16(acc, sx, s_w)


def linear_swiglu_ref_rows(x_bf16, q_w, s_w, rows=None):
    """The exact fused fc1 value for the given rows: (ref, |g u|), see swiglu_ref."""
    qx, sx = rotate_quant_act(x_bf16, rows)
    acc = gemm_s32(qx, q_w)
    return swiglu_ref(acc, sx, s_w)


# ------------------------------------------------------------------ attention

def attention_quant(x_bf16: np.ndarray):
    """Per token-head int8 quantization of Q or K: raw bf16 [rows, d] -> codes
    [rows, d], scales [rows] (the per-row quantizer, no rotation)."""
    return quantize_rows(bf16_to_f32(x_bf16))


def to_fp16(x_bf16: np.ndarray) -> np.ndarray:
    """bf16 bits -> fp16 values, round to nearest even (numpy's cast)."""
    return bf16_to_f32(x_bf16).astype(np.float16)


def attention_rows(qc, sq, kc, sk, v_f16):
    """One head: O [nq, d] and the rounding scale sum p|v|/sum p, both fp64,
    for query codes qc [nq, d] / scales sq against all keys kc [s, d] / sk and
    fp16 values v_f16 [s, d]."""
    qc = np.ascontiguousarray(qc, dtype=np.int8)
    kc = np.ascontiguousarray(kc, dtype=np.int8)
    sq = np.ascontiguousarray(sq, dtype=np.float32)
    sk = np.ascontiguousarray(sk, dtype=np.float32)
    v = np.ascontiguousarray(np.asarray(v_f16, dtype=np.float16), dtype=np.float64)
    nq, d = qc.shape
    s = kc.shape[0]
    assert kc.shape == (s, d) and v.shape == (s, d) and sq.size == nq and sk.size == s
    out = np.empty((nq, d), np.float64)
    absw = np.empty((nq, d), np.float64)
    lib().orc_attention_rows(_p(qc), _p(sq), nq, _p(kc), _p(sk), _p(v), s, d, _p(out), _p(absw))
    return out, absw


def split_heads(x_bf16: np.ndarray, heads: int) -> np.ndarray:
    """[s, heads * d] -> [heads, s, d] (a view change, no arithmetic)."""
    s, w = x_bf16.shape
    return np.ascontiguousarray(x_bf16.reshape(s, heads, w // heads).transpose(1, 0, 2))


def attention(q_bf16, k_bf16, v_bf16, heads: int, rows=None):
    """Full attention of [s, heads * d] bf16 Q, K, V (raw bits): per head,
    quantize Q and K, convert V to fp16, softmax-attend.  Returns O [heads,
    nq, d] fp64, absw likewise, and the codes/scales (qc, sq, kc, sk) per head.
    ``rows`` restricts the queries (all keys are always used)."""
    qh, kh, vh = (split_heads(t, heads) for t in (q_bf16, k_bf16, v_bf16))
    outs, absws, qcs, sqs, kcs, sks = [], [], [], [], [], []
    for h in range(heads):
        qc, sq = attention_quant(qh[h])
        kc, sk = attention_quant(kh[h])
        sel = slice(None) if rows is None else np.asarray(rows, np.int64)
        o, a = attention_rows(qc[sel], sq[sel], kc, sk, to_fp16(vh[h]))
        outs.append(o); absws.append(a)
        qcs.append(qc); sqs.append(sq); kcs.append(kc); sks.append(sk)
    return (np.stack(outs), np.stack(absws),
            (np.stack(qcs), np.stack(sqs), np.stack(kcs), np.stack(sks)))


# ------------------------------------------------------------------ MXFP4

def mx_quantize(v: np.ndarray):
    """fp32 rows [r, k] (k % 32 == 0) -> (FP4 E2M1 codes packed two per byte
    [r, k/2] uint8, E8M0 block scales [r, k/32] uint8)."""
    v = np.ascontiguousarray(v, dtype=np.float32)
    r, k = v.shape
    assert k % 32 == 0
    codes = np.zeros((r, k // 2), np.uint8)
    scales = np.zeros((r, k // 32), np.uint8)
    lib().orc_mx_quantize_rows(_p(v), r, k, _p(codes), _p(scales))
    return codes, scales


def mx_quantize_act(x_bf16: np.ndarray):
    """MXFP4 of bf16 activation rows (widened exactly)."""
    return mx_quantize(bf16_to_f32(x_bf16))


def mx_decode(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    r, k2 = codes.shape
    out = np.empty((r, 2 * k2), np.float64)
    lib().orc_mx_decode(_p(codes), _p(scales), r, 2 * k2, _p(out))
    return out


def mx_gemm(ac, asc, bc, bsc):
    """fp64 y = A B^T of two MXFP4 matrices, and sum |a b| per output."""
    ac = np.ascontiguousarray(ac, dtype=np.uint8)
    asc = np.ascontiguousarray(asc, dtype=np.uint8)
    bc = np.ascontiguousarray(bc, dtype=np.uint8)
    bsc = np.ascontiguousarray(bsc, dtype=np.uint8)
    m, k2 = ac.shape
    n = bc.shape[0]
    assert bc.shape[1] == k2 and asc.shape == (m, k2 // 16) and bsc.shape == (n, k2 // 16)
    y = np.empty((m, n), np.float64)
    absacc = np.empty((m, n), np.float64)
    lib().orc_mx_gemm(_p(ac), _p(asc), m, _p(bc), _p(bsc), n, 2 * k2, _p(y), _p(absacc))
    return y, absacc


def mx_quantize_rotated(v: np.ndarray):
    """MXFP4 of fp32 rows after the orthonormal Hadamard-256 rotation of the
    int8 ConvRot path (the pinned rotation, then the pinned MX quantizer)."""
    return mx_quantize(rotate_rows(np.ascontiguousarray(v, dtype=np.float32)))


def mx_quantize_act_rotated(x_bf16: np.ndarray):
    return mx_quantize_rotated(bf16_to_f32(x_bf16))
