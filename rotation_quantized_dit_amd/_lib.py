"""ctypes binding of libconvrot.so (the C ABI in include/convrot.h).

Argument marshalling only: shapes, dtypes and devices are checked, outputs are
allocated with torch (unless passed in), and torch's current HIP stream is
handed to the library.  Every step of the computation runs in the library's
HIP kernels; there is no fallback of any kind.  If the library is not built
the first call raises.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libconvrot.so")

GROUP = 256
MAX_K = 133120

OK, ERR_NULL, ERR_SHAPE, ERR_ALIGN, ERR_WORKSPACE, ERR_LAUNCH, ERR_SCRATCH = range(7)

# the fixed device array convrot_linear_noalloc uses as its workspace
NOALLOC_SCRATCH_BYTES = 64 << 20

SYMBOLS = (
    "convrot_quantize_weight", "convrot_rotate_quant_act", "convrot_workspace_bytes",
    "convrot_linear", "convrot_linear_swiglu", "convrot_gemm_dequant", "convrot_gemm_swiglu",
    "convrot_gemm_s32", "convrot_swiglu_rotate_quant_act", "convrot_dequantize_weight",
    "convrot_lora_add", "convrot_merge_workspace_bytes", "convrot_merge_lora", "convrot_status_string",
    "convrot_attention_workspace", "convrot_attention_prep", "convrot_attention_prepared",
    "convrot_attention", "convrot_mx_quantize_act", "convrot_mx_quantize_weight", "convrot_mx_gemm",
    "convrot_mx_workspace_bytes", "convrot_mx_linear", "convrot_linear_noalloc",
)

ATTN_HEAD_DIM = 128


class ConvRotError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__("%s failed with status %d: %s" % (fn, status, msg))
        self.status = status


_lock = threading.Lock()
_lib = None


def load_library() -> ctypes.CDLL:
    """Load libconvrot.so (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libconvrot.so is not built (%s); run "
                               "`python -m rotation_quantized_dit_amd.build`" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        P, I64, SZ, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t, ctypes.c_int
        sig = {
            "convrot_quantize_weight": ([P, I64, I64, P, P, P], I),
            "convrot_rotate_quant_act": ([P, I64, I64, P, P, P], I),
            "convrot_swiglu_rotate_quant_act": ([P, I64, I64, P, P, P], I),
            "convrot_workspace_bytes": ([I64, I64], SZ),
            "convrot_linear": ([P, I64, I64, P, P, I64, P, P, SZ, P], I),
            "convrot_linear_swiglu": ([P, I64, I64, P, P, I64, P, P, SZ, P], I),
            "convrot_linear_noalloc": ([P, I64, I64, P, P, I64, P, P], I),
            "convrot_gemm_dequant": ([P, P, P, P, I64, I64, I64, P, P], I),
            "convrot_gemm_swiglu": ([P, P, P, P, I64, I64, I64, P, P], I),
            "convrot_gemm_s32": ([P, P, I64, I64, I64, P, P], I),
            "convrot_dequantize_weight": ([P, P, I64, I64, P, P], I),
            "convrot_lora_add": ([P, I64, I64, P, P, I64, ctypes.c_float, P], I),
            "convrot_merge_workspace_bytes": ([I64, I64], SZ),
            "convrot_merge_lora": ([P, P, I64, I64, P, P, I64, ctypes.c_float, P, P, P, SZ, P], I),
            "convrot_status_string": ([I], ctypes.c_char_p),
            "convrot_attention_workspace": ([I64, I64, I64, P], SZ),
            "convrot_attention_prep": ([P, P, P, I64, I64, I64, I64, P, SZ, P], I),
            "convrot_attention_prepared": ([P, SZ, I64, I64, I64, P, I64, P], I),
            "convrot_attention": ([P, P, P, I64, I64, I64, I64, P, I64, P, SZ, P], I),
            "convrot_mx_quantize_act": ([P, I64, I64, I, P, P, P], I),
            "convrot_mx_quantize_weight": ([P, I64, I64, I, P, P, P], I),
            "convrot_mx_gemm": ([P, P, P, P, I64, I64, I64, P, P], I),
            "convrot_mx_workspace_bytes": ([I64, I64], SZ),
            "convrot_mx_linear": ([P, I64, I64, I, P, P, I64, P, P, SZ, P], I),
        }
        for name, (args, res) in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        _lib = L
        return L


def status_string(status: int) -> str:
    return load_library().convrot_status_string(int(status)).decode()


def workspace_bytes(m: int, k: int) -> int:
    return int(load_library().convrot_workspace_bytes(int(m), int(k)))


def _check(fn: str, st: int) -> None:
    if st != OK:
        raise ConvRotError(fn, st, status_string(st))


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _dev(t: torch.Tensor, name: str, dtype: torch.dtype, ndim: int) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if not t.is_cuda:
        raise ValueError("%s must be a GPU tensor (got %s)" % (name, t.device))
    if t.device.index != torch.cuda.current_device():
        raise ValueError("%s is on %s, but the library launches on the current device cuda:%d"
                         % (name, t.device, torch.cuda.current_device()))
    if t.dtype != dtype:
        raise TypeError("%s must be %s (got %s)" % (name, dtype, t.dtype))
    if t.dim() != ndim:
        raise ValueError("%s must have %d dims (got %s)" % (name, ndim, tuple(t.shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _out(out, shape, dtype, like: torch.Tensor, name: str) -> torch.Tensor:
    if out is None:
        return torch.empty(shape, dtype=dtype, device=like.device)
    _dev(out, name, dtype, len(shape))
    if tuple(out.shape) != tuple(shape):
        raise ValueError("%s must have shape %s (got %s)" % (name, tuple(shape), tuple(out.shape)))
    return out


def quantize_weight(w: torch.Tensor, q_w=None, s_w=None):
    """fp32 W [n, k] -> (int8 codes [n, k], fp32 per-row scales [n]) of the rotated rows."""
    _dev(w, "w", torch.float32, 2)
    n, k = w.shape
    q_w = _out(q_w, (n, k), torch.int8, w, "q_w")
    s_w = _out(s_w, (n,), torch.float32, w, "s_w")
    _check("convrot_quantize_weight", load_library().convrot_quantize_weight(
        w.data_ptr(), n, k, q_w.data_ptr(), s_w.data_ptr(), _stream()))
    return q_w, s_w


def rotate_quant_act(x: torch.Tensor, q_x=None, s_x=None):
    """bf16 x [m, k] -> (int8 codes [m, k], fp32 per-token scales [m])."""
    _dev(x, "x", torch.bfloat16, 2)
    m, k = x.shape
    q_x = _out(q_x, (m, k), torch.int8, x, "q_x")
    s_x = _out(s_x, (m,), torch.float32, x, "s_x")
    _check("convrot_rotate_quant_act", load_library().convrot_rotate_quant_act(
        x.data_ptr(), m, k, q_x.data_ptr(), s_x.data_ptr(), _stream()))
    return q_x, s_x


def swiglu_rotate_quant_act(gu: torch.Tensor, q_h=None, s_h=None):
    """fc1's bf16 output gu [m, 2i] (gate columns [0, i), up [i, 2i)) ->
    codes [m, i] and per-token scales [m] of h = bf16(silu(gate) * up),
    rotated and quantized as rotate_quant_act does."""
    _dev(gu, "gu", torch.bfloat16, 2)
    m, n2 = gu.shape
    if n2 % 2:
        raise ValueError("gu must have an even number of columns (got %d)" % n2)
    i = n2 // 2
    q_h = _out(q_h, (m, i), torch.int8, gu, "q_h")
    s_h = _out(s_h, (m,), torch.float32, gu, "s_h")
    _check("convrot_swiglu_rotate_quant_act", load_library().convrot_swiglu_rotate_quant_act(
        gu.data_ptr(), m, i, q_h.data_ptr(), s_h.data_ptr(), _stream()))
    return q_h, s_h


def _ws_check(workspace) -> None:
    """A caller's workspace: a contiguous uint8 tensor on the current GPU."""
    if not (isinstance(workspace, torch.Tensor) and workspace.is_cuda and workspace.dtype == torch.uint8
            and workspace.is_contiguous()):
        raise TypeError("workspace must be a contiguous uint8 GPU tensor")
    if workspace.device.index != torch.cuda.current_device():
        raise ValueError("workspace is on %s, but the library launches on the current device cuda:%d"
                         % (workspace.device, torch.cuda.current_device()))


def _workspace(workspace, m, k, like):
    need = max(workspace_bytes(m, k), 16)
    if workspace is None:
        return torch.empty(need, dtype=torch.uint8, device=like.device)
    _ws_check(workspace)
    return workspace


def linear(x: torch.Tensor, q_w: torch.Tensor, s_w: torch.Tensor, out=None, workspace=None):
    """ConvRot int8 linear: bf16 x [m, k] -> bf16 y [m, n]."""
    _dev(x, "x", torch.bfloat16, 2)
    _dev(q_w, "q_w", torch.int8, 2)
    _dev(s_w, "s_w", torch.float32, 1)
    m, k = x.shape
    n = q_w.shape[0]
    if q_w.shape[1] != k or s_w.shape[0] != n:
        raise ValueError("shape mismatch: x %s, q_w %s, s_w %s" % (tuple(x.shape), tuple(q_w.shape), tuple(s_w.shape)))
    y = _out(out, (m, n), torch.bfloat16, x, "out")
    ws = _workspace(workspace, m, k, x)
    _check("convrot_linear", load_library().convrot_linear(
        x.data_ptr(), m, k, q_w.data_ptr(), s_w.data_ptr(), n, y.data_ptr(), ws.data_ptr(),
        ws.numel(), _stream()))
    return y


def linear_noalloc(x: torch.Tensor, q_w: torch.Tensor, s_w: torch.Tensor, out=None):
    """convrot_linear_noalloc: the ConvRot linear with the library's own device
    scratch as its workspace (m k + 4 m <= NOALLOC_SCRATCH_BYTES); the library
    allocates nothing (out is allocated here unless passed)."""
    _dev(x, "x", torch.bfloat16, 2)
    _dev(q_w, "q_w", torch.int8, 2)
    _dev(s_w, "s_w", torch.float32, 1)
    m, k = x.shape
    n = q_w.shape[0]
    if q_w.shape[1] != k or s_w.shape[0] != n:
        raise ValueError("shape mismatch: x %s, q_w %s, s_w %s" % (tuple(x.shape), tuple(q_w.shape), tuple(s_w.shape)))
    y = _out(out, (m, n), torch.bfloat16, x, "out")
    _check("convrot_linear_noalloc", load_library().convrot_linear_noalloc(
        x.data_ptr(), m, k, q_w.data_ptr(), s_w.data_ptr(), n, y.data_ptr(), _stream()))
    return y


def linear_swiglu(x: torch.Tensor, q_w: torch.Tensor, s_w: torch.Tensor, out=None, workspace=None):
    """fc1 ConvRot linear with fused SwiGLU: q_w has 2i rows (gate then up); y is [m, i]."""
    _dev(x, "x", torch.bfloat16, 2)
    _dev(q_w, "q_w", torch.int8, 2)
    _dev(s_w, "s_w", torch.float32, 1)
    m, k = x.shape
    n2 = q_w.shape[0]
    if n2 % 2 or q_w.shape[1] != k or s_w.shape[0] != n2:
        raise ValueError("shape mismatch: x %s, q_w %s, s_w %s" % (tuple(x.shape), tuple(q_w.shape), tuple(s_w.shape)))
    i = n2 // 2
    y = _out(out, (m, i), torch.bfloat16, x, "out")
    ws = _workspace(workspace, m, k, x)
    _check("convrot_linear_swiglu", load_library().convrot_linear_swiglu(
        x.data_ptr(), m, k, q_w.data_ptr(), s_w.data_ptr(), i, y.data_ptr(), ws.data_ptr(),
        ws.numel(), _stream()))
    return y


def _gemm_args(q_x, s_x, q_w, s_w):
    _dev(q_x, "q_x", torch.int8, 2)
    _dev(q_w, "q_w", torch.int8, 2)
    if s_x is not None:
        _dev(s_x, "s_x", torch.float32, 1)
    if s_w is not None:
        _dev(s_w, "s_w", torch.float32, 1)
    m, k = q_x.shape
    n, k2 = q_w.shape
    if k != k2 or (s_x is not None and s_x.shape[0] != m) or (s_w is not None and s_w.shape[0] != n):
        raise ValueError("shape mismatch")
    return m, n, k


def gemm_dequant(q_x, s_x, q_w, s_w, out=None):
    """bf16 y [m, n] = bf16(((float)(q_x . q_w^T) * s_x) * s_w) on prepared codes."""
    m, n, k = _gemm_args(q_x, s_x, q_w, s_w)
    y = _out(out, (m, n), torch.bfloat16, q_x, "out")
    _check("convrot_gemm_dequant", load_library().convrot_gemm_dequant(
        q_x.data_ptr(), s_x.data_ptr(), q_w.data_ptr(), s_w.data_ptr(), m, n, k, y.data_ptr(),
        _stream()))
    return y


def gemm_swiglu(q_x, s_x, q_w, s_w, out=None):
    """bf16 y [m, i] = SwiGLU epilogue of the contraction with 2i weight rows."""
    m, n2, k = _gemm_args(q_x, s_x, q_w, s_w)
    if n2 % 2:
        raise ValueError("q_w must have an even number of rows (gate then up)")
    i = n2 // 2
    y = _out(out, (m, i), torch.bfloat16, q_x, "out")
    _check("convrot_gemm_swiglu", load_library().convrot_gemm_swiglu(
        q_x.data_ptr(), s_x.data_ptr(), q_w.data_ptr(), s_w.data_ptr(), m, i, k, y.data_ptr(),
        _stream()))
    return y


def gemm_s32(q_x, q_w, out=None):
    """int32 acc [m, n] = q_x . q_w^T (raw accumulators of the same main loop)."""
    m, n, k = _gemm_args(q_x, None, q_w, None)
    acc = _out(out, (m, n), torch.int32, q_x, "out")
    _check("convrot_gemm_s32", load_library().convrot_gemm_s32(
        q_x.data_ptr(), q_w.data_ptr(), m, n, k, acc.data_ptr(), _stream()))
    return acc


# ------------------------------------------------------------------ load-time weight operations

def dequantize_weight(q_w: torch.Tensor, s_w: torch.Tensor, out=None):
    """int8 codes [n, k] + fp32 row scales [n] -> fp32 W [n, k] (unrotated)."""
    _dev(q_w, "q_w", torch.int8, 2)
    _dev(s_w, "s_w", torch.float32, 1)
    n, k = q_w.shape
    if s_w.shape[0] != n:
        raise ValueError("s_w must have %d entries" % n)
    w = _out(out, (n, k), torch.float32, q_w, "out")
    _check("convrot_dequantize_weight", load_library().convrot_dequantize_weight(
        q_w.data_ptr(), s_w.data_ptr(), n, k, w.data_ptr(), _stream()))
    return w


def _lora_args(n, k, b, a):
    if b is None or a is None:
        raise ValueError("lora_b and lora_a are required")
    _dev(b, "lora_b", torch.float32, 2)
    _dev(a, "lora_a", torch.float32, 2)
    rank = b.shape[1]
    if b.shape[0] != n or tuple(a.shape) != (rank, k):
        raise ValueError("lora_b must be [%d, r] and lora_a [r, %d] (got %s, %s)"
                         % (n, k, tuple(b.shape), tuple(a.shape)))
    return rank


def lora_add(w: torch.Tensor, lora_b: torch.Tensor, lora_a: torch.Tensor, scale: float):
    """In place: w [n, k] += scale * (lora_b [n, r] . lora_a [r, k]); returns w."""
    _dev(w, "w", torch.float32, 2)
    n, k = w.shape
    rank = _lora_args(n, k, lora_b, lora_a)
    _check("convrot_lora_add", load_library().convrot_lora_add(
        w.data_ptr(), n, k, lora_b.data_ptr(), lora_a.data_ptr(), rank, float(scale), _stream()))
    return w


def merge_lora(q_w: torch.Tensor, s_w: torch.Tensor, lora_b: torch.Tensor, lora_a: torch.Tensor,
               scale: float, q_out=None, s_out=None, workspace=None):
    """Dequantize, add scale * (lora_b . lora_a), requantize: new (q_w, s_w).
    Pass q_out=q_w, s_out=s_w to update in place."""
    _dev(q_w, "q_w", torch.int8, 2)
    _dev(s_w, "s_w", torch.float32, 1)
    n, k = q_w.shape
    rank = _lora_args(n, k, lora_b, lora_a)
    q_out = _out(q_out, (n, k), torch.int8, q_w, "q_out")
    s_out = _out(s_out, (n,), torch.float32, q_w, "s_out")
    need = int(load_library().convrot_merge_workspace_bytes(n, k))
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q_w.device)
    _check("convrot_merge_lora", load_library().convrot_merge_lora(
        q_w.data_ptr(), s_w.data_ptr(), n, k, lora_b.data_ptr(), lora_a.data_ptr(), rank, float(scale),
        q_out.data_ptr(), s_out.data_ptr(), workspace.data_ptr(), workspace.numel(), _stream()))
    return q_out, s_out


# ------------------------------------------------------------------ attention

def attention_workspace(s: int, heads: int):
    """(bytes, offsets of the five regions) of the attention workspace for s
    tokens and ``heads`` heads of dimension 128 (see convrot.h)."""
    off = (ctypes.c_size_t * 5)()
    n = int(load_library().convrot_attention_workspace(int(s), int(heads), ATTN_HEAD_DIM, off))
    if n == 0 and (s != 0 and heads != 0):
        raise ValueError("invalid attention sizes s=%d heads=%d" % (s, heads))
    return n, [int(x) for x in off]


def _rows_view(t: torch.Tensor, name: str) -> int:
    """Row stride of a 2-D bf16 GPU tensor whose rows are contiguous (a column
    slice of a wider matrix is allowed)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if not t.is_cuda:
        raise ValueError("%s must be a GPU tensor (got %s)" % (name, t.device))
    if t.device.index != torch.cuda.current_device():
        raise ValueError("%s is on %s, but the library launches on the current device cuda:%d"
                         % (name, t.device, torch.cuda.current_device()))
    if t.dtype != torch.bfloat16:
        raise TypeError("%s must be bfloat16 (got %s)" % (name, t.dtype))
    if t.dim() != 2 or (t.shape[1] > 1 and t.stride(1) != 1):
        raise ValueError("%s must be 2-D with unit column stride" % name)
    return t.stride(0) if t.shape[0] > 1 else t.shape[1]


def _attn_inputs(q, k, v, heads):
    ld = _rows_view(q, "q")
    for t, nm in ((k, "k"), (v, "v")):
        if _rows_view(t, nm) != ld and t.shape[0] > 1:
            raise ValueError("q, k and v must share one row stride")
        if tuple(t.shape) != tuple(q.shape):
            raise ValueError("q, k and v must have one shape (got %s, %s)" % (tuple(q.shape), tuple(t.shape)))
    s, w = q.shape
    if w != heads * ATTN_HEAD_DIM:
        raise ValueError("q has %d columns, expected heads * 128 = %d" % (w, heads * ATTN_HEAD_DIM))
    return s, ld


def _attn_workspace(workspace, s, heads, like):
    need, _ = attention_workspace(s, heads)
    if workspace is None:
        return torch.empty(max(need, 16), dtype=torch.uint8, device=like.device)
    _ws_check(workspace)
    return workspace


def attention_prep(q, k, v, heads: int, workspace=None):
    """Quantize Q and K per token-head and lay out V (fp16) in the workspace
    (a uint8 GPU tensor, allocated if None); returns the workspace."""
    s, ld = _attn_inputs(q, k, v, heads)
    ws = _attn_workspace(workspace, s, heads, q)
    _check("convrot_attention_prep", load_library().convrot_attention_prep(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), ld, s, heads, ATTN_HEAD_DIM, ws.data_ptr(),
        ws.numel(), _stream()))
    return ws


def attention_prepared(workspace, s: int, heads: int, out=None):
    """Attention over a prepared workspace -> bf16 [s, heads * 128]."""
    _ws_check(workspace)
    o = _out(out, (s, heads * ATTN_HEAD_DIM), torch.bfloat16, workspace, "out")
    _check("convrot_attention_prepared", load_library().convrot_attention_prepared(
        workspace.data_ptr(), workspace.numel(), s, heads, ATTN_HEAD_DIM, o.data_ptr(),
        heads * ATTN_HEAD_DIM, _stream()))
    return o


def attention(q, k, v, heads: int, out=None, workspace=None):
    """int8 Q.K^T / fp16 P.V attention of bf16 [s, heads * 128] Q, K, V (column
    slices of one QKV matrix are accepted) -> bf16 [s, heads * 128]."""
    s, ld = _attn_inputs(q, k, v, heads)
    ws = _attn_workspace(workspace, s, heads, q)
    o = _out(out, (s, heads * ATTN_HEAD_DIM), torch.bfloat16, q, "out")
    _check("convrot_attention", load_library().convrot_attention(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), ld, s, heads, ATTN_HEAD_DIM, o.data_ptr(),
        heads * ATTN_HEAD_DIM, ws.data_ptr(), ws.numel(), _stream()))
    return o


# ------------------------------------------------------------------ MXFP4

def _mx_outputs(rows, k, like, codes, scales):
    codes = _out(codes, (rows, k // 2), torch.uint8, like, "codes")
    scales = _out(scales, (k // 128, rows, 4), torch.uint8, like, "scales")
    return codes, scales


def mx_quantize_act(x: torch.Tensor, codes=None, scales=None, rotate=False):
    """bf16 x [m, k] -> MXFP4: codes [m, k/2] uint8 and E8M0 scales
    [k/128, m, 4] uint8 (chunk-major), of the Hadamard-256-rotated rows if
    ``rotate``."""
    _dev(x, "x", torch.bfloat16, 2)
    m, k = x.shape
    codes, scales = _mx_outputs(m, k, x, codes, scales)
    _check("convrot_mx_quantize_act", load_library().convrot_mx_quantize_act(
        x.data_ptr(), m, k, int(bool(rotate)), codes.data_ptr(), scales.data_ptr(), _stream()))
    return codes, scales


def mx_quantize_weight(w: torch.Tensor, codes=None, scales=None, rotate=False):
    """fp32 W [n, k] -> MXFP4 codes and scales (load time), rotated if ``rotate``."""
    _dev(w, "w", torch.float32, 2)
    n, k = w.shape
    codes, scales = _mx_outputs(n, k, w, codes, scales)
    _check("convrot_mx_quantize_weight", load_library().convrot_mx_quantize_weight(
        w.data_ptr(), n, k, int(bool(rotate)), codes.data_ptr(), scales.data_ptr(), _stream()))
    return codes, scales


def mx_gemm(a_codes, a_scales, b_codes, b_scales, out=None):
    """bf16 [m, n] = A . B^T of MXFP4 operands."""
    _dev(a_codes, "a_codes", torch.uint8, 2)
    _dev(b_codes, "b_codes", torch.uint8, 2)
    _dev(a_scales, "a_scales", torch.uint8, 3)
    _dev(b_scales, "b_scales", torch.uint8, 3)
    m, k2 = a_codes.shape
    n = b_codes.shape[0]
    k = 2 * k2
    if (b_codes.shape[1] != k2 or tuple(a_scales.shape) != (k // 128, m, 4)
            or tuple(b_scales.shape) != (k // 128, n, 4)):
        raise ValueError("MXFP4 operand shapes do not match")
    y = _out(out, (m, n), torch.bfloat16, a_codes, "out")
    _check("convrot_mx_gemm", load_library().convrot_mx_gemm(
        a_codes.data_ptr(), a_scales.data_ptr(), b_codes.data_ptr(), b_scales.data_ptr(), m, n, k,
        y.data_ptr(), _stream()))
    return y


def mx_workspace_bytes(m: int, k: int) -> int:
    return int(load_library().convrot_mx_workspace_bytes(int(m), int(k)))


def mx_linear(x: torch.Tensor, w_codes: torch.Tensor, w_scales: torch.Tensor, out=None, workspace=None,
              rotate=False):
    """MXFP4 linear: bf16 x [m, k] -> bf16 y [m, n] with an MXFP4 weight prepared
    with the same ``rotate`` flag."""
    _dev(x, "x", torch.bfloat16, 2)
    _dev(w_codes, "w_codes", torch.uint8, 2)
    _dev(w_scales, "w_scales", torch.uint8, 3)
    m, k = x.shape
    n = w_codes.shape[0]
    if w_codes.shape[1] != k // 2 or tuple(w_scales.shape) != (k // 128, n, 4):
        raise ValueError("weight shapes do not match x %s" % (tuple(x.shape),))
    y = _out(out, (m, n), torch.bfloat16, x, "out")
    need = max(mx_workspace_bytes(m, k), 16)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    _check("convrot_mx_linear", load_library().convrot_mx_linear(
        x.data_ptr(), m, k, int(bool(rotate)), w_codes.data_ptr(), w_scales.data_ptr(), n, y.data_ptr(),
        workspace.data_ptr(), workspace.numel(), _stream()))
    return y
