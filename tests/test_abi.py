"""The C ABI loads, exports what include/convrot.h declares, and rejects bad
arguments on the host before anything touches a device (CPU only: every call
here fails validation or is a zero-size no-op, so no HIP call is made)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "convrot.h")


@pytest.fixture(scope="module")
def L():
    from rotation_quantized_dit_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from rotation_quantized_dit_amd import build
        build.build()
    return _lib.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(convrot_\w+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for must in ("convrot_quantize_weight", "convrot_rotate_quant_act", "convrot_linear",
                 "convrot_linear_swiglu"):
        assert must in names


def test_library_exports_every_declared_symbol(L):
    from rotation_quantized_dit_amd import _lib
    names = declared_functions()
    assert sorted(_lib.SYMBOLS) == names
    for n in names:
        assert hasattr(L, n), n
    # and exports them with C linkage (unmangled), nothing else named convrot_
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = sorted(set(re.findall(r"\bT (convrot_\w+)$", out, flags=re.M)))
    assert exported == names


def test_status_strings(L):
    from rotation_quantized_dit_amd import _lib
    for st in range(7):
        s = _lib.status_string(st)
        assert isinstance(s, str) and s
    assert _lib.status_string(0) == "ok"
    assert "unknown" in _lib.status_string(99)


def test_workspace_bytes(L):
    assert L.convrot_workspace_bytes(32256, 5376) == 32256 * 5376 + 4 * 32256
    assert L.convrot_workspace_bytes(0, 256) == 0
    assert L.convrot_workspace_bytes(10, 255) == 0
    assert L.convrot_workspace_bytes(-1, 256) == 0
    assert L.convrot_workspace_bytes(1, 133120) == 133120 + 4
    assert L.convrot_workspace_bytes(1, 133376) == 0


A = 0x10000        # aligned fake device addresses: never dereferenced, validation fails first
B = 0x20000
C = 0x30000
D = 0x40000
MIS = 0x10008


def test_k_bounds(L):
    """k must be a positive multiple of 256 and at most 133120 (127^2 k < 2^31)."""
    from rotation_quantized_dit_amd._lib import ERR_SHAPE
    for k in (0, -256, 100, 257, 133376, 1 << 20):
        assert L.convrot_rotate_quant_act(A, 4, k, B, C, None) == ERR_SHAPE, k
        assert L.convrot_quantize_weight(A, 4, k, B, C, None) == ERR_SHAPE, k
        assert L.convrot_gemm_s32(A, B, 4, 4, k, C, None) == ERR_SHAPE, k
        assert L.convrot_linear(A, 4, k, B, C, 4, D, A, 1 << 30, None) == ERR_SHAPE, k
        assert L.convrot_swiglu_rotate_quant_act(A, 4, k, B, C, None) == ERR_SHAPE, k


def test_negative_sizes(L):
    from rotation_quantized_dit_amd._lib import ERR_SHAPE
    assert L.convrot_rotate_quant_act(A, -1, 256, B, C, None) == ERR_SHAPE
    assert L.convrot_quantize_weight(A, -5, 256, B, C, None) == ERR_SHAPE
    assert L.convrot_gemm_s32(A, B, -1, 4, 256, C, None) == ERR_SHAPE
    assert L.convrot_gemm_s32(A, B, 4, -1, 256, C, None) == ERR_SHAPE
    assert L.convrot_gemm_dequant(A, B, C, D, 4, -1, 256, A, None) == ERR_SHAPE
    assert L.convrot_gemm_swiglu(A, B, C, D, 4, -1, 256, A, None) == ERR_SHAPE
    assert L.convrot_linear(A, 4, 256, B, C, -1, D, A, 1 << 20, None) == ERR_SHAPE
    assert L.convrot_linear_swiglu(A, 4, 256, B, C, -3, D, A, 1 << 20, None) == ERR_SHAPE
    assert L.convrot_rotate_quant_act(A, 1 << 32, 256, B, C, None) == ERR_SHAPE
    assert L.convrot_swiglu_rotate_quant_act(A, -1, 256, B, C, None) == ERR_SHAPE


def test_null_pointers(L):
    from rotation_quantized_dit_amd._lib import ERR_NULL
    assert L.convrot_rotate_quant_act(None, 4, 256, B, C, None) == ERR_NULL
    assert L.convrot_rotate_quant_act(A, 4, 256, None, C, None) == ERR_NULL
    assert L.convrot_rotate_quant_act(A, 4, 256, B, None, None) == ERR_NULL
    assert L.convrot_quantize_weight(A, 4, 256, B, None, None) == ERR_NULL
    assert L.convrot_gemm_s32(None, B, 4, 4, 256, C, None) == ERR_NULL
    assert L.convrot_gemm_s32(A, B, 4, 4, 256, None, None) == ERR_NULL
    assert L.convrot_gemm_dequant(A, None, C, D, 4, 4, 256, A, None) == ERR_NULL
    assert L.convrot_gemm_dequant(A, B, C, None, 4, 4, 256, A, None) == ERR_NULL
    assert L.convrot_gemm_swiglu(A, B, None, D, 4, 4, 256, A, None) == ERR_NULL
    assert L.convrot_linear(A, 4, 256, B, None, 4, D, A, 1 << 20, None) == ERR_NULL
    assert L.convrot_linear_swiglu(A, 4, 256, B, C, 4, None, A, 1 << 20, None) == ERR_NULL
    assert L.convrot_swiglu_rotate_quant_act(None, 4, 256, B, C, None) == ERR_NULL
    assert L.convrot_swiglu_rotate_quant_act(A, 4, 256, None, C, None) == ERR_NULL
    assert L.convrot_swiglu_rotate_quant_act(A, 4, 256, B, None, None) == ERR_NULL


def test_alignment(L):
    from rotation_quantized_dit_amd._lib import ERR_ALIGN
    assert L.convrot_rotate_quant_act(MIS, 4, 256, B, C, None) == ERR_ALIGN
    assert L.convrot_rotate_quant_act(A, 4, 256, B + 1, C, None) == ERR_ALIGN
    assert L.convrot_quantize_weight(A, 4, 256, B, C + 4, None) == ERR_ALIGN
    assert L.convrot_gemm_s32(A, B + 2, 4, 4, 256, C, None) == ERR_ALIGN
    assert L.convrot_gemm_dequant(A, B, C, D, 4, 4, 256, A + 8, None) == ERR_ALIGN
    assert L.convrot_linear(A, 4, 256, B, C, 4, D, MIS, 1 << 20, None) == ERR_ALIGN
    assert L.convrot_swiglu_rotate_quant_act(MIS, 4, 256, B, C, None) == ERR_ALIGN
    assert L.convrot_swiglu_rotate_quant_act(A, 4, 256, B, C + 4, None) == ERR_ALIGN


def test_workspace_checks(L):
    from rotation_quantized_dit_amd._lib import ERR_WORKSPACE
    need = L.convrot_workspace_bytes(4, 256)
    assert L.convrot_linear(A, 4, 256, B, C, 4, D, None, need, None) == ERR_WORKSPACE
    assert L.convrot_linear(A, 4, 256, B, C, 4, D, A, need - 1, None) == ERR_WORKSPACE
    assert L.convrot_linear_swiglu(A, 4, 256, B, C, 4, D, A, need - 1, None) == ERR_WORKSPACE


def test_zero_sizes_are_noops(L):
    """m == 0 or n == 0 succeed without launching (safe with fake pointers)."""
    from rotation_quantized_dit_amd._lib import OK
    assert L.convrot_rotate_quant_act(A, 0, 256, B, C, None) == OK
    assert L.convrot_quantize_weight(A, 0, 512, B, C, None) == OK
    assert L.convrot_gemm_s32(A, B, 0, 4, 256, C, None) == OK
    assert L.convrot_gemm_s32(A, B, 4, 0, 256, C, None) == OK
    assert L.convrot_gemm_dequant(A, B, C, D, 0, 4, 256, A, None) == OK
    assert L.convrot_gemm_swiglu(A, B, C, D, 4, 0, 256, A, None) == OK
    assert L.convrot_linear(A, 0, 256, B, C, 4, D, None, 0, None) == OK
    assert L.convrot_linear_swiglu(A, 7, 256, B, C, 0, D, None, 0, None) == OK
    assert L.convrot_swiglu_rotate_quant_act(None, 0, 512, None, None, None) == OK
    # empty calls may pass NULL (torch's empty tensors do), but bad shapes still fail
    assert L.convrot_rotate_quant_act(None, 0, 256, None, None, None) == OK
    assert L.convrot_gemm_s32(None, None, 0, 0, 256, None, None) == OK
    assert L.convrot_linear(None, 0, 512, None, None, 9, None, None, 0, None) == OK
    assert L.convrot_rotate_quant_act(None, 0, 300, None, None, None) != OK


def test_python_binding_rejects_cpu_tensors():
    import torch
    import rotation_quantized_dit_amd as cr
    with pytest.raises(ValueError):
        cr.rotate_quant_act(torch.zeros(4, 256, dtype=torch.bfloat16))
    with pytest.raises((TypeError, ValueError)):
        cr.quantize_weight(torch.zeros(4, 256, dtype=torch.float64))


def test_weight_ops_validation(L):
    """Load-time weight entry points: host-side checks before any launch."""
    from rotation_quantized_dit_amd._lib import ERR_ALIGN, ERR_NULL, ERR_SHAPE, ERR_WORKSPACE, OK
    assert L.convrot_dequantize_weight(A, B, 4, 300, C, None) == ERR_SHAPE
    assert L.convrot_dequantize_weight(A, B, -1, 256, C, None) == ERR_SHAPE
    assert L.convrot_dequantize_weight(None, B, 4, 256, C, None) == ERR_NULL
    assert L.convrot_dequantize_weight(A, B, 4, 256, C + 4, None) == ERR_ALIGN
    assert L.convrot_dequantize_weight(None, None, 0, 256, None, None) == OK
    assert L.convrot_lora_add(A, 4, 256, B, C, -1, 1.0, None) == ERR_SHAPE
    assert L.convrot_lora_add(A, 4, 512, None, C, 3, 1.0, None) == ERR_NULL
    assert L.convrot_lora_add(A, 4, 512, B, None, 3, 1.0, None) == ERR_NULL
    assert L.convrot_lora_add(A, 4, 512, B + 4, C, 3, 1.0, None) == ERR_ALIGN
    assert L.convrot_lora_add(A, 0, 512, None, None, 3, 1.0, None) == OK
    assert L.convrot_merge_workspace_bytes(10, 512) == 4 * 10 * 512
    assert L.convrot_merge_workspace_bytes(10, 500) == 0
    need = L.convrot_merge_workspace_bytes(4, 256)
    assert L.convrot_merge_lora(A, B, 4, 256, C, D, 2, 1.0, A, B, D, need - 1, None) == ERR_WORKSPACE
    assert L.convrot_merge_lora(A, B, 4, 256, C, D, 2, 1.0, A, B, None, need, None) == ERR_WORKSPACE
    assert L.convrot_merge_lora(A, B, 4, 256, C, D, 2, 1.0, A, B, MIS, need, None) == ERR_ALIGN
    assert L.convrot_merge_lora(A, None, 4, 256, C, D, 2, 1.0, A, B, D, need, None) == ERR_NULL
    assert L.convrot_merge_lora(A, B, 4, 257, C, D, 2, 1.0, A, B, D, need, None) == ERR_SHAPE
    assert L.convrot_merge_lora(None, None, 0, 256, None, None, 2, 1.0, None, None, None, 0, None) == OK


def test_attention_validation(L):
    """Attention entry points: sizes, head dimension, strides, pointers and the
    workspace are checked on the host; empty calls are no-ops."""
    from rotation_quantized_dit_amd._lib import ERR_ALIGN, ERR_NULL, ERR_SHAPE, ERR_WORKSPACE, OK
    off = (ctypes.c_size_t * 5)()
    need = L.convrot_attention_workspace(65, 2, 128, off)
    s_pad = 128
    assert list(off) == [0, 16640, 17408, 17408 + 2 * s_pad * 128, 50176 + 1024]
    assert need == off[4] + 2 * s_pad * 128 * 2
    assert L.convrot_attention_workspace(65, 2, 64, None) == 0
    assert L.convrot_attention_workspace(-1, 2, 128, None) == 0
    assert L.convrot_attention_workspace((1 << 24) + 1, 1, 128, None) == 0
    # the largest accepted s: one head's V blocks (s_pad x 128 fp16) end just
    # below 2^32 bytes; every s that pads to 2^24 keys is rejected before launch
    assert L.convrot_attention_workspace((1 << 24) - 64, 1, 128, None) > 0
    for s in ((1 << 24) - 63, (1 << 24) - 1, 1 << 24):
        assert L.convrot_attention_workspace(s, 1, 128, None) == 0, s
        assert L.convrot_attention_prep(A, B, C, 128, s, 1, 128, D, 1 << 40, None) == ERR_SHAPE, s
        assert L.convrot_attention_prepared(D, 1 << 40, s, 1, 128, A, 128, None) == ERR_SHAPE, s
        assert L.convrot_attention(A, B, C, 128, s, 1, 128, A, 128, D, 1 << 40, None) == ERR_SHAPE, s
    assert L.convrot_attention_workspace(0, 5, 128, None) == 0
    ld = 3 * 2 * 128
    assert L.convrot_attention_prep(A, B, C, ld, 65, 2, 64, D, need, None) == ERR_SHAPE
    assert L.convrot_attention_prep(A, B, C, 255, 65, 2, 128, D, need, None) == ERR_SHAPE
    assert L.convrot_attention_prep(A, B, C, 128, 65, 2, 128, D, need, None) == ERR_SHAPE
    assert L.convrot_attention_prep(A, B, C, ld, -3, 2, 128, D, need, None) == ERR_SHAPE
    assert L.convrot_attention_prep(None, B, C, ld, 65, 2, 128, D, need, None) == ERR_NULL
    assert L.convrot_attention_prep(MIS, B, C, ld, 65, 2, 128, D, need, None) == ERR_ALIGN
    assert L.convrot_attention_prep(A, B, C, ld, 65, 2, 128, D, need - 1, None) == ERR_WORKSPACE
    assert L.convrot_attention_prep(A, B, C, ld, 65, 2, 128, None, need, None) == ERR_WORKSPACE
    assert L.convrot_attention_prep(A, B, C, ld, 65, 2, 128, MIS, need, None) == ERR_ALIGN
    assert L.convrot_attention_prepared(D, need, 65, 2, 128, None, 256, None) == ERR_NULL
    assert L.convrot_attention_prepared(D, need, 65, 2, 128, A, 200, None) == ERR_SHAPE
    assert L.convrot_attention_prepared(D, need - 1, 65, 2, 128, A, 256, None) == ERR_WORKSPACE
    assert L.convrot_attention_prepared(D, need, 65, 2, 128, MIS, 256, None) == ERR_ALIGN
    assert L.convrot_attention(A, B, C, ld, 65, 2, 128, None, 256, D, need, None) == ERR_NULL
    assert L.convrot_attention(A, B, C, ld, 65, 2, 128, A, 100, D, need, None) == ERR_SHAPE
    # empty calls: nothing enqueued, NULL pointers allowed
    assert L.convrot_attention(None, None, None, 768, 0, 2, 128, None, 256, None, 0, None) == OK
    assert L.convrot_attention_prep(None, None, None, 0, 10, 0, 128, None, 0, None) == OK
    assert L.convrot_attention_prepared(None, 0, 0, 3, 128, None, 384, None) == OK


def test_mx_validation(L):
    """MXFP4 entry points: k multiple of 128 (256 when rotating), pointers,
    workspace; empty calls are no-ops."""
    from rotation_quantized_dit_amd._lib import ERR_ALIGN, ERR_NULL, ERR_SHAPE, ERR_WORKSPACE, OK
    assert L.convrot_mx_quantize_act(A, 4, 200, 0, B, C, None) == ERR_SHAPE
    assert L.convrot_mx_quantize_act(A, 4, 384, 1, B, C, None) == ERR_SHAPE
    assert L.convrot_mx_quantize_act(A, -1, 256, 0, B, C, None) == ERR_SHAPE
    assert L.convrot_mx_quantize_act(None, 4, 256, 0, B, C, None) == ERR_NULL
    assert L.convrot_mx_quantize_act(MIS, 4, 256, 0, B, C, None) == ERR_ALIGN
    assert L.convrot_mx_quantize_act(None, 0, 256, 1, None, None, None) == OK
    assert L.convrot_mx_quantize_weight(A, 4, (1 << 20) + 128, 0, B, C, None) == ERR_SHAPE
    assert L.convrot_mx_quantize_weight(A, 4, 256, 0, None, C, None) == ERR_NULL
    assert L.convrot_mx_gemm(A, B, C, D, 4, 4, 100, A, None) == ERR_SHAPE
    assert L.convrot_mx_gemm(A, B, C, None, 4, 4, 128, A, None) == ERR_NULL
    assert L.convrot_mx_gemm(A, B, C, D, 4, 4, 128, MIS, None) == ERR_ALIGN
    assert L.convrot_mx_gemm(None, None, None, None, 0, 4, 128, None, None) == OK
    need = L.convrot_mx_workspace_bytes(10, 512)
    assert need == 2560 + 10 * 16
    assert L.convrot_mx_workspace_bytes(10, 100) == 0
    assert L.convrot_mx_linear(A, 10, 512, 0, B, C, 4, D, D, need - 1, None) == ERR_WORKSPACE
    assert L.convrot_mx_linear(A, 10, 512, 0, B, C, 4, D, None, need, None) == ERR_WORKSPACE
    assert L.convrot_mx_linear(A, 10, 512, 0, B, C, 4, D, MIS, need, None) == ERR_ALIGN
    assert L.convrot_mx_linear(A, 10, 384, 1, B, C, 4, D, D, need, None) == ERR_SHAPE
    assert L.convrot_mx_linear(None, 0, 512, 0, None, None, 4, None, None, 0, None) == OK


@pytest.mark.parametrize("lang", ["c", "c++"])
def test_header_compiles_as_c_and_cpp(lang):
    """include/convrot.h stands alone as C99 and as C++17, warnings as errors."""
    from tests import c_abi_build
    c_abi_build.compile_only("c-header" if lang == "c" else "c++")


def test_c_abi_check_source_compiles():
    """tests/c_abi_check.c (the C-side check run on the GPU) is valid C11."""
    from tests import c_abi_build
    c_abi_build.compile_only("c")


def test_linear_noalloc_validation(L):
    """convrot_linear_noalloc: the checks of convrot_linear, then the size bound
    of its built-in scratch (m k + 4 m bytes), all on the host before any HIP
    call; empty calls are no-ops."""
    from rotation_quantized_dit_amd._lib import (ERR_ALIGN, ERR_NULL, ERR_SCRATCH, ERR_SHAPE, NOALLOC_SCRATCH_BYTES,
                                                 OK)
    f = L.convrot_linear_noalloc
    assert NOALLOC_SCRATCH_BYTES == 64 << 20
    for k in (0, 100, 133376):
        assert f(A, 4, k, B, C, 4, D, None) == ERR_SHAPE, k
    assert f(A, -1, 256, B, C, 4, D, None) == ERR_SHAPE
    assert f(None, 0, 256, None, None, 4, None, None) == OK
    assert f(None, 4, 256, None, None, 0, None, None) == OK
    assert f(None, 4, 256, B, C, 4, D, None) == ERR_NULL
    assert f(MIS, 4, 256, B, C, 4, D, None) == ERR_ALIGN
    # the largest m that fits at k = 5376, and the next one
    k = 5376
    m_max = NOALLOC_SCRATCH_BYTES // (k + 4)
    assert m_max * (k + 4) <= NOALLOC_SCRATCH_BYTES < (m_max + 1) * (k + 4)
    assert f(A, m_max + 1, k, B, C, 16, D, None) == ERR_SCRATCH
    assert f(A, 1 << 20, 14336, B, C, 16, D, None) == ERR_SCRATCH
    assert "scratch" in L.convrot_status_string(ERR_SCRATCH).decode()
