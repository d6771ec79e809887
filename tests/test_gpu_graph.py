"""HIP graph capture of the library's calls.

Every entry point enqueues kernels on the caller's stream and allocates,
synchronizes and clears nothing, so a caller can capture a sequence of calls
into a HIP graph and replay it.  Each test captures a sequence once, replays it
several times with the program's own eager work and synchronizations between
the replays (new input bytes copied into the captured input buffer, outputs
overwritten), and requires every replay to match the eager result on the same
input bit for bit.  The eager results are tied to the oracle on sampled rows,
so the graph path carries the same parity as the eager one."""
import numpy as np
import pytest

import oracle
import workloads
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

REPLAYS = 3


@pytest.fixture(scope="module")
def cr():
    import rotation_quantized_dit_amd as cr
    cr.load_library()
    return cr


def _capture(fn):
    """Warm fn up on a side stream, then capture it into a graph."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _replay_and_compare(g, inputs, outputs, new_inputs, eager):
    """For each replay: copy the next input set into the captured buffers,
    overwrite the outputs, replay, and compare with eager(new inputs)."""
    import torch
    for r in range(REPLAYS):
        src = new_inputs[r % len(new_inputs)]
        for dst, val in zip(inputs, src):
            dst.copy_(val)
        for o in outputs:
            o.view(torch.uint8).fill_(0xA5)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        want = eager(src)
        torch.cuda.synchronize()
        for got, exp in zip(outputs, want):
            assert torch.equal(got.view(torch.uint8), exp.view(torch.uint8)), "replay %d differs from eager" % r


def _bf16_input(m, k, seed):
    rng = np.random.default_rng(seed)
    return gu.dev_bf16(workloads.to_bf16_bits(rng.standard_normal((m, k)).astype(np.float32)))


def _weight(n, k, seed):
    rng = np.random.default_rng(seed)
    return gu.dev((rng.standard_normal((n, k)) * 0.02).astype(np.float32))


def test_graph_ffn_step(cr):
    """The FFN step (rotate+quantize, SwiGLU GEMM, rotate+quantize, down GEMM)
    on ragged sizes, captured as four launches."""
    import torch
    m, k1, i, n2 = 777, 1024, 768, 520
    wu = _weight(2 * i, k1, 11)
    wd = _weight(n2, i, 12)
    qwu, swu = cr.quantize_weight(wu)
    qwd, swd = cr.quantize_weight(wd)
    x = _bf16_input(m, k1, 13)
    qx1 = torch.empty((m, k1), dtype=torch.int8, device="cuda")
    sx1 = torch.empty((m,), dtype=torch.float32, device="cuda")
    h = torch.empty((m, i), dtype=torch.bfloat16, device="cuda")
    qx2 = torch.empty((m, i), dtype=torch.int8, device="cuda")
    sx2 = torch.empty((m,), dtype=torch.float32, device="cuda")
    y = torch.empty((m, n2), dtype=torch.bfloat16, device="cuda")

    def step():
        cr.rotate_quant_act(x, qx1, sx1)
        cr.gemm_swiglu(qx1, sx1, qwu, swu, out=h)
        cr.rotate_quant_act(h, qx2, sx2)
        cr.gemm_dequant(qx2, sx2, qwd, swd, out=y)

    def eager(src):
        (xe,) = src
        a, sa = cr.rotate_quant_act(xe)
        he = cr.gemm_swiglu(a, sa, qwu, swu)
        b, sb = cr.rotate_quant_act(he)
        return [a, sa, he, b, sb, cr.gemm_dequant(b, sb, qwd, swd)]

    g = _capture(step)
    news = [(_bf16_input(m, k1, 20 + r),) for r in range(REPLAYS)]
    _replay_and_compare(g, [x], [qx1, sx1, h, qx2, sx2, y], news, eager)

    # the eager step itself against the oracle on sampled rows: the first
    # layer's codes and scales bit for bit, its SwiGLU output within the bound
    rows = np.array([0, 1, 383, 384, 776])
    x_np = gu.host_bf16(news[-1][0])
    q_ref, s_ref = oracle.rotate_quant_act(x_np[rows])
    np.testing.assert_array_equal(gu.host(qx1)[rows], q_ref)
    np.testing.assert_array_equal(gu.host(sx1)[rows].view(np.uint32), s_ref.view(np.uint32))
    ref, mag = oracle.linear_swiglu_ref_rows(x_np, gu.host(qwu), gu.host(swu), rows=rows)
    gu.assert_swiglu_bound(gu.host_bf16(h)[rows], ref, mag, "graph ffn_up rows")


def test_graph_fused_entry_points(cr):
    """convrot_linear_swiglu then convrot_linear with one caller workspace."""
    import torch
    m, k, i, n = 500, 768, 512, 264
    wu = _weight(2 * i, k, 31)
    wd = _weight(n, i, 32)
    qwu, swu = cr.quantize_weight(wu)
    qwd, swd = cr.quantize_weight(wd)
    x = _bf16_input(m, k, 33)
    ws = torch.empty(max(cr.workspace_bytes(m, k), cr.workspace_bytes(m, i)), dtype=torch.uint8, device="cuda")
    h = torch.empty((m, i), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")

    def step():
        cr.linear_swiglu(x, qwu, swu, out=h, workspace=ws)
        cr.linear(h, qwd, swd, out=y, workspace=ws)

    def eager(src):
        (xe,) = src
        he = cr.linear_swiglu(xe, qwu, swu)
        return [he, cr.linear(he, qwd, swd)]

    g = _capture(step)
    _replay_and_compare(g, [x], [h, y], [(_bf16_input(m, k, 40 + r),) for r in range(REPLAYS)], eager)


def test_graph_attention(cr):
    """Attention (prep + flash) on column slices of one QKV matrix, with a
    caller workspace."""
    import torch
    s, heads = 300, 2
    w = heads * cr.ATTN_HEAD_DIM
    qkv = _bf16_input(s, 3 * w, 51)
    ws = torch.empty(max(cr.attention_workspace(s, heads)[0], 16), dtype=torch.uint8, device="cuda")
    o = torch.empty((s, w), dtype=torch.bfloat16, device="cuda")

    def step():
        cr.attention(qkv[:, :w], qkv[:, w:2 * w], qkv[:, 2 * w:], heads, out=o, workspace=ws)

    def eager(src):
        (qe,) = src
        return [cr.attention(qe[:, :w], qe[:, w:2 * w], qe[:, 2 * w:], heads)]

    g = _capture(step)
    _replay_and_compare(g, [qkv], [o], [(_bf16_input(s, 3 * w, 60 + r),) for r in range(REPLAYS)], eager)


@pytest.mark.parametrize("rotate", [False, True])
def test_graph_mx_linear(cr, rotate):
    """The MXFP4 linear (quantize + scaled FP4 GEMM) with a caller workspace."""
    import torch
    m, k, n = 300, 512, 256
    wc, wsc = cr.mx_quantize_weight(_weight(n, k, 71), rotate=rotate)
    x = _bf16_input(m, k, 72)
    ws = torch.empty(max(cr.mx_workspace_bytes(m, k), 16), dtype=torch.uint8, device="cuda")
    y = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")

    def step():
        cr.mx_linear(x, wc, wsc, out=y, workspace=ws, rotate=rotate)

    def eager(src):
        (xe,) = src
        return [cr.mx_linear(xe, wc, wsc, rotate=rotate)]

    g = _capture(step)
    _replay_and_compare(g, [x], [y], [(_bf16_input(m, k, 80 + r),) for r in range(REPLAYS)], eager)
