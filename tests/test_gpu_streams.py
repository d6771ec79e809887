"""Calls on several streams at once.

The library keeps no state between calls: every buffer is the caller's and
every launch goes to the stream the call names.  Independent calls issued on
different streams, with nothing ordering them, must therefore give the same
bytes as the same calls made one after another on one stream.  (All streams
here have the default priority.)"""
import numpy as np
import pytest

from tests import gpu_util as gu
import workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def cr():
    import rotation_quantized_dit_amd as cr
    cr.load_library()
    return cr


def _bf16(m, k, seed):
    rng = np.random.default_rng(seed)
    return gu.dev_bf16(workloads.to_bf16_bits(rng.standard_normal((m, k)).astype(np.float32)))


def _weight(n, k, seed):
    rng = np.random.default_rng(seed)
    return gu.dev((rng.standard_normal((n, k)) * 0.02).astype(np.float32))


def test_concurrent_streams_match_sequential(cr):
    import torch
    heads, s = 2, 400
    w = heads * cr.ATTN_HEAD_DIM
    m, k, i, n = 900, 1024, 768, 520
    qwu, swu = cr.quantize_weight(_weight(2 * i, k, 1))
    qwd, swd = cr.quantize_weight(_weight(n, i, 2))
    mxc, mxs = cr.mx_quantize_weight(_weight(n, k, 3), rotate=True)
    xs = [_bf16(m, k, 10 + j) for j in range(3)]
    qkv = _bf16(s, 3 * w, 20)
    torch.cuda.synchronize()

    def ffn(x, out_h, out_y, ws):
        cr.linear_swiglu(x, qwu, swu, out=out_h, workspace=ws)
        cr.linear(out_h, qwd, swd, out=out_y, workspace=ws)

    def attn(o, ws):
        cr.attention(qkv[:, :w], qkv[:, w:2 * w], qkv[:, 2 * w:], heads, out=o, workspace=ws)

    def mx(x, y, ws):
        cr.mx_linear(x, mxc, mxs, out=y, workspace=ws, rotate=True)

    def buffers():
        return {
            "h": [torch.empty((m, i), dtype=torch.bfloat16, device="cuda") for _ in xs],
            "y": [torch.empty((m, n), dtype=torch.bfloat16, device="cuda") for _ in xs],
            "ws": [torch.empty(cr.workspace_bytes(m, k), dtype=torch.uint8, device="cuda") for _ in xs],
            "o": torch.empty((s, w), dtype=torch.bfloat16, device="cuda"),
            "aws": torch.empty(max(cr.attention_workspace(s, heads)[0], 16), dtype=torch.uint8, device="cuda"),
            "my": torch.empty((m, n), dtype=torch.bfloat16, device="cuda"),
            "mws": torch.empty(max(cr.mx_workspace_bytes(m, k), 16), dtype=torch.uint8, device="cuda"),
        }

    # one after another on the current stream
    seq = buffers()
    for j, x in enumerate(xs):
        ffn(x, seq["h"][j], seq["y"][j], seq["ws"][j])
    attn(seq["o"], seq["aws"])
    mx(xs[0], seq["my"], seq["mws"])
    torch.cuda.synchronize()

    # the same calls spread over five streams, nothing ordering them
    con = buffers()
    for b in con["h"] + con["y"] + [con["o"], con["my"]]:
        b.view(torch.uint8).fill_(0x5A)
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in range(5)]
    for j, x in enumerate(xs):
        with torch.cuda.stream(streams[j]):
            ffn(x, con["h"][j], con["y"][j], con["ws"][j])
    with torch.cuda.stream(streams[3]):
        attn(con["o"], con["aws"])
    with torch.cuda.stream(streams[4]):
        mx(xs[0], con["my"], con["mws"])
    torch.cuda.synchronize()

    for key in ("h", "y"):
        for j in range(len(xs)):
            assert torch.equal(con[key][j].view(torch.int16), seq[key][j].view(torch.int16)), (key, j)
    assert torch.equal(con["o"].view(torch.int16), seq["o"].view(torch.int16))
    assert torch.equal(con["my"].view(torch.int16), seq["my"].view(torch.int16))
