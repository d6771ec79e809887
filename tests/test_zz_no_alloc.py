"""convrot_linear_noalloc (the linear with the library's own device scratch as
its workspace) against convrot_linear with a caller workspace, through the C
ABI: two calls in a row, the first at the largest size the scratch accepts,
the second smaller, each bit for bit equal to convrot_linear's output (the
same kernels on the same codes); the smaller one also against the oracle."""
import ctypes

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


def _case(rng, m, n, k):
    x = rng.standard_normal((m, k), dtype=np.float32)
    x[:, rng.choice(k, max(1, k // 100), replace=False)] *= 30
    w = (0.02 * rng.standard_normal((n, k))).astype(np.float32)
    return workloads.to_bf16_bits(x), w


def test_noalloc_matches_linear_two_calls(cr):
    import torch
    from rotation_quantized_dit_amd import _lib
    L = _lib.load_library()
    k1 = 5376
    m1 = _lib.NOALLOC_SCRATCH_BYTES // (k1 + 4)          # the largest m at this k
    rng = np.random.default_rng(11)
    for (m, n, k) in ((m1, 320, k1), (300, 513, 768)):
        print("noalloc case m=%d n=%d k=%d" % (m, n, k), flush=True)
        x_bits, w = _case(rng, m, n, k)
        xd, wd = gu.dev_bf16(x_bits), gu.dev(w)
        qw, sw = cr.quantize_weight(wd)
        y_ref = cr.linear(xd, qw, sw)
        y = torch.full((m, n), float("nan"), dtype=torch.bfloat16, device=xd.device)
        st = L.convrot_linear_noalloc(xd.data_ptr(), m, k, qw.data_ptr(), sw.data_ptr(), n, y.data_ptr(),
                                      ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        assert st == _lib.OK, _lib.status_string(st)
        torch.cuda.synchronize()
        gu.assert_equal(gu.host_bf16(y), gu.host_bf16(y_ref), "noalloc %dx%dx%d vs convrot_linear" % (m, n, k))
        if m * n * k <= 300 * 513 * 768:
            oqw, osw = oracle.quantize_weight(w)
            gu.assert_bf16_parity(gu.host_bf16(y), oracle.linear_rows(x_bits, oqw, osw), "noalloc vs oracle")
        del xd, wd, qw, sw, y, y_ref
    # the binding raises on the size bound without enqueuing anything
    x = torch.zeros((m1 + 1, k1), dtype=torch.bfloat16, device="cuda")
    qw = torch.zeros((8, k1), dtype=torch.int8, device="cuda")
    sw = torch.zeros((8,), dtype=torch.float32, device="cuda")
    with pytest.raises(_lib.ConvRotError) as e:
        cr.linear_noalloc(x, qw, sw)
    assert e.value.status == _lib.ERR_SCRATCH
