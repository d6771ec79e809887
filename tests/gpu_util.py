"""Helpers for the GPU parity tests: host <-> device copies and the comparison
rules (bit-exact for codes, scales and accumulators; the relative bound for
bf16 outputs, with bit equality wherever both sides evaluate the same
rounding sequence, and a derived per-element bound for the fused SwiGLU
epilogue, which runs on the hardware exponential and reciprocal)."""
import numpy as np
import torch

REL_TOL = 1e-2
ABS_FLOOR = 1e-3


def dev_bf16(x_bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16)).view(torch.bfloat16).cuda()


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host_bf16(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def host(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().cpu().numpy()


def bf16_f64(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)


def max_rel_err(y_gpu_bits: np.ndarray, y_ref_bits: np.ndarray) -> float:
    """max_i |y_gpu - y_ref| / max(|y_ref|, 1e-3) over bf16 outputs."""
    a = bf16_f64(y_gpu_bits)
    b = bf16_f64(y_ref_bits)
    if a.size == 0:
        return 0.0
    return float(np.max(np.abs(a - b) / np.maximum(np.abs(b), ABS_FLOOR)))


def assert_bf16_parity(y_gpu_bits, y_ref_bits, what=""):
    """The output bar (relative error <= 1e-2 with a 1e-3 floor) and, since both
    sides evaluate the same rounding sequence, bit equality."""
    assert y_gpu_bits.shape == y_ref_bits.shape, (what, y_gpu_bits.shape, y_ref_bits.shape)
    err = max_rel_err(y_gpu_bits, y_ref_bits)
    assert err <= REL_TOL, (what, err)
    diff = int(np.count_nonzero(y_gpu_bits != y_ref_bits))
    assert diff == 0, (what, "non-identical bf16 elements", diff, y_gpu_bits.size, err)


def assert_swiglu_bound(y_gpu_bits, ref, mag, what=""):
    """The fused SwiGLU epilogue against the oracle's exact value ref (fp64,
    from the same fp32 dequantized g and u): per element
    |y - ref| <= 2^-8 |ref| + 2^-120 (1 + |g u|), i.e. one bf16 rounding (2^-9)
    plus the fp32 evaluation's ~1.2e-5 relative error with margin, and an
    absolute term far below any normal bf16 value for the case where the
    reciprocal of 1 + e^-g > 2^126 flushes; and the output bar (relative error
    <= 1e-2 with a 1e-3 floor)."""
    assert y_gpu_bits.shape == ref.shape, (what, y_gpu_bits.shape, ref.shape)
    y = bf16_f64(y_gpu_bits)
    err = np.abs(y - ref)
    tol = 2.0 ** -8 * np.abs(ref) + 2.0 ** -120 * (1.0 + mag)
    bad = ~(err <= tol)
    if bad.any():
        i = np.unravel_index(int(np.argmax(np.where(bad, err / tol, 0))), err.shape)
        raise AssertionError("%s: %d of %d outside the bound; worst at %s: gpu %r ref %r tol %r" % (
            what, int(bad.sum()), bad.size, i, y[i], ref[i], tol[i]))
    if y.size:
        rel = float(np.max(err / np.maximum(np.abs(ref), ABS_FLOOR)))
        assert rel <= REL_TOL, (what, rel)
        exact = ref.astype(np.float32)
        rounded = bf16_f64((exact.view(np.uint32) + 0x7FFF + ((exact.view(np.uint32) >> 16) & 1)) >> 16)
        print("%s: max err / bound %.3f, %d of %d elements differ from the exact value rounded once" % (
            what, float(np.max(err / tol)), int(np.count_nonzero(y != rounded)), y.size), flush=True)


def assert_equal(a, b, what=""):
    assert a.shape == b.shape, (what, a.shape, b.shape)
    if not np.array_equal(a, b):
        bad = np.argwhere(a != b) if a.ndim else None
        raise AssertionError("%s: %d mismatches, first %s" % (
            what, int(np.count_nonzero(a != b)), None if bad is None else bad[:5].tolist()))
