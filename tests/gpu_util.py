"""Helpers for the GPU parity tests: host <-> device copies and the comparison
rules (bit-exact for codes, scales and accumulators; the relative bound for
bf16 outputs)."""
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


def assert_equal(a, b, what=""):
    assert a.shape == b.shape, (what, a.shape, b.shape)
    if not np.array_equal(a, b):
        bad = np.argwhere(a != b) if a.ndim else None
        raise AssertionError("%s: %d mismatches, first %s" % (
            what, int(np.count_nonzero(a != b)), None if bad is None else bad[:5].tolist()))
