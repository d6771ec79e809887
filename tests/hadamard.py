"""Independent test-side constructions used to pin the oracle (no oracle code).

The Sylvester Hadamard matrix is written from its closed form
H[i][j] = (-1)^popcount(i & j); nothing here is shared with the oracle or the
HIP library."""
import numpy as np

G = 256


def sylvester(n: int = G) -> np.ndarray:
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    bits = np.vectorize(lambda v: bin(int(v)).count("1"))(i & j)
    return np.where(bits % 2 == 0, 1, -1).astype(np.int64)


_H = None


def H() -> np.ndarray:
    global _H
    if _H is None:
        _H = sylvester(G)
    return _H


def rotate_fp64(x: np.ndarray) -> np.ndarray:
    """Dense fp64 group-wise rotation x -> x . blockdiag(H/16) along the last axis."""
    x = np.asarray(x, dtype=np.float64)
    k = x.shape[-1]
    h = H().astype(np.float64) / 16.0
    out = np.empty_like(x)
    for g in range(0, k, G):
        out[..., g:g + G] = x[..., g:g + G] @ h  # H symmetric: row . H == (H . row^T)^T
    return out


def bf16_bits_to_f64(h: np.ndarray) -> np.ndarray:
    return (np.asarray(h, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)


def is_bf16_exact(x: np.ndarray) -> bool:
    f = np.asarray(x, dtype=np.float32)
    return bool(np.all((f.view(np.uint32) & 0xFFFF) == 0)) and bool(np.all(f.astype(np.float64) == np.asarray(x, np.float64)))


def rn_f32(q) -> float:
    """Exact round-to-nearest-even of a rational (fractions.Fraction) to a
    normal fp32 value, from the definition of the format."""
    from fractions import Fraction
    q = Fraction(q)
    if q == 0:
        return 0.0
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    elif Fraction(2) ** (e + 1) <= a:
        e += 1
    assert -126 <= e <= 127
    ulp = Fraction(2) ** (e - 23)
    n = a / ulp
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * float(fl * ulp)


def rint_half_even(x: float) -> int:
    """Round half to even of an exact binary value."""
    from fractions import Fraction
    f = Fraction(x)
    fl = f.numerator // f.denominator
    rem = f - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return int(fl)
