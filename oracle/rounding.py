"""Round-to-nearest-even of float64 values to the storage dtype.  TEST INFRASTRUCTURE ONLY.

The stored value of a rotated vector element is its exact float64 value rounded once to the storage dtype
(bf16: 8 significant bits and fp32's exponent range; fp32).  The pages do not name the rounding mode; the
reading taken is IEEE round-to-nearest, ties to even.
"""
import numpy as np

_BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127


def rne_bf16(x: np.ndarray) -> np.ndarray:
    """float64 -> nearest bf16 value (ties to even), returned as float64.

    x = m * 2**e with 0.5 <= |m| < 1; bf16 keeps 8 significant bits, so the quantum is 2**(e-8), and never
    below the subnormal quantum 2**-133.  Scaling by a power of two is exact, and np.rint rounds half to even.
    """
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    e = np.maximum(e, -125)
    q = np.ldexp(1.0, e - 8)
    r = np.rint(x / q) * q
    return np.where(np.abs(r) > _BF16_MAX, np.copysign(np.inf, r), r)


def rne_f32(x: np.ndarray) -> np.ndarray:
    """float64 -> nearest float32 value (numpy's conversion rounds to nearest even), returned as float64."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def rne(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return rne_bf16(x)
    if dtype == "fp32":
        return rne_f32(x)
    raise ValueError(dtype)


def storage_bytes(dtype: str) -> int:
    return {"bf16": 2, "fp32": 4}[dtype]
