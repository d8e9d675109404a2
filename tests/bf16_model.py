"""A numpy model of the library's documented bf16 rounding points (float32
products rounded once to nearest-even bf16):

    X0 = bf16(M / (||M|| + eps))            (the short side first)
    A  = bf16(X X^T)
    C  = a I + b A + c A A,  C_hi = bf16(C),  C_lo = bf16(C - C_hi)
    X' = bf16((C_hi + C_lo) X)

The pages cast the iteration to bf16; this model reproduces that precision
exactly (up to the order of float32 accumulation), so a test can tell the
method's own bf16 error on an ill-conditioned matrix from a kernel fault.  It
is test code: the library does not use it and it is not the fp64 oracle."""
import numpy as np


def bf16(x) -> np.ndarray:
    """Round to bf16 (nearest, ties to even) and return as float64."""
    b = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    r = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32).astype(np.float64)


def newton_schulz_bf16(m, coeffs, steps: int, eps: float = 1e-7) -> np.ndarray:
    m = np.asarray(m, np.float64)
    tall = m.shape[0] > m.shape[1]
    x = m.T if tall else m
    x = bf16(x / (np.linalg.norm(x) + eps))
    for k in range(steps):
        a, b, c = coeffs[0] if len(coeffs) == 1 else coeffs[k]
        A = bf16(x @ x.T)
        C = a * np.eye(A.shape[0]) + b * A + c * (A @ A)
        hi = bf16(C)
        lo = bf16(C - hi)
        x = bf16((hi + lo) @ x)
    return x.T if tall else x
