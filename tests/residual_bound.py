"""How far the device's block absmax of a fused residual R = base - alpha B A may lie
from the exact one.

The device forms B A on the bf16 matrix cores from split operands: x = hi + lo + err with
hi = bf16(x), lo = bf16(x - hi) and |err| <= 2^-18 |x|, accumulating hi*hi + hi*lo + lo*hi
in fp32.  Each product term is then off by at most 3.02 * 2^-18 |a b|, and the fp32
accumulation of at most 3 * 64 terms adds at most 192 * 2^-24 of their absolute sum, so
|(B A)_dev - B A| <= 2^-15 (|B| |A|) elementwise.  Forming R and taking the block
maximum add one fp32 rounding (2^-24 relative), bounded here by 2^-23.
"""
import numpy as np

C_PRODUCT = 2.0 ** -15


def block_bound(B, A, alpha=1.0):
    """Per 64-element block of the row-major rows(B) x cols(A) product: the bound on its
    absmax error coming from B A (rows(B) * cols(A) must be a multiple of 64)."""
    E = C_PRODUCT * abs(alpha) * (np.abs(B.astype(np.float64)) @ np.abs(A.astype(np.float64)))
    return E.reshape(-1, 64).max(axis=1)


def check_absmax(dev_am, exact_am, bound):
    """|dev - exact| <= bound + 2^-23 |exact| for every block."""
    d = np.abs(np.asarray(dev_am, np.float64) - np.asarray(exact_am, np.float64))
    lim = np.asarray(bound, np.float64) + 2.0 ** -23 * np.abs(np.asarray(exact_am, np.float64))
    assert np.all(d <= lim), float(np.max(d - lim))
