"""NF4 (4-bit NormalFloat) blockwise quantization, written out plainly.

Test infrastructure only (see the package docstring).

What the pages fix:
  * NF4 is a quantile quantizer: its levels come from the quantile function
    (inverse CDF) of the standard normal, which makes it information-theoretically
    optimal for normally distributed weights ([QLoRA notes], NF4 bullet; related
    blurb on quantile quantization; [PEFT guide] BitsAndBytesConfig bullets).
  * The printed codebook starts -1.0, -0.6962, -0.5251 and ends at 1.0
    ([QLoRA blog] §2.1 sample code).
  * Quantizing = divide by the absmax so values lie in [-1, 1], then take the
    nearest codebook entry by argmin of the distance ([QLoRA blog] §2.1).
  * A CUDA-matching re-implementation compares against the midpoints of the NF4
    table ([QLoRA notes], related blurb "NF4量化算法的PyTorch实现").

Readings where the pages are silent or garbled:
  * Codebook construction: 8 positive levels Phi^-1 of 9 evenly spaced
    probabilities from delta to 1/2 (the last, 1/2, dropped), 7 negative levels
    -Phi^-1 of 8 evenly spaced probabilities from delta to 1/2 (last dropped), an
    exact zero, normalised by the largest magnitude.  delta = 1 - (1/32 + 1/30)/2.
    The two printed interior values (-0.6962, -0.5251) only hold for delta in a
    narrow window around 0.9677 (pinned in the tests); this delta lies inside.
  * Absmax blocks are 64 consecutive elements of the row-major flattening; a
    ragged last block takes the remaining elements.
  * x = fl32(R / a) in IEEE fp32; a block with a = 0 encodes every element as the
    exact-zero code (no 0/0).
  * Ties (x exactly at a midpoint) go to the lower code (argmin keeps the first).
  * Two codes per byte, element 2i in the high nibble.
  * Lower-bit NormalFloat (k = 2, 3 bits; [LoftQ blog] reports 2- and 3-bit
    LoftQ but gives no codebook): the same construction with 2^(k-1) positive
    and 2^(k-1) - 1 negative quantile levels and
    delta_k = 1 - (1/2^(k+1) + 1/(2 (2^k - 1)))/2, which is delta at k = 4.
    A k-bit code is stored in a nibble like an NF4 code.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = ["DELTA", "nf_delta", "norm_ppf", "nf4_codebook", "nf_codebook", "nf4_midpoints", "block_absmax",
           "nf4_encode", "pack_nibbles", "unpack_nibbles", "dequantize", "quantize_residual"]

DELTA = 1.0 - 0.5 * (1.0 / 32.0 + 1.0 / 30.0)


def nf_delta(bits: int) -> float:
    """delta_k = 1 - (1/2^(k+1) + 1/(2 (2^k - 1))) / 2 (= DELTA at k = 4)."""
    return 1.0 - 0.5 * (1.0 / 2.0 ** (bits + 1) + 1.0 / (2.0 * (2.0 ** bits - 1.0)))


def _phi(x: float) -> float:
    """Standard normal CDF, Phi(x) = erfc(-x / sqrt 2) / 2."""
    return 0.5 * math.erfc(-x / math.sqrt(2.0))


def norm_ppf(p: float) -> float:
    """Quantile function Phi^-1(p) of the standard normal, by bisection on Phi.

    Bisection runs until the bracket cannot shrink in fp64, then returns the
    bracket end whose CDF is closer to p.
    """
    if not (0.0 < p < 1.0):
        raise ValueError("p must lie in (0, 1)")
    if p == 0.5:
        return 0.0
    if p < 0.5:
        return -norm_ppf(1.0 - p)
    lo, hi = 0.0, 40.0
    while True:
        mid = 0.5 * (lo + hi)
        if mid <= lo or mid >= hi:
            break
        if _phi(mid) < p:
            lo = mid
        else:
            hi = mid
    return lo if abs(_phi(lo) - p) <= abs(_phi(hi) - p) else hi


def nf4_codebook(delta: float = DELTA) -> np.ndarray:
    """The 16 NF4 levels, ascending, as fp32 (index 0 = -1, index 7 = 0, index 15 = +1)."""
    return _normal_float_levels(8, 7, delta)


def nf_codebook(bits: int = 4) -> np.ndarray:
    """The 2^bits k-bit NormalFloat levels, ascending, fp32 (bits = 2, 3 or 4; 4 is NF4)."""
    if bits not in (2, 3, 4):
        raise ValueError("bits must be 2, 3 or 4")
    half = 2 ** (bits - 1)
    return _normal_float_levels(half, half - 1, nf_delta(bits))


def _normal_float_levels(npos: int, nneg: int, delta: float) -> np.ndarray:
    """npos levels Phi^-1 of npos + 1 evenly spaced probabilities from delta to 1/2
    (1/2 dropped), nneg levels -Phi^-1 of nneg + 1 such probabilities (1/2 dropped),
    an exact zero; normalised by the largest magnitude; ascending fp32."""
    pos_p = np.linspace(delta, 0.5, npos + 1)[:-1]
    neg_p = np.linspace(delta, 0.5, nneg + 1)[:-1]
    levels = [norm_ppf(float(p)) for p in pos_p] + [-norm_ppf(float(p)) for p in neg_p] + [0.0]
    v = np.array(sorted(levels), dtype=np.float64)
    v = v / np.max(np.abs(v))
    return v.astype(np.float32)


def nf4_midpoints(codebook: np.ndarray | None = None) -> np.ndarray:
    """Exact fp64 midpoints between neighbouring fp32 levels (15 values)."""
    c = (nf4_codebook() if codebook is None else codebook).astype(np.float64)
    return 0.5 * (c[:-1] + c[1:])


def _check_finite(x: np.ndarray) -> None:
    if not np.all(np.isfinite(x)):
        raise ValueError("NF4 input must be finite")


def block_absmax(R: np.ndarray, blocksize: int = 64) -> np.ndarray:
    """a_b = max |R| over each block of ``blocksize`` consecutive elements (fp32, exact)."""
    r = np.ascontiguousarray(R, dtype=np.float32).ravel()
    _check_finite(r)
    n = r.size
    nb = -(-n // blocksize)
    pad = np.zeros(nb * blocksize, dtype=np.float32)
    pad[:n] = np.abs(r)
    return pad.reshape(nb, blocksize).max(axis=1) if nb else np.zeros(0, np.float32)


def nf4_encode(R: np.ndarray, absmax: np.ndarray, blocksize: int = 64,
               codebook: np.ndarray | None = None, chunk: int = 1 << 20) -> np.ndarray:
    """Nearest-level NF4 code of every element: argmin_j |c_j - fl32(R / a)|, first on ties."""
    c = (nf4_codebook() if codebook is None else codebook).astype(np.float64)
    r = np.ascontiguousarray(R, dtype=np.float32).ravel()
    _check_finite(r)
    n = r.size
    a = np.repeat(np.asarray(absmax, dtype=np.float32), blocksize)[:n]
    codes = np.empty(n, dtype=np.uint8)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        rs = r[s:e].astype(np.float64)
        asb = a[s:e].astype(np.float64)
        safe = np.where(asb > 0, asb, 1.0)
        x = np.where(asb > 0, rs / safe, 0.0).astype(np.float32).astype(np.float64)
        dist = np.abs(c[None, :] - x[:, None])
        codes[s:e] = np.argmin(dist, axis=1).astype(np.uint8)
    return codes


def quantize_residual(R: np.ndarray, blocksize: int = 64, codebook: np.ndarray | None = None):
    """(codes, absmax) of an fp32 residual: blockwise absmax then nearest-level encode."""
    am = block_absmax(R, blocksize)
    return nf4_encode(R, am, blocksize, codebook), am


def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """Two 4-bit codes per byte, element 2i in the high nibble; odd length pads a zero nibble."""
    c = np.asarray(codes, dtype=np.uint8).ravel()
    if c.size % 2:
        c = np.concatenate([c, np.zeros(1, np.uint8)])
    return ((c[0::2] << 4) | c[1::2]).astype(np.uint8)


def unpack_nibbles(packed: np.ndarray, n: int) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8).ravel()
    out = np.empty(2 * p.size, dtype=np.uint8)
    out[0::2] = p >> 4
    out[1::2] = p & 0xF
    return out[:n]


def dequantize(codes: np.ndarray, scale: np.ndarray, blocksize: int = 64,
               W: np.ndarray | None = None, codebook: np.ndarray | None = None) -> np.ndarray:
    """deq = fl32(c[code] * a') per element; with W given, returns E = fl32(W - deq).

    ``scale`` holds one fp32 a' per block (the absmax, or its double-quantized
    reconstruction).  Each product and difference is one correctly rounded fp32
    operation (computed exactly in fp64, then rounded once).
    """
    c = (nf4_codebook() if codebook is None else codebook).astype(np.float64)
    code = np.asarray(codes, dtype=np.uint8).ravel()
    n = code.size
    a = np.repeat(np.asarray(scale, dtype=np.float32), blocksize)[:n].astype(np.float64)
    deq = (c[code] * a).astype(np.float32)
    if W is None:
        return deq
    w = np.ascontiguousarray(W, dtype=np.float32).ravel().astype(np.float64)
    return (w - deq.astype(np.float64)).astype(np.float32)
