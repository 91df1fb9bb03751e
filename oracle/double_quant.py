"""Double quantization of the NF4 absmax constants, written out plainly.

Test infrastructure only (see the package docstring).

The pages only say that the quantization constants are quantized a second time
to save memory per parameter ([QLoRA notes], double-quantization bullet;
[PEFT course] §4.2; [PEFT guide], bnb_4bit_use_double_quant bullet).  They give
no bit width, block size or format.

Reading (parity unpinned against any external format): the same blockwise
absmax scheme as the first level, applied at 8 bits to groups of 256
consecutive absmax values (the last group may be ragged):
    s   = fl32(max_group / 127)
    q   = clamp(rint_half_even(fl32(a / s)), 0, 127)      (s = 0  =>  q = 0)
    a'  = fl32(q * s)
The absmax values are non-negative, so the codes use 0..127 of int8.  No mean is
subtracted, so no order-dependent global sum enters the format.
"""
from __future__ import annotations

import numpy as np

__all__ = ["double_quant", "dq_scales_expand"]


def double_quant(absmax: np.ndarray, dq_blocksize: int = 256):
    """Return (qabsmax int8[nb], dq_scale fp32[ceil(nb / dq_blocksize)])."""
    a = np.asarray(absmax, dtype=np.float32).ravel()
    if not np.all(np.isfinite(a)) or np.any(a < 0):
        raise ValueError("absmax must be finite and non-negative")
    nb = a.size
    ng = -(-nb // dq_blocksize)
    q = np.zeros(nb, dtype=np.int8)
    s = np.zeros(ng, dtype=np.float32)
    for g in range(ng):
        lo, hi = g * dq_blocksize, min(nb, (g + 1) * dq_blocksize)
        blk = a[lo:hi].astype(np.float64)
        sg = np.float32(blk.max() / 127.0)
        s[g] = sg
        if sg == 0:
            continue
        x = (blk / np.float64(sg)).astype(np.float32).astype(np.float64)
        q[lo:hi] = np.clip(np.rint(x), 0, 127).astype(np.int8)
    return q, s


def dq_scales_expand(qabsmax: np.ndarray, dq_scale: np.ndarray, dq_blocksize: int = 256) -> np.ndarray:
    """Reconstructed absmax a' = fl32(q * s) for every first-level block."""
    q = np.asarray(qabsmax, dtype=np.int8).ravel().astype(np.float64)
    s = np.repeat(np.asarray(dq_scale, dtype=np.float32), dq_blocksize)[:q.size].astype(np.float64)
    return (q * s).astype(np.float32)
