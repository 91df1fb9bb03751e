"""Merging a LoRA adapter into NF4 weights and taking it out again.

Test infrastructure only (see the package docstring).

[PEFT guide] "量化", section on merging adapters into quantized weights:
merge_adapter() dequantizes the base weight, adds the adapter's weight and
quantizes the sum again; unmerge_adapter() does the reverse (dequantize,
subtract the adapter, quantize again), so it does not give back the original
quantized weight, and repeated merge/unmerge cycles accumulate rounding.

Readings:
  * The adapter's weight is alpha * B A (B rows x r, A r x cols); alpha stands
    for whatever scaling the caller applies (1.0 for the factors LoftQ returns,
    which carry no alpha / r factor).
  * The sum deq(Q) +- alpha B A is formed in fp64 (the product too) and rounded
    once to fp32, the same reading as the residual of the alternation; it is then
    quantized exactly like any residual: blockwise-64 absmax, nearest NF4 level
    (ties to the lower index), and with double quant the new absmax values are
    double-quantized again.
  * Unmerge is merge with -alpha.
"""
from __future__ import annotations

import numpy as np

from .nf4 import quantize_residual, dequantize
from .double_quant import double_quant

__all__ = ["merge_adapter", "unmerge_adapter"]


def merge_adapter(codes: np.ndarray, scale: np.ndarray, B, A, alpha: float = 1.0, *, double_quant_on: bool = True,
                  blocksize: int = 64, dq_blocksize: int = 256) -> dict:
    """Q' = NF4(deq(Q) + alpha B A).

    ``codes``: one NF4 code per element (row-major); ``scale``: one fp32 dequant
    scale per block (the absmax, or its double-quantized reconstruction a').
    B, A may both be None (no adapter: Q is only requantized).  Returns the new
    codes and absmax, and qabsmax / dq_scale when double_quant_on.
    """
    D = dequantize(codes, scale, blocksize).astype(np.float64)
    if B is None:
        R = D.astype(np.float32)
    else:
        prod = (np.asarray(B, dtype=np.float64) @ np.asarray(A, dtype=np.float64)).ravel()
        R = (D + alpha * prod).astype(np.float32)
    new_codes, absmax = quantize_residual(R, blocksize)
    out = dict(R=R, codes=new_codes, absmax=absmax)
    if double_quant_on:
        qa, s = double_quant(absmax, dq_blocksize)
        out.update(qabsmax=qa, dq_scale=s)
    return out


def unmerge_adapter(codes: np.ndarray, scale: np.ndarray, B, A, alpha: float = 1.0, **kw) -> dict:
    """Q'' = NF4(deq(Q') - alpha B A): the reverse step, not an exact inverse."""
    return merge_adapter(codes, scale, B, A, -alpha, **kw)
