"""The QLoRA forward pass of one adapted layer (the consumer of LoftQ's Q, B, A).

Test infrastructure only (see the package docstring).

The pages: [PEFT course] §2.2, the LoRA output adds to the frozen weight's,
h = W x + B A x; §4.3, QLoRA runs its 4-bit base with compute dtype bfloat16
(bnb_4bit_compute_dtype); [QLoRA notes], NF4 weights with double-quantized scales.

Readings:
  * Tokens are rows: Y (n x rows) = X (n x cols) W^T + alpha (X A^T) B^T, with
    W = deq(Q) (rows x cols), B rows x r, A r x cols (LoftQ's factors), alpha the
    caller's LoRA scaling.
  * bfloat16 compute: X is given in bf16; deq(Q) is formed exactly in fp32 (as in
    the dequantization) and rounded to bf16; A and B are rounded to bf16; every
    product accumulates in fp32 (here: fp64); the intermediate X A^T and the
    output Y stay in fp32.  Rounding to bf16 is round-to-nearest-even.
"""
from __future__ import annotations

import numpy as np

from .nf4 import dequantize, nf_codebook

__all__ = ["bf16_round", "qlora_forward"]


def bf16_round(x: np.ndarray) -> np.ndarray:
    """fp32 -> nearest bf16 (ties to even), returned as fp32 values.

    bf16 keeps the top 16 bits of an fp32; the rounding adds 0x7FFF plus the
    lowest kept bit before truncating.  Inputs must be finite.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)) << np.uint64(16)
    return (r & np.uint64(0xFFFFFFFF)).astype(np.uint32).view(np.float32).reshape(np.shape(x))


def qlora_forward(X: np.ndarray, codes: np.ndarray, scale: np.ndarray, rows: int, cols: int, B=None, A=None,
                  alpha: float = 1.0, bits: int = 4, blocksize: int = 64) -> np.ndarray:
    """Y = X bf16(deq(Q))^T + alpha (X bf16(A)^T) bf16(B)^T in fp64 (X already bf16 values)."""
    W = dequantize(codes, scale, blocksize, codebook=nf_codebook(bits)).reshape(rows, cols)
    Xb = np.asarray(X, dtype=np.float64)
    Y = Xb @ bf16_round(W).astype(np.float64).T
    if B is not None:
        T = Xb @ bf16_round(np.asarray(A, np.float32)).astype(np.float64).T
        Y = Y + alpha * (T @ bf16_round(np.asarray(B, np.float32)).astype(np.float64).T)
    return Y
