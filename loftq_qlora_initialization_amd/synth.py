"""Seeded synthetic inputs for the LoftQ initialisation workloads.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic (no quantization, no codebook, no SVD).  Both the HIP path's
tests/benchmark and the CPU oracle's tests read their inputs from here, so the
two sides always see identical bytes.

Workloads (shapes are the LoRA target modules of a 7B-class decoder, the
attention/FFN projections named in "LoftQ：协同优化量化与LoRA，实现高效大语言模型微调"
§3.2; values are Gaussian because NF4 assumes normally distributed weights,
"QLoRA: Efficient Finetuning of Quantized LLMs" summary, NF4 bullet):

  c1  256x256 fp32, 0.02*N(0,1), seed 0; no double quant; r=4; T=1; exact SVD
  c2  4096x4096 bf16, 0.02*N(0,1) with 0.1% of entries replaced by 0.1*t(3);
      double quant; r=16; T=5; p=8; q=2
  c3  11008x4096 bf16, 0.02*N(0,1) rows scaled by exp(U[ln .5, ln 2]);
      double quant; r=64; T=5; p=16; q=2
  c4  224 matrices of a 32-layer decoder (q,k,v,o 4096x4096; gate,up 11008x4096;
      down 4096x11008), 0.02*N(0,1) with 0.1% 0.1*t(3) outliers, seed 4000+i;
      double quant; r=16; T=5; p=8; q=2
  c5  8192x28672 bf16, 0.015*N(0,1) plus a planted rank-32 term U diag(s) V^T,
      s = linspace(0.5, 0.05, 32), U and V Haar-orthonormal; double quant;
      r=64; T=5; p=16; q=3

Every component draws from its own child stream of ``SeedSequence(seed)`` so that
chunked generation (row panels) reproduces the same bytes as one big draw.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "workload", "c4_matrix_specs", "make_weight",
    "f32_to_bf16_bits", "bf16_bits_to_f32", "random_factors", "random_residual", "spectral_matrix",
    "tiny_scale_blocks",
]

LORA_SEED = 42  # loftq_config default seed printed on the LoftQ blog (§3.2)
_ROW_CHUNK = 1024


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    rows: int
    cols: int
    dtype: str            # "f32" or "bf16": storage type of W
    rank: int
    iterative_steps: int
    double_quant: bool
    oversample: int
    power_iters: int
    exact_svd: bool
    seed: int             # matrix seed
    kind: str             # generator recipe
    std: float = 0.02
    sketch_seed: int = LORA_SEED

    @property
    def numel(self) -> int:
        return self.rows * self.cols


WORKLOADS = {
    "c1": Workload("c1_256x256_f32", 256, 256, "f32", 4, 1, False, 0, 0, True, 0, "gauss"),
    "c2": Workload("c2_4096x4096_bf16", 4096, 4096, "bf16", 16, 5, True, 8, 2, False, 2, "outliers"),
    "c3": Workload("c3_11008x4096_bf16", 11008, 4096, "bf16", 64, 5, True, 16, 2, False, 3, "row_scaled"),
    "c5": Workload("c5_8192x28672_bf16", 8192, 28672, "bf16", 64, 5, True, 16, 3, False, 5, "planted",
                   std=0.015),
}


def workload(key: str) -> Workload:
    return WORKLOADS[key]


def c4_matrix_specs() -> List[Workload]:
    """The 224 matrices of c4, index i = 7*layer + slot (q,k,v,o,gate,up,down)."""
    shapes = [(4096, 4096)] * 4 + [(11008, 4096)] * 2 + [(4096, 11008)]
    names = ["q", "k", "v", "o", "gate", "up", "down"]
    out = []
    for layer in range(32):
        for slot in range(7):
            i = 7 * layer + slot
            r, c = shapes[slot]
            out.append(Workload(f"c4_l{layer}_{names[slot]}_{r}x{c}_bf16", r, c, "bf16", 16, 5, True,
                                8, 2, False, 4000 + i, "outliers"))
    return out


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (round to nearest even); returns the uint16 bit patterns.
    Inputs here are finite, so no NaN handling is needed."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    # finite values stay below 0xFF800000, so the 32-bit sum cannot wrap
    u = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return u.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _haar(rng: np.random.Generator, n: int, m: int) -> np.ndarray:
    g = rng.standard_normal((n, m))
    q, r = np.linalg.qr(g)
    return q * np.sign(np.diag(r))[None, :]


def make_weight(w: Workload, rows: Optional[int] = None):
    """Return (storage, values_f32) for workload ``w``.

    ``storage`` is the array handed to the device: float32 for "f32", uint16 bf16
    bit patterns for "bf16".  ``values_f32`` is the exact fp32 value of every stored
    element.  ``rows`` truncates the matrix to its first rows (same bytes as the
    full matrix's leading rows), used for oracle-sized samples.
    """
    nrows = w.rows if rows is None else min(rows, w.rows)
    ss = np.random.SeedSequence(w.seed)
    s_gauss, s_mask, s_tail, s_extra = ss.spawn(4)
    g_gauss = np.random.Generator(np.random.PCG64(s_gauss))
    g_mask = np.random.Generator(np.random.PCG64(s_mask))
    g_tail = np.random.Generator(np.random.PCG64(s_tail))
    g_extra = np.random.Generator(np.random.PCG64(s_extra))

    out32 = np.empty((nrows, w.cols), dtype=np.float32)
    if w.kind == "row_scaled":
        fac = np.exp(g_extra.uniform(np.log(0.5), np.log(2.0), size=w.rows))[:nrows]
    elif w.kind == "planted":
        k = 32
        U = _haar(g_extra, w.rows, k)[:nrows]
        V = _haar(g_extra, w.cols, k)
        s = np.linspace(0.5, 0.05, k)
        Vs = (V * s[None, :]).T.copy()  # k x cols
    for r0 in range(0, nrows, _ROW_CHUNK):
        r1 = min(nrows, r0 + _ROW_CHUNK)
        blk = w.std * g_gauss.standard_normal((r1 - r0, w.cols))
        if w.kind == "outliers":
            mask = g_mask.random((r1 - r0, w.cols)) < 0.001
            cnt = int(mask.sum())
            blk[mask] = 0.1 * g_tail.standard_t(3, size=cnt)
        elif w.kind == "row_scaled":
            blk *= fac[r0:r1, None]
        elif w.kind == "planted":
            blk += U[r0:r1] @ Vs
        out32[r0:r1] = blk.astype(np.float32)
    if w.dtype == "f32":
        return out32, out32
    bits = f32_to_bf16_bits(out32)
    return bits, bf16_bits_to_f32(bits).reshape(nrows, w.cols)


def random_factors(rows: int, cols: int, r: int, seed: int, scale: float = 0.01):
    """Random LoRA factors B (rows x r) and A (r x cols), fp32, for residual tests."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed)))
    B = (scale * g.standard_normal((rows, r))).astype(np.float32)
    A = (scale * g.standard_normal((r, cols))).astype(np.float32)
    return B, A


def random_residual(n: int, seed: int, std: float = 0.02) -> np.ndarray:
    """A flat fp32 array of n Gaussian values (a residual handed straight to the quantizer)."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed)))
    return (std * g.standard_normal(n)).astype(np.float32)


def spectral_matrix(rows: int, cols: int, sigma, seed: int, noise: float = 0.0) -> np.ndarray:
    """fp32 U diag(sigma) V^T (+ noise * N(0,1) entries): U, V Haar-orthonormal.

    ``sigma`` lists the singular values (length <= min(rows, cols)); fewer values than
    min(rows, cols) give a matrix of that rank (before the fp32 rounding and noise).
    """
    s = np.asarray(sigma, dtype=np.float64)
    ss = np.random.SeedSequence(seed)
    gu, gv, gn = (np.random.Generator(np.random.PCG64(c)) for c in ss.spawn(3))
    U = _haar(gu, rows, s.size)
    V = _haar(gv, cols, s.size)
    M = (U * s[None, :]) @ V.T
    if noise:
        M = M + noise * gn.standard_normal((rows, cols))
    return M.astype(np.float32)


def tiny_scale_blocks(scales, seed: int) -> np.ndarray:
    """Blocks of 64 fp32 values, block b drawn as scales[b] * U[-1, 1] rounded to fp32,
    with one element exactly +-scales[b] (so it is the block's absmax), a few exact
    zeros and, where representable, values a few ulps either side of scales[b] * 2^-j."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed)))
    out = np.empty((len(scales), 64), np.float32)
    for b, a in enumerate(scales):
        a = np.float32(a)
        v = (np.float64(a) * g.uniform(-1.0, 1.0, 64)).astype(np.float32)
        v[g.integers(0, 64)] = a if b % 2 == 0 else -a
        for z in g.choice(64, 3, replace=False):
            if abs(v[z]) != a:
                v[z] = 0.0
        out[b] = v
    return out.ravel()
