"""Plain CPU oracle for LoftQ initialisation (NF4 + double quant + rank-r SVD).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call, link
or execute anything in this package; only the test suite, the smoke check in
``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` use it.  It shares
no code, tables or constants with the HIP library.

The oracle is written for obviousness, not speed: fp64 numpy throughout except
where a step is defined in fp32, an explicit argmin for nearest-code rounding,
LAPACK-free Householder QR and one-sided Jacobi SVD.

Pages cited (their titles; sections as printed on each page):
  [LoftQ blog]   "LoftQ：协同优化量化与LoRA，实现高效大语言模型微调"
  [QLoRA blog]   "QLoRA技术解析：量化与低秩适配在LLM微调中的突破"
  [PEFT course]  "参数高效微调：LoRA、Adapter 与 QLoRA"
  [QLoRA notes]  "QLoRA论文概述" (summary of "QLORA: Efficient Finetuning of Quantized LLMs")
  [PEFT guide]   "量化" (PEFT developer guide, quantization)

Parity status of each function (pins live in tests/test_oracle_*.py):
  nf4_codebook            pinned (printed values, exact zero, quantile definition)
  nf_codebook (2, 3 bits) pinned (reduces to NF4 at 4 bits; the 2-bit levels in
                          closed form from library normal quantiles)
  nf4_encode              pinned (round trip, midpoint transitions, ties, monotone)
  absmax / pack / unpack  pinned (closed forms, hand-computed fixture)
  double_quant            parity unpinned against any external format (the pages
                          give no format); pinned only by its own invariants
  dequantize              pinned (exact round trip of codebook multiples)
  householder_qr          pinned (Q^T Q = I, QR = Y, triangular; LAPACK check)
  jacobi_svd              pinned (Eckart-Young vs LAPACK and brute force)
  randomized_svd          pinned (reduces to the exact SVD when l = min(d, k))
  rademacher_sketch       pinned (SplitMix64 published first output)
  loftq_init              pinned (T=0 = plain NF4 error; objective identity)
  merge / unmerge_adapter pinned (zero adapter requantizes to the same codes,
                          doubling and cancelling closed forms, hand-worked block)
  bf16_round              pinned (hand values, ties to even, torch's own conversion)
  qlora_forward           pinned (bf16-exact weights give X W^T + alpha X A^T B^T computed
                          directly; linear in X)
  warm_sketch             pinned (T = 1 reduces to the cold start; a warm sketch
                          spanning a rank-r E's row space recovers the exact SVD
                          with no power iteration)
"""
from .nf4 import (nf4_codebook, nf_codebook, nf_delta, norm_ppf, nf4_midpoints, block_absmax, nf4_encode,
                  pack_nibbles, unpack_nibbles, dequantize, quantize_residual)
from .double_quant import double_quant, dq_scales_expand
from .rng import splitmix64_stream, rademacher_sketch
from .lowrank import householder_qr, jacobi_svd, randomized_svd, exact_svd, lora_factors
from .loftq import loftq_step, loftq_init, objective, warm_sketch
from .merge import merge_adapter, unmerge_adapter
from .forward import bf16_round, qlora_forward

__all__ = [
    "nf4_codebook", "nf_codebook", "nf_delta", "norm_ppf", "nf4_midpoints", "block_absmax", "nf4_encode", "pack_nibbles",
    "unpack_nibbles", "dequantize", "quantize_residual", "double_quant", "dq_scales_expand",
    "splitmix64_stream", "rademacher_sketch", "householder_qr", "jacobi_svd", "randomized_svd",
    "exact_svd", "lora_factors", "loftq_step", "loftq_init", "objective", "merge_adapter", "unmerge_adapter", "warm_sketch", "bf16_round", "qlora_forward",
]
