"""LoftQ's alternating minimisation of ||W - (Q + BA)||_F, step by step.

Test infrastructure only (see the package docstring).

The pages ([LoftQ blog] §2.2-2.3, §3.2; [PEFT guide] "LoftQ 初始化"):
  * objective: min over Q and a rank-r Delta = BA of ||W - (Q + Delta)||_F^2;
  * quantization step: with Delta fixed, quantize the residual W - Delta
    (round-to-nearest);
  * low-rank step: with Q fixed, Delta = best rank-r approximation of W - Q;
  * alternate a preset number of times (iterative_steps, default 5);
  * the one-step variant (replace_lora_weights_loftq) is a single alternation
    that keeps NF4(W) as the base and only refits the LoRA weights.

Readings:
  * Delta_0 = 0, so alternation 1 quantizes W itself; T = 0 is plain NF4 QLoRA
    (B = A = 0).
  * Q is NF4 with blockwise-64 absmax; with double quant on, the codes are chosen
    with the fp32 absmax and Q is reconstructed with the double-quantized a'.
  * The residual W - B A is formed in fp64 and rounded once to fp32 before
    quantization.
  * objective[0] = ||W - Q_1|| / ||W|| (plain NF4 error); objective[t] =
    ||W - Q_t - B_t A_t|| / ||W|| for t = 1..T, each computed directly.
  * Resume ([LoftQ blog] §2.3: the initialisation is computed once and its
    result kept): a run may start from the factors (B_k, A_k) of k completed
    alternations instead of Delta_0 = 0 and carry on with alternations
    k+1 .. k+T, the sketch counter continuing at k+1, so that k alternations
    followed by T resumed ones take the same steps as k+T alternations in one
    run.  objective[0] is then ||W - Q_{k+1}|| / ||W||, the error of the run's
    first quantization alone (for k = 0 the plain NF4 error above).
"""
from __future__ import annotations

import numpy as np

from .nf4 import quantize_residual, dequantize, nf_codebook
from .double_quant import double_quant, dq_scales_expand
from .rng import rademacher_sketch
from .lowrank import exact_svd, randomized_svd, lora_factors

__all__ = ["loftq_step", "loftq_init", "objective", "warm_sketch"]


def warm_sketch(V_prev: np.ndarray, seed: int, t: int, k: int, l: int) -> np.ndarray:
    """Sketch of a warm-started alternation t >= 2: [sqrt(k) V_{t-1} | the last l - r
    columns of the +-1 sketch of (seed, t)], k x l.

    A performance variant the pages do not describe (subspace iteration started
    from the previous alternation's right singular vectors, so fewer power
    iterations reach the same accuracy); the V columns are scaled to the norm of
    a +-1 column.  Only the span of E Omega matters to the randomized SVD, so the
    signs of V's columns are immaterial.
    """
    om = rademacher_sketch(seed, t, k, l)
    r = V_prev.shape[1]
    om[:, :r] = np.sqrt(float(k)) * np.asarray(V_prev, dtype=np.float64)
    return om


def _residual(W32: np.ndarray, B, A) -> np.ndarray:
    if B is None:
        return np.asarray(W32, dtype=np.float32)
    prod = np.asarray(B, dtype=np.float64) @ np.asarray(A, dtype=np.float64)
    return (np.asarray(W32, dtype=np.float64) - prod).astype(np.float32)


def loftq_step(W32: np.ndarray, B_prev, A_prev, *, rank: int, t: int = 1, blocksize: int = 64,
               double_quant_on: bool = True, dq_blocksize: int = 256, exact: bool = False,
               oversample: int = 8, power_iters: int = 2, seed: int = 42, omega=None, bits: int = 4) -> dict:
    """One alternation: Q_t = NF_bits(W - B_prev A_prev), then (B_t, A_t) = SVD_r(W - deq Q_t)."""
    W32 = np.asarray(W32, dtype=np.float32)
    d, k = W32.shape
    cb = nf_codebook(bits)
    R = _residual(W32, B_prev, A_prev)
    codes, absmax = quantize_residual(R.ravel(), blocksize, cb)
    out = dict(R=R, codes=codes, absmax=absmax)
    if double_quant_on:
        qa, s = double_quant(absmax, dq_blocksize)
        scale = dq_scales_expand(qa, s, dq_blocksize)
        out.update(qabsmax=qa, dq_scale=s)
    else:
        scale = absmax
    out["scale"] = scale
    E = dequantize(codes, scale, blocksize, W=W32.ravel(), codebook=cb).reshape(d, k)
    out["E"] = E
    out["E_sumsq"] = float(np.sum(E.astype(np.float64) ** 2))
    if exact:
        U, s_r, V = exact_svd(E, rank)
    else:
        l = rank + oversample
        if omega is None:
            omega = rademacher_sketch(seed, t, k, l)
        U, s_r, V = randomized_svd(E, rank, omega, power_iters)
        out["omega"] = omega
    B, A = lora_factors(U, s_r, V)
    out.update(B=B, A=A, sigma=s_r, U=U, V=V)
    return out


def objective(W32: np.ndarray, codes: np.ndarray, scale: np.ndarray, B, A, blocksize: int = 64,
              bits: int = 4) -> float:
    """||W - deq(Q) - BA||_F / ||W||_F in fp64."""
    W = np.asarray(W32, dtype=np.float64)
    deq = dequantize(codes, scale, blocksize, codebook=nf_codebook(bits)).astype(np.float64).reshape(W.shape)
    res = W - deq
    if B is not None:
        res = res - np.asarray(B, dtype=np.float64) @ np.asarray(A, dtype=np.float64)
    return float(np.sqrt(np.sum(res * res)) / np.sqrt(np.sum(W * W)))


def loftq_init(W32: np.ndarray, *, rank: int, iterative_steps: int = 5, blocksize: int = 64,
               double_quant_on: bool = True, dq_blocksize: int = 256, exact: bool = False,
               oversample: int = 8, power_iters: int = 2, seed: int = 42, keep_steps: bool = False,
               warm_start: bool = False, bits: int = 4, resume_from: int = 0, init_B=None, init_A=None,
               init_sigma=None) -> dict:
    """The whole initialisation: T alternations from Delta_0 = 0, objective per alternation.

    warm_start: alternations t >= 2 of the randomized SVD use warm_sketch(V_{t-1}, ...)
    instead of the fresh sketch of (seed, t) (a variant; off reproduces the pages' method).
    resume_from = k >= 1: start from init_B, init_A (B_k, A_k; with warm_start also
    init_sigma = sigma_k) and run alternations k+1 .. k+T.
    """
    W32 = np.asarray(W32, dtype=np.float32)
    d, k = W32.shape
    T = int(iterative_steps)
    k0 = int(resume_from)
    if k0 < 0 or (k0 > 0 and (init_B is None or init_A is None or T == 0)):
        raise ValueError("resume needs k >= 1, B_k, A_k and T >= 1")
    kw = dict(rank=rank, blocksize=blocksize, double_quant_on=double_quant_on, dq_blocksize=dq_blocksize, bits=bits,
              exact=exact, oversample=oversample, power_iters=power_iters, seed=seed)
    obj = np.zeros(T + 1)
    steps = []
    B = A = None
    last = None
    if k0 > 0:
        B, A = np.asarray(init_B), np.asarray(init_A)
        if warm_start and not exact:
            if init_sigma is None:
                raise ValueError("a warm-started resume needs sigma_k")
            # A_k = diag(sqrt sigma) V^T  =>  V = A_k^T diag(sigma^-1/2)
            sg = np.asarray(init_sigma, dtype=np.float64)
            last = dict(V=np.asarray(A, dtype=np.float64).T / np.sqrt(sg)[None, :])
    if T == 0:
        codes, absmax = quantize_residual(W32.ravel(), blocksize, nf_codebook(bits))
        res = dict(codes=codes, absmax=absmax)
        if double_quant_on:
            qa, s = double_quant(absmax, dq_blocksize)
            res.update(qabsmax=qa, dq_scale=s)
            scale = dq_scales_expand(qa, s, dq_blocksize)
        else:
            scale = absmax
        obj[0] = objective(W32, codes, scale, None, None, blocksize, bits)
        res.update(B=np.zeros((d, rank)), A=np.zeros((rank, k)), sigma=np.zeros(rank), objective=obj)
        return res
    for t in range(1, T + 1):
        om = None
        if warm_start and not exact and last is not None:
            om = warm_sketch(last["V"], seed, k0 + t, k, rank + oversample)
        st = loftq_step(W32, B, A, t=k0 + t, omega=om, **kw)
        if t == 1:
            obj[0] = objective(W32, st["codes"], st["scale"], None, None, blocksize, bits)
        obj[t] = objective(W32, st["codes"], st["scale"], st["B"], st["A"], blocksize, bits)
        B, A = st["B"], st["A"]
        last = st
        if keep_steps:
            steps.append(st)
    res = {key: last[key] for key in ("codes", "absmax", "B", "A", "sigma", "scale")}
    if double_quant_on:
        res.update(qabsmax=last["qabsmax"], dq_scale=last["dq_scale"])
    res["objective"] = obj
    if keep_steps:
        res["steps"] = steps
    return res
