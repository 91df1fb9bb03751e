"""The low-rank step: best rank-r approximation of the quantization residual.

Test infrastructure only (see the package docstring).

The pages: with Q fixed, the optimal rank-r Delta is the truncated SVD of W - Q,
Delta = U_r Sigma_r V_r^T built from the r largest singular values and their
singular vectors ([LoftQ blog] §2.3, low-rank factorization step).  LoRA writes
Delta = BA with B in R^{d x r}, A in R^{r x k} ([PEFT course] §2.2).

Readings:
  * Exact mode computes the SVD itself: one-sided (Hestenes) Jacobi in fp64,
    cyclic pair order, LAPACK-free.
  * Randomized mode (the large workloads) follows the randomized subspace
    iteration of Halko, Martinsson and Tropp ("Finding structure with
    randomness", SIAM Review 2011, Algorithms 4.4 and 5.1): Y = E Omega, q rounds
    of orthonormalise / multiply by E^T / orthonormalise / multiply by E, then
    C = E^T Q (so B_small = C^T = Q^T E), and the SVD of B_small through a QR of C
    and a Jacobi SVD of its l x l triangular factor.
  * B = U_r Sigma_r^{1/2}, A = Sigma_r^{1/2} V_r^T; no lora_alpha / r scaling.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = ["householder_qr", "jacobi_svd", "randomized_svd", "exact_svd", "lora_factors"]


def householder_qr(Y: np.ndarray):
    """Thin QR by Householder reflections: Y (m x n, m >= n) = Q (m x n) R (n x n)."""
    A = np.array(Y, dtype=np.float64, copy=True)
    m, n = A.shape
    if m < n:
        raise ValueError("householder_qr needs rows >= cols")
    vs = []
    for j in range(n):
        x = A[j:, j]
        nx = math.sqrt(float(x @ x))
        alpha = -nx if x[0] >= 0 else nx
        v = x.copy()
        v[0] -= alpha
        vv = float(v @ v)
        if vv > 0.0:
            v /= math.sqrt(vv)
            A[j:, j:] -= 2.0 * np.outer(v, v @ A[j:, j:])
        else:
            v[:] = 0.0
        vs.append(v)
    R = np.triu(A[:n, :n])
    Q = np.zeros((m, n))
    Q[:n, :n] = np.eye(n)
    for j in reversed(range(n)):
        v = vs[j]
        Q[j:, :] -= 2.0 * np.outer(v, v @ Q[j:, :])
    return Q, R


def jacobi_svd(M: np.ndarray, tol: float = 1e-14, max_sweeps: int = 60):
    """One-sided Jacobi SVD of M (m x n, m >= n): M = U diag(s) V^T, s descending.

    Columns p < q are rotated in cyclic-by-row order until every pair is
    orthogonal to ``tol`` relative to the product of their norms.
    """
    A = np.array(M, dtype=np.float64, copy=True)
    m, n = A.shape
    if m < n:
        raise ValueError("jacobi_svd needs rows >= cols; pass the transpose")
    V = np.eye(n)
    for _ in range(max_sweeps):
        rotated = False
        for p in range(n - 1):
            for q in range(p + 1, n):
                ap, aq = A[:, p], A[:, q]
                alpha = float(ap @ ap)
                beta = float(aq @ aq)
                gamma = float(ap @ aq)
                if gamma == 0.0 or abs(gamma) <= tol * math.sqrt(alpha * beta):
                    continue
                rotated = True
                zeta = (beta - alpha) / (2.0 * gamma)
                t = (1.0 if zeta >= 0 else -1.0) / (abs(zeta) + math.sqrt(1.0 + zeta * zeta))
                c = 1.0 / math.sqrt(1.0 + t * t)
                s = c * t
                new_p = c * ap - s * aq
                new_q = s * ap + c * aq
                A[:, p], A[:, q] = new_p, new_q
                vp, vq = V[:, p].copy(), V[:, q].copy()
                V[:, p] = c * vp - s * vq
                V[:, q] = s * vp + c * vq
        if not rotated:
            break
    s = np.sqrt(np.sum(A * A, axis=0))
    order = np.argsort(-s, kind="stable")
    s = s[order]
    A = A[:, order]
    V = V[:, order]
    U = np.zeros_like(A)
    nz = s > 0
    U[:, nz] = A[:, nz] / s[nz]
    return U, s, V


def exact_svd(E: np.ndarray, r: int):
    """Top-r singular triplets of E by the full Jacobi SVD: (U_r, s_r, V_r)."""
    E = np.asarray(E, dtype=np.float64)
    d, k = E.shape
    if d >= k:
        U, s, V = jacobi_svd(E)
    else:
        V, s, U = jacobi_svd(E.T)
    return U[:, :r], s[:r], V[:, :r]


def randomized_svd(E: np.ndarray, r: int, omega: np.ndarray, q: int):
    """Top-r triplets from randomized subspace iteration with sketch ``omega`` (k x l)."""
    E = np.asarray(E, dtype=np.float64)
    omega = np.asarray(omega, dtype=np.float64)
    d, k = E.shape
    l = omega.shape[1]
    if omega.shape[0] != k or not (r <= l <= min(d, k)):
        raise ValueError("sketch must be k x l with r <= l <= min(d, k)")
    Q, _ = householder_qr(E @ omega)
    for _ in range(q):
        Z, _ = householder_qr(E.T @ Q)
        Q, _ = householder_qr(E @ Z)
    C = E.T @ Q                       # k x l, the transpose of Q^T E
    Qc, Rc = householder_qr(C)        # C = Qc Rc
    Ur, s, Vr = jacobi_svd(Rc)        # Rc = Ur diag(s) Vr^T
    # Q^T E = C^T = Vr diag(s) (Qc Ur)^T  =>  E ~ (Q Vr) diag(s) (Qc Ur)^T
    U = Q @ Vr[:, :r]
    V = Qc @ Ur[:, :r]
    return U, s[:r], V


def lora_factors(U: np.ndarray, s: np.ndarray, V: np.ndarray):
    """B = U diag(sqrt s), A = diag(sqrt s) V^T."""
    rs = np.sqrt(np.asarray(s, dtype=np.float64))
    return U * rs[None, :], (V * rs[None, :]).T
