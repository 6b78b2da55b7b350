"""fp64 CPU oracle for the offline per-head factorisation.

TEST INFRASTRUCTURE ONLY (like the rest of this package): only the test
suite, the package smoke check and the benchmark's CPU-baseline leg may
import or run it; the GPU library never calls it and shares no code with
it.

The pages ("WSVD: Weighted Low-Rank Approximation for Fast and Efficient
Execution of Low-Precision Vision-Language Models", gist.science) factor
each head's slice of the key (and value) projection separately, W_Kh ~
A_Kh B_Kh with A_Kh in R^{E x r} and B_Kh in R^{r x H} (Arabic page section
2a, German page section 2A, Japanese page section 2.1), and then refine the
factors against an importance-weighted error, min || F^(1/2) (.) (W - A B) ||_F^2
with F from Fisher information (Arabic page section 2b, German page section
2B, Japanese page section 2.2).  Readings:

* W [E, nh H] holds the heads side by side (column block h is W_h);
* the unweighted factors are the truncated SVD W_h = U S V^T cut at rank
  r, split as A_h = U_r S_r (the latent carries the singular values) and
  B_h = V_r^T (orthonormal rows);
* the weighted refinement is alternating weighted least squares: with B
  fixed each row of A solves its weighted normal equations, then with A
  fixed each column of B does; F is an input (real Fisher weights need
  gradients of a trained model).
"""
from __future__ import annotations

import numpy as np

__all__ = ["svd_factors", "weighted_objective", "als_step_A", "als_step_B", "weighted_factors"]


def svd_factors(W: np.ndarray, nh: int, r: int):
    """(A [E, nh r], B [nh, r, H]) from the rank-r truncated SVD of each head.

    Parity: pinned by the Eckart-Young optimum (error = sum of the discarded
    squared singular values, from an independent eigenvalue routine),
    orthonormal rows of B, exact recovery of rank-r heads and a hand case.
    """
    W = np.asarray(W, dtype=np.float64)
    E, NH = W.shape
    H = NH // nh
    A = np.zeros((E, nh * r))
    B = np.zeros((nh, r, H))
    for h in range(nh):
        U, s, Vt = np.linalg.svd(W[:, h * H:(h + 1) * H], full_matrices=False)
        A[:, h * r:(h + 1) * r] = U[:, :r] * s[:r]
        B[h] = Vt[:r]
    return A, B


def weighted_objective(W, F, A, B, nh: int) -> np.ndarray:
    """sum F (.) (W_h - A_h B_h)^2 per head."""
    W = np.asarray(W, np.float64)
    F = np.asarray(F, np.float64)
    H = W.shape[1] // nh
    r = B.shape[1]
    out = np.zeros(nh)
    for h in range(nh):
        R = W[:, h * H:(h + 1) * H] - A[:, h * r:(h + 1) * r] @ B[h]
        out[h] = np.sum(F[:, h * H:(h + 1) * H] * R * R)
    return out


def als_step_A(W, F, B, nh: int):
    """Each row a of A_h: argmin sum_j F_ej (W_ej - a . b_j)^2, i.e.
    (B diag(F_e) B^T) a = B diag(F_e) W_e^T."""
    W = np.asarray(W, np.float64)
    F = np.asarray(F, np.float64)
    E = W.shape[0]
    H = W.shape[1] // nh
    r = B.shape[1]
    A = np.zeros((E, nh * r))
    for h in range(nh):
        Bh = B[h]
        for e in range(E):
            f = F[e, h * H:(h + 1) * H]
            M = (Bh * f) @ Bh.T
            rhs = (Bh * f) @ W[e, h * H:(h + 1) * H]
            A[e, h * r:(h + 1) * r] = np.linalg.solve(M, rhs)
    return A


def als_step_B(W, F, A, nh: int):
    """Each column b_j of B_h: argmin sum_e F_ej (W_ej - a_e . b)^2, i.e.
    (A^T diag(F_j) A) b = A^T diag(F_j) W_j."""
    W = np.asarray(W, np.float64)
    F = np.asarray(F, np.float64)
    H = W.shape[1] // nh
    r = A.shape[1] // nh
    B = np.zeros((nh, r, H))
    for h in range(nh):
        Ah = A[:, h * r:(h + 1) * r]
        for j in range(H):
            f = F[:, h * H + j]
            M = Ah.T @ (Ah * f[:, None])
            rhs = Ah.T @ (f * W[:, h * H + j])
            B[h, :, j] = np.linalg.solve(M, rhs)
    return B


def weighted_factors(W, F, A0, B0, nh: int, iters: int):
    """`iters` rounds of (A step, then B step) from (A0, B0)."""
    A, B = np.asarray(A0, np.float64), np.asarray(B0, np.float64)
    for _ in range(iters):
        A = als_step_A(W, F, B, nh)
        B = als_step_B(W, F, A, nh)
    return A, B
