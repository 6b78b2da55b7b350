"""fp64 CPU oracle for the W8A8 projection of the new token's latents.

TEST INFRASTRUCTURE ONLY (like the rest of this package): only the test
suite, the package smoke check and the benchmark's CPU-baseline leg may
import or run it; the GPU library never calls it and shares no code with
it.

The pages ("WSVD: Weighted Low-Rank Approximation for Fast and Efficient
Execution of Low-Precision Vision-Language Models", gist.science) run the
low-rank layers at W8A8 and smooth activation outliers with an orthogonal
Hadamard rotation S1 before quantising (German page section 2C, Italian
page section 2C, Japanese page section 2.3, Arabic page section 2c).  They
give neither the rotation's size nor the quantiser, so the readings here
are:

* S1 is the normalised Walsh-Hadamard matrix of size E (Sylvester order,
  E a power of two), H = H_E / sqrt(E).  H is symmetric and orthogonal, so
  x . A = (x H) . (H A): the rotation of A is folded offline.
* weights: A' = H A, quantised per output column with an fp32 scale
  s_A[n] = max_e |A'[e, n]| / 127, codes clamp(round_half_even(A' / s_A),
  -127, 127);
* activations: x~ = x H, quantised per token the same way (fp32 s_x[b]);
* the product accumulates the integer codes exactly (int32 on the GPU),
  and the latent is acc * s_x[b] * s_A[n].

Quantisation decisions are taken in fp32 (the kernel's precision): the
exact rotated value is rounded to fp32 once, max|.| / 127 and value / scale
are single fp32 operations.
"""
from __future__ import annotations

import numpy as np

from .wsvd_oracle import upcast

__all__ = ["hadamard_matrix", "rotate_rows", "quantize_rows_f32", "prepare_factor", "quantize_activations",
           "w8a8_latents"]


def hadamard_matrix(n: int) -> np.ndarray:
    """Sylvester Hadamard matrix of order n (a power of two), entries +-1.

    H_1 = [1], H_2k = [[H_k, H_k], [H_k, -H_k]].  Parity: pinned against
    the textbook construction in scipy.linalg.hadamard and H H^T = n I.
    """
    if n < 1 or n & (n - 1):
        raise ValueError("Hadamard order must be a power of two")
    h = np.ones((1, 1), dtype=np.int64)
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


def rotate_rows(x: np.ndarray, x_dt: str) -> np.ndarray:
    """x . H_E / sqrt(E) in float64 for rows of x [.., E] (stored dtype x_dt)."""
    xx = upcast(x, x_dt)
    E = xx.shape[-1]
    return (xx @ hadamard_matrix(E).astype(np.float64)) / np.sqrt(E)


def quantize_rows_f32(v: np.ndarray):
    """Symmetric absmax int8 codes of rows (last axis) with an fp32 scale.

    scale = fp32(max |fp32(v)| / 127); code = clamp(round_half_even(fp32(v) /
    scale), -127, 127); a zero row has scale 0 and codes 0.  Returns
    (codes int8, scale float32).  Parity: pinned by hand-worked rows.
    """
    v32 = np.asarray(v, dtype=np.float64).astype(np.float32)
    amax = np.max(np.abs(v32), axis=-1)
    scale = np.divide(amax, np.float32(127.0), dtype=np.float32)
    s = scale[..., None]
    ratio = np.divide(v32, np.where(s > 0, s, np.float32(1.0)), dtype=np.float32)
    codes = np.where(s > 0, np.rint(ratio), np.float32(0.0))
    return np.clip(codes, -127, 127).astype(np.int8), scale


def prepare_factor(A: np.ndarray, A_dt: str):
    """Rotated, column-quantised factor: (A^T codes [N, E] int8, s_A [N] fp32).

    A' = H_E A / sqrt(E) for A [E, N]; column n of A' is quantised as one
    row (quantize_rows_f32), stored k-contiguous as row n of the result.
    """
    AA = upcast(A, A_dt)
    E = AA.shape[0]
    rot = (hadamard_matrix(E).astype(np.float64) @ AA) / np.sqrt(E)
    return quantize_rows_f32(rot.T)


def quantize_activations(x: np.ndarray, x_dt: str):
    """Per-token int8 codes of the rotated activations: (codes [nb, E], s_x [nb])."""
    return quantize_rows_f32(rotate_rows(x, x_dt))


def w8a8_latents(xq: np.ndarray, sx: np.ndarray, AqT: np.ndarray, sA: np.ndarray, nh: int, r: int) -> np.ndarray:
    """Latents [nb, nh, r] in float64: (sum_e xq[b, e] AqT[n, e]) * s_x[b] * s_A[n].

    The integer sum is exact (int64 here).  Column n = h r + i is entry i of
    head h's latent.
    """
    acc = np.asarray(xq, dtype=np.int64) @ np.asarray(AqT, dtype=np.int64).T
    c = acc.astype(np.float64) * np.asarray(sx, np.float64)[:, None] * np.asarray(sA, np.float64)[None, :]
    return c.reshape(c.shape[0], nh, r)
