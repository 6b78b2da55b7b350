"""fp64 CPU oracle for decoding over a conventional (whole-matrix) factorisation.

TEST INFRASTRUCTURE ONLY (like the rest of this package): only the test
suite, the package smoke check and the benchmark's CPU-baseline leg may
import or run it; the GPU library never calls it and shares no code with
it.

The pages ("WSVD: Weighted Low-Rank Approximation for Fast and Efficient
Execution of Low-Precision Vision-Language Models", gist.science) set WSVD
against the usual SVD compression, which factors the whole K (V)
projection, W_K ~ A B with a single latent of global rank R shared by all
heads, so every head rebuilds its keys and values from that shared latent
during decoding (Japanese page section 1, German page section 1, Italian
page section 1, Arabic page section 1); the per-head form shrinks the
latent from L x R to L x r and the rebuild cost by r / R (Arabic page
section 2a, Italian page section 2A).  Readings:

* the shared latent of sequence b is C_K[b] in R^{L x R}; the factor
  B_K in R^{R x nh H} holds head h's map in its column block
  [h H, (h + 1) H), so head h's keys are C_K[b] B_K[:, hH:(h+1)H]; values
  likewise with C_V, B_V;
* attention, softmax scale and the treatment of empty sequences are those
  of the per-head oracle.
"""
from __future__ import annotations

import numpy as np

from .wsvd_oracle import _sigma, attend, upcast

__all__ = ["decode_attn_shared", "decode_attn_shared_one"]


def decode_attn_shared_one(inp, b: int, h: int, softmax_scale=None) -> np.ndarray:
    """out[b, h, :]: attention of q[b, h] over K = C_K[b] B_K[:, hH:(h+1)H]
    and V = C_V[b] B_V[:, hH:(h+1)H] for the first L[b] tokens.

    Parity: pinned by the block-diagonal embedding of per-head latents
    (which must reproduce the per-head oracle), identity factors against
    library attention, and brute-force loops on tiny inputs.
    """
    H = inp.H
    ell = int(min(max(int(inp.L[b]), 0), inp.L_cap))
    if ell == 0:
        return np.zeros(H)
    cols = slice(h * H, (h + 1) * H)
    K = upcast(inp.C_K[b, :ell], inp.dt) @ upcast(inp.B_K, inp.dt)[:, cols]
    V = upcast(inp.C_V[b, :ell], inp.dt) @ upcast(inp.B_V, inp.dt)[:, cols]
    return attend(upcast(inp.q[b, h], inp.dt), K, V, _sigma(H, softmax_scale))


def decode_attn_shared(inp, softmax_scale=None, pairs=None):
    """out [nb, nh, H] (or a dict over `pairs`)."""
    if pairs is not None:
        return {(b, h): decode_attn_shared_one(inp, b, h, softmax_scale) for (b, h) in pairs}
    out = np.zeros((inp.nb, inp.nh, inp.H))
    for b in range(inp.nb):
        for h in range(inp.nh):
            out[b, h] = decode_attn_shared_one(inp, b, h, softmax_scale)
    return out
