"""fp64 CPU oracle for decoding with a rotary position step after reconstruction.

TEST INFRASTRUCTURE ONLY (like the rest of this package): only the test
suite, the package smoke check and the benchmark's CPU-baseline leg may
import or run it; the GPU library never calls it and shares no code with
it.

The pages ("WSVD: Weighted Low-Rank Approximation for Fast and Efficient
Execution of Low-Precision Vision-Language Models", gist.science) describe
the fused kernel as loading latent tiles, rebuilding K and V on chip through
the head's factor and using them at once (German page section 2D, Italian
page section 2D, Japanese page section 2.4, Arabic page section 2c).  They
never mention a position encoding.  The language models they run use rotary
position embeddings, which act on each reconstructed key row, so a key can
no longer be folded into q' = B_K q.  Readings:

* rotary step, half-split pairing: element i is paired with i + H/2, and at
  token position t the pair is rotated by angle t * theta_i with
  theta_i = base^(-2 i / H), i < H/2 (the convention of the LLaMA family);
* the cached token t sits at position t (0-based); the query arrives
  already rotated to its own position, so only keys are rotated here;
* values carry no rotation.
"""
from __future__ import annotations

import numpy as np

from .wsvd_oracle import _sigma, attend, dequant_latent, reconstruct, upcast

__all__ = ["rope_angles", "rope_rotate", "decode_attn_rope"]


def rope_angles(positions, H: int, base: float = 10000.0) -> np.ndarray:
    """Angles t * theta_i, [len(positions), H/2], in float64."""
    i = np.arange(H // 2, dtype=np.float64)
    theta = base ** (-2.0 * i / H)
    return np.asarray(positions, dtype=np.float64)[:, None] * theta[None, :]


def rope_rotate(X: np.ndarray, positions, base: float = 10000.0) -> np.ndarray:
    """Rows X[t] rotated to positions[t]: pairs (i, i + H/2) by t * theta_i.

    Parity: pinned by hand-worked angles, norm preservation, composition of
    rotations and the relative-position identity of the dot product.
    """
    X = np.asarray(X, dtype=np.float64)
    H = X.shape[-1]
    a = rope_angles(positions, H, base)
    c, s = np.cos(a), np.sin(a)
    x1, x2 = X[..., : H // 2], X[..., H // 2:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def decode_attn_rope(inp, base: float = 10000.0, softmax_scale=None, pairs=None):
    """out [nb, nh, H] (or a dict over `pairs`): attention of the (already
    rotated) query over K rows rebuilt as C_K B_K and then rotated to their
    token positions, with V = C_V B_V unrotated."""
    nb, nh, H = inp.q.shape

    def one(b, h):
        ell = int(min(max(int(inp.L[b]), 0), inp.L_cap))
        if ell == 0:
            return np.zeros(H)
        sK = None if inp.s_K is None else inp.s_K[b, h, :ell]
        sV = None if inp.s_V is None else inp.s_V[b, h, :ell]
        K = reconstruct(dequant_latent(inp.C_K[b, h, :ell], inp.C_dt, sK), upcast(inp.B_K[h], inp.B_dt))
        V = reconstruct(dequant_latent(inp.C_V[b, h, :ell], inp.C_dt, sV), upcast(inp.B_V[h], inp.B_dt))
        K = rope_rotate(K, np.arange(ell), base)
        return attend(upcast(inp.q[b, h], inp.q_dt), K, V, _sigma(H, softmax_scale))

    if pairs is not None:
        return {(b, h): one(b, h) for (b, h) in pairs}
    out = np.zeros((nb, nh, H))
    for b in range(nb):
        for h in range(nh):
            out[b, h] = one(b, h)
    return out
