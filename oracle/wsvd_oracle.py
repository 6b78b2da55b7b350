"""fp64 CPU oracle for the WSVD per-head low-rank decode step.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and
the benchmark's CPU-baseline leg may import or run this module.  The GPU
library never calls it, and it shares no code with the GPU library.

What it computes is the plain definition: upcast every stored input to
float64 exactly, rebuild K = C_K . B_K and V = C_V . B_V per head, and run
ordinary softmax attention of q over the L cached tokens.  It is slow on
purpose: one (b, h) at a time, explicit reconstruction, no fusion.

Citations name the page "WSVD: Weighted Low-Rank Approximation for Fast and
Efficient Execution of Low-Precision Vision-Language Models" on gist.science
by language and section:

* per-head factors W_Kh ~ A_Kh B_Kh, A_Kh in R^{E x r}, B_Kh in R^{r x H},
  and an L x r latent cache per head: Arabic page section 2a, German page
  section 2A, Japanese page section 2.1;
* the fused kernel streams latent tiles, multiplies them by the factor
  on chip and feeds the result straight into qK^T, softmax and the V
  product (Flash-Decoding pipeline): German page section 2D, Italian page
  section 2D, Arabic page section 2c, Japanese page section 2.4.  Since
  that kernel only reorders the same arithmetic, its exact result is the
  attention below over reconstructed K and V.
* the V side is written out only for K on the pages; V is taken to be
  factored the same way (C_Vh = X A_Vh, V_h = C_Vh B_Vh).

Readings where the pages are silent:

* softmax scale sigma = 1/sqrt(H) unless given; no rotary position step;
* split s of a sequence with l tokens over S splits covers tokens
  [s*ceil(l/S), min(l, (s+1)*ceil(l/S))); a split's partial is the
  attention restricted to that range plus lse = log sum exp(score) in
  natural-log units, an empty range gives (0, -inf); partials merge with
  weights exp(lse_s - max lse);
* l = 0 gives a zero output;
* int8 latents dequantise as code * fp16 scale of their (b, h, token) row;
* an appended latent row is x . A_Kh computed exactly and rounded once to
  the cache dtype (nearest, ties to even);
* an int8 cache row (8-bit storage of the pages' W8A8 setting) is stored
  as symmetric absmax codes: scale = fp16(absmax / 127), code =
  clamp(round_half_even(c / scale), -127, 127), a zero row has scale 0.
  Where these decisions turn floats into integers they are taken in fp32,
  the precision the GPU takes them in.

Parity status of each function is stated in its docstring; every function
here is pinned by tests that do not reuse its own formula.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "upcast", "dequant_latent", "reconstruct", "softmax_weights", "attend",
    "split_bounds", "segment_attend", "combine", "decode_attn",
    "decode_attn_one", "decode_partials_one", "append_latents",
    "apply_append", "round_to_bf16_bits", "quantize_latent_rows",
    "apply_append_int8",
]


# ---------------------------------------------------------------------------
# exact upcasts of the storage dtypes
# ---------------------------------------------------------------------------
def upcast(a: np.ndarray, dt: str) -> np.ndarray:
    """Exact float64 value of a stored tensor.

    bf16 is stored as its 16-bit pattern: the value is the float32 whose
    upper half is that pattern.  Pinned by hand-checked bit patterns.
    """
    if dt == "f64":
        return np.asarray(a, dtype=np.float64)
    if dt == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    if dt == "bf16":
        bits = np.asarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    if dt == "f16":
        return np.asarray(a, dtype=np.float16).astype(np.float64)
    if dt == "i8":
        return np.asarray(a, dtype=np.int8).astype(np.float64)
    raise ValueError(f"unknown dtype {dt!r}")


def dequant_latent(C: np.ndarray, C_dt: str, scale: np.ndarray | None = None) -> np.ndarray:
    """Latent rows as float64; int8 rows times their fp16 per-row scale.

    Both factors are exact in float64 and so is their product (8-bit
    integer times 11-bit significand).
    """
    c = upcast(C, C_dt)
    if C_dt == "i8":
        if scale is None:
            raise ValueError("int8 latents need their per-row scales")
        c = c * upcast(scale, "f16")[..., None]
    return c


# ---------------------------------------------------------------------------
# reconstruction and attention for one head
# ---------------------------------------------------------------------------
def reconstruct(c_hat: np.ndarray, B: np.ndarray) -> np.ndarray:
    """K_h = C_Kh B_Kh (l x r times r x H): the per-head factor of the
    Arabic page section 2a applied to the cached latent rows."""
    return c_hat @ B


def softmax_weights(s: np.ndarray) -> np.ndarray:
    """p_t = exp(s_t - max s) / sum_u exp(s_u - max s)."""
    m = np.max(s)
    e = np.exp(s - m)
    return e / np.sum(e)


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, sigma: float) -> np.ndarray:
    """Softmax attention of one query over l tokens (l >= 1)."""
    s = sigma * (K @ q)
    return softmax_weights(s) @ V


def split_bounds(ell: int, S: int):
    """Token range of each split: chunks of ceil(l/S) tokens, last ones may be short or empty."""
    if S <= 0:
        raise ValueError("S must be positive")
    chunk = -(-ell // S) if ell > 0 else 0
    out = []
    for s in range(S):
        a = min(ell, s * chunk)
        e = min(ell, (s + 1) * chunk)
        out.append((a, e))
    return out


def segment_attend(q, K, V, sigma, a, e):
    """Attention restricted to tokens [a, e) and its log-sum-exp (natural log).

    Returns (o, lse) with o normalised over the segment; an empty segment
    gives (zeros, -inf).
    """
    H = V.shape[1]
    if e <= a:
        return np.zeros(H), -math.inf
    s = sigma * (K[a:e] @ q)
    m = np.max(s)
    w = np.exp(s - m)
    tot = np.sum(w)
    return (w / tot) @ V[a:e], float(m + math.log(tot))


def combine(o_parts: np.ndarray, lse_parts: np.ndarray) -> np.ndarray:
    """Merge normalised partials: out = sum_s w_s o_s / sum_s w_s,
    w_s = exp(lse_s - max lse).  All partials empty -> zeros."""
    lse = np.asarray(lse_parts, dtype=np.float64)
    o = np.asarray(o_parts, dtype=np.float64)
    if lse.size == 0 or not np.any(np.isfinite(lse)):
        return np.zeros(o.shape[-1])
    M = np.max(lse)
    w = np.where(np.isfinite(lse), np.exp(lse - M), 0.0)
    return (w @ o) / np.sum(w)


# ---------------------------------------------------------------------------
# whole decode step
# ---------------------------------------------------------------------------
def _sigma(H, softmax_scale):
    return 1.0 / math.sqrt(H) if (softmax_scale is None or softmax_scale <= 0) else float(softmax_scale)


def decode_attn_one(inp, b: int, h: int, softmax_scale=None, *, C_K=None, C_V=None):
    """Output row out[b, h, :] in float64 (materialises K and V of that head).

    C_K / C_V override the input's caches (used after an append).
    """
    C_K = inp.C_K if C_K is None else C_K
    C_V = inp.C_V if C_V is None else C_V
    H = inp.q.shape[-1]
    ell = int(min(max(int(inp.L[b]), 0), inp.L_cap))
    if ell == 0:
        return np.zeros(H)
    sK = None if inp.s_K is None else inp.s_K[b, h, :ell]
    sV = None if inp.s_V is None else inp.s_V[b, h, :ell]
    ck = dequant_latent(C_K[b, h, :ell], inp.C_dt, sK)
    cv = dequant_latent(C_V[b, h, :ell], inp.C_dt, sV)
    K = reconstruct(ck, upcast(inp.B_K[h], inp.B_dt))
    V = reconstruct(cv, upcast(inp.B_V[h], inp.B_dt))
    q = upcast(inp.q[b, h], inp.q_dt)
    return attend(q, K, V, _sigma(H, softmax_scale))


def decode_attn(inp, softmax_scale=None, *, C_K=None, C_V=None, pairs=None):
    """out [nb, nh, H] float64, or only the listed (b, h) pairs (dict)."""
    if pairs is not None:
        return {(b, h): decode_attn_one(inp, b, h, softmax_scale, C_K=C_K, C_V=C_V)
                for (b, h) in pairs}
    nb, nh, H = inp.q.shape
    out = np.zeros((nb, nh, H))
    for b in range(nb):
        for h in range(nh):
            out[b, h] = decode_attn_one(inp, b, h, softmax_scale, C_K=C_K, C_V=C_V)
    return out


def decode_partials_one(inp, b, h, S, softmax_scale=None):
    """Per-split (o_s, lse_s) of one head, with the split rule above."""
    H = inp.q.shape[-1]
    ell = int(min(max(int(inp.L[b]), 0), inp.L_cap))
    sK = None if inp.s_K is None else inp.s_K[b, h, :ell]
    sV = None if inp.s_V is None else inp.s_V[b, h, :ell]
    K = reconstruct(dequant_latent(inp.C_K[b, h, :ell], inp.C_dt, sK), upcast(inp.B_K[h], inp.B_dt))
    V = reconstruct(dequant_latent(inp.C_V[b, h, :ell], inp.C_dt, sV), upcast(inp.B_V[h], inp.B_dt))
    q = upcast(inp.q[b, h], inp.q_dt)
    sig = _sigma(H, softmax_scale)
    o = np.zeros((S, H))
    lse = np.full(S, -math.inf)
    for s, (a, e) in enumerate(split_bounds(ell, S)):
        o[s], lse[s] = segment_attend(q, K, V, sig, a, e)
    return o, lse


# ---------------------------------------------------------------------------
# appending the new token's latent
# ---------------------------------------------------------------------------
def round_to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """Round float64 values once to bfloat16 (nearest, ties to even).

    bfloat16 keeps 8 significant bits and float32's exponent range; below
    2^-126 the spacing is fixed at 2^-133.  Finite inputs only.
    """
    v = np.asarray(v, dtype=np.float64)
    out = np.zeros(v.shape, dtype=np.float64)
    nz = v != 0
    m, e = np.frexp(v[nz])                    # v = m 2^e, 0.5 <= |m| < 1
    quantum = np.ldexp(1.0, np.maximum(e - 8, -133))
    out[nz] = np.rint(v[nz] / quantum) * quantum   # np.rint: ties to even
    bits = out.astype(np.float32).view(np.uint32) >> np.uint32(16)
    return bits.astype(np.uint16)


def append_latents(x: np.ndarray, x_dt: str, A: np.ndarray, A_dt: str, nh: int, r: int) -> np.ndarray:
    """c[b, h, :] = x[b] . A[:, h r:(h+1) r] in float64 -> [nb, nh, r].

    A's column block h is A_Kh in R^{E x r} (per-head factor, Arabic page
    section 2a); the product with the token's activation is the new row of
    that head's latent cache.
    """
    xx = upcast(x, x_dt)
    AA = upcast(A, A_dt)
    nb = xx.shape[0]
    c = np.zeros((nb, nh, r))
    for h in range(nh):
        c[:, h, :] = xx @ AA[:, h * r:(h + 1) * r]
    return c


def apply_append(inp):
    """Caches after writing x.A_Kh / x.A_Vh (rounded to bf16) at row pos[b].

    Returns (C_K, C_V, latK_f64, latV_f64).  Rows with pos outside
    [0, L_cap) are not written.
    """
    if inp.C_dt != "bf16":
        raise ValueError("the oracle's append covers bf16 caches")
    cK = append_latents(inp.x, inp.x_dt, inp.A_K, inp.A_dt, inp.nh, inp.r)
    cV = append_latents(inp.x, inp.x_dt, inp.A_V, inp.A_dt, inp.nh, inp.r)
    C_K = inp.C_K.copy()
    C_V = inp.C_V.copy()
    for b in range(inp.nb):
        p = int(inp.pos[b])
        if 0 <= p < inp.L_cap:
            C_K[b, :, p, :] = round_to_bf16_bits(cK[b])
            C_V[b, :, p, :] = round_to_bf16_bits(cV[b])
    return C_K, C_V, cK, cV


def quantize_latent_rows(c: np.ndarray):
    """Symmetric absmax int8 storage of latent rows (last axis) -> (codes, scales).

    The pages quantise activations and cached latents to 8 bits (W8A8;
    German page section 2C, Arabic page section 2c) without fixing the
    quantiser; the reading here is the common symmetric per-row form:
    scale = fp16(max |c| / 127), code = clamp(round_half_even(c / scale),
    -127, 127), and a row whose scale is 0 stores zeros.  The decisions are
    taken in fp32, as the kernel takes them: c is rounded to fp32 once,
    max|c| / 127 and c / scale are single fp32 operations, and the scale is
    rounded to fp16 (nearest, ties to even).  Scales are returned as
    float16 values.

    Parity: pinned by hand-worked rows (rounding, ties, clamp, zero row).
    """
    c32 = np.asarray(c, dtype=np.float64).astype(np.float32)
    amax = np.max(np.abs(c32), axis=-1)
    scale16 = np.divide(amax, np.float32(127.0), dtype=np.float32).astype(np.float16)
    s32 = scale16.astype(np.float32)[..., None]
    codes = np.zeros(c32.shape, dtype=np.float32)
    ok = np.broadcast_to(s32 > 0, c32.shape)
    ratio = np.divide(c32, np.where(s32 > 0, s32, np.float32(1.0)), dtype=np.float32)
    codes[ok] = np.rint(ratio[ok])
    codes = np.clip(codes, -127, 127).astype(np.int8)
    return codes, scale16


def apply_append_int8(inp):
    """Int8 caches after appending x.A_Kh / x.A_Vh at row pos[b].

    The latent is computed exactly (append_latents), then stored with
    quantize_latent_rows.  Returns (C_K, C_V, s_K, s_V, latK_f64, latV_f64)
    with codes int8 and scales float16; rows with pos outside [0, L_cap) are
    not written.
    """
    if inp.C_dt != "i8":
        raise ValueError("apply_append_int8 covers int8 caches")
    cK = append_latents(inp.x, inp.x_dt, inp.A_K, inp.A_dt, inp.nh, inp.r)
    cV = append_latents(inp.x, inp.x_dt, inp.A_V, inp.A_dt, inp.nh, inp.r)
    C_K, C_V = inp.C_K.copy(), inp.C_V.copy()
    s_K = np.asarray(inp.s_K, dtype=np.float16).copy()
    s_V = np.asarray(inp.s_V, dtype=np.float16).copy()
    for b in range(inp.nb):
        p = int(inp.pos[b])
        if 0 <= p < inp.L_cap:
            C_K[b, :, p, :], s_K[b, :, p] = quantize_latent_rows(cK[b])
            C_V[b, :, p, :], s_V[b, :, p] = quantize_latent_rows(cV[b])
    return C_K, C_V, s_K, s_V, cK, cV
