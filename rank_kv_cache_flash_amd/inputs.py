"""Seeded synthetic inputs for the WSVD low-rank decode step.

This module is shared by the GPU path's tests and benchmark and by the CPU
oracle's tests.  It only *draws* tensors and stores them in their storage
dtypes; it contains none of the decode arithmetic (no reconstruction, no
softmax, no projection).  Every tensor is a NumPy array:

    fp32  -> np.float32
    bf16  -> np.uint16 holding the bfloat16 bit pattern
    fp16  -> np.float16
    int8  -> np.int8

Recipe (one seed per configuration, ``seed = 1000 + config id``):

* Each tensor, and for batched tensors each batch row b, draws from its own
  PCG64 stream keyed by ``SeedSequence([seed, tensor_id, b])``, so a single
  sequence of a large configuration can be regenerated alone and the draw
  does not depend on thread count.
* Values are N(0, 1) divided by the square root of the tensor's last
  dimension: q by sqrt(H), latents by sqrt(r), B_K / B_V ([nh, r, H]) by
  sqrt(H), x by sqrt(E), A_K / A_V ([E, nh*r]) by sqrt(r).  With these
  scales x.A_Kh has the same per-entry variance (1/r) as the drawn latents.
* Draws are float32 and are rounded once to the storage dtype
  (round-to-nearest-even).
* The int8 cache (W8A8-style configuration) marks 1 % of latent entries,
  independently per entry and independently for K and V, multiplies them
  by 20, and then stores each (b, h, token) row symmetrically: an fp16 scale
  absmax/127 and int8 codes round(c / scale) clamped to +-127 (an all-zero
  row gets scale 0 and codes 0).  This is how the synthetic cache is
  produced, not part of the decode step: decode consumes the stored codes
  and scales as they are.
* Ragged configuration: L[b] is uniform over the integers [1024, 8192];
  rows 0 .. L[b]-2 of each cache are drawn, the rest are zero, and the new
  token is appended at pos[b] = L[b]-1, so L[b] counts the tokens attended
  after the append.

The shapes follow the per-head factorisation W_Kh ~ A_Kh B_Kh with
A_Kh in R^{E x r} and B_Kh in R^{r x H} and a per-head latent cache of
L x r values ("WSVD: Weighted Low-Rank Approximation for Fast and Efficient
Execution of Low-Precision Vision-Language Models", Arabic page section 2a;
German page section 2A).
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

# Stream identifiers; fixed forever so stored fixtures stay reproducible.
T_Q, T_CK, T_CV, T_BK, T_BV, T_MK, T_MV, T_L, T_X, T_AK, T_AV = range(1, 12)


def _rng(seed: int, *key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, *key])))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def _store(x32: np.ndarray, dt: str) -> np.ndarray:
    if dt == "f32":
        return np.ascontiguousarray(x32, dtype=np.float32)
    if dt == "bf16":
        return f32_to_bf16_bits(x32)
    if dt == "f16":
        return x32.astype(np.float16)
    raise ValueError(dt)


def _normal(seed, key, shape, scale):
    g = _rng(seed, *key)
    return g.standard_normal(shape, dtype=np.float32) * np.float32(scale)


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _pmap(fn, items):
    items = list(items)
    if len(items) <= 1:
        return [fn(i) for i in items]
    with ThreadPoolExecutor(_workers()) as ex:
        return list(ex.map(fn, items))


@dataclass
class DecodeInputs:
    """Everything one decode step consumes, in storage dtypes."""
    nb: int
    nh: int
    H: int
    r: int
    L_cap: int
    q: np.ndarray            # [nb, nh, H]
    q_dt: str
    C_K: np.ndarray          # [nb, nh, L_cap, r]
    C_V: np.ndarray
    C_dt: str                # "f32" | "bf16" | "i8"
    B_K: np.ndarray          # [nh, r, H]
    B_V: np.ndarray
    B_dt: str
    L: np.ndarray            # int32 [nb], tokens attended
    out_dt: str
    s_K: np.ndarray | None = None   # fp16 [nb, nh, L_cap] (int8 caches)
    s_V: np.ndarray | None = None
    # ragged/append configuration only
    E: int = 0
    x: np.ndarray | None = None     # [nb, E]
    x_dt: str = "bf16"
    A_K: np.ndarray | None = None   # [E, nh*r]
    A_V: np.ndarray | None = None
    A_dt: str = "bf16"
    pos: np.ndarray | None = None   # int32 [nb], row the append writes
    meta: dict = field(default_factory=dict)


def _int8_rows(c: np.ndarray):
    """Symmetric per-row absmax storage of a float32 [..., r] block."""
    amax = np.abs(c).max(axis=-1)
    scale16 = (amax / np.float32(127.0)).astype(np.float16)
    s32 = scale16.astype(np.float32)
    safe = np.where(s32 > 0, s32, np.float32(1.0))
    codes = np.rint(c / safe[..., None])
    codes = np.where(s32[..., None] > 0, codes, 0.0)
    codes = np.clip(codes, -127, 127).astype(np.int8)
    return codes, scale16


def _latent_block(seed, tid, mid, b, nh, fill, L_cap, r, C_dt, outlier_p, outlier_mul):
    c = np.zeros((nh, L_cap, r), dtype=np.float32)
    if fill > 0:
        c[:, :fill, :] = _normal(seed, (tid, b), (nh, fill, r), 1.0 / np.sqrt(r))
    if C_dt != "i8":
        return _store(c, C_dt), None
    if outlier_p > 0 and fill > 0:
        m = _rng(seed, mid, b).random((nh, fill, r), dtype=np.float32) < np.float32(outlier_p)
        blk = c[:, :fill, :]
        blk[m] *= np.float32(outlier_mul)
    return _int8_rows(c)


def make_decode_inputs(nb, nh, H, r, L, L_cap, *, seed, act_dt="bf16", C_dt="bf16",
                       out_dt=None, fill=None, outlier_p=0.0, outlier_mul=1.0,
                       q_gain=1.0) -> DecodeInputs:
    """Draw one decode step's inputs.

    L      : int or int array [nb] -- tokens attended per sequence.
    fill   : rows of each cache that hold drawn latents (defaults to L).
    q_gain : multiplies q before rounding (peaked-softmax variants).
    """
    L = np.broadcast_to(np.asarray(L, dtype=np.int32), (nb,)).copy()
    fill = L.copy() if fill is None else np.broadcast_to(np.asarray(fill, dtype=np.int32), (nb,)).copy()
    out_dt = out_dt or act_dt
    q = np.stack([_normal(seed, (T_Q, b), (nh, H), q_gain / np.sqrt(H)) for b in range(nb)])
    ck = _pmap(lambda b: _latent_block(seed, T_CK, T_MK, b, nh, int(fill[b]), L_cap, r, C_dt,
                                       outlier_p, outlier_mul), range(nb))
    cv = _pmap(lambda b: _latent_block(seed, T_CV, T_MV, b, nh, int(fill[b]), L_cap, r, C_dt,
                                       outlier_p, outlier_mul), range(nb))
    C_K = np.stack([c for c, _ in ck])
    C_V = np.stack([c for c, _ in cv])
    s_K = np.stack([s for _, s in ck]) if C_dt == "i8" else None
    s_V = np.stack([s for _, s in cv]) if C_dt == "i8" else None
    B_K = _normal(seed, (T_BK,), (nh, r, H), 1.0 / np.sqrt(H))
    B_V = _normal(seed, (T_BV,), (nh, r, H), 1.0 / np.sqrt(H))
    return DecodeInputs(nb=nb, nh=nh, H=H, r=r, L_cap=L_cap,
                        q=_store(q, act_dt), q_dt=act_dt,
                        C_K=C_K, C_V=C_V, C_dt=C_dt,
                        B_K=_store(B_K, act_dt), B_V=_store(B_V, act_dt), B_dt=act_dt,
                        L=L, out_dt=out_dt, s_K=s_K, s_V=s_V,
                        meta=dict(seed=seed, q_gain=q_gain))


def make_ragged_step_inputs(nb, nh, H, r, E, L_lo, L_hi, L_cap, *, seed, q_gain=1.0,
                            dt="bf16", C_dt=None) -> DecodeInputs:
    """Full decode step: append x.A_Kh / x.A_Vh at pos = L-1, then attend L tokens.

    x, A, q and B are stored in `dt`; the caches in `C_dt` (default `dt`;
    "i8" gives int8 codes with fp16 per-row scales)."""
    L = _rng(seed, T_L).integers(L_lo, L_hi, size=nb, endpoint=True).astype(np.int32)
    inp = make_decode_inputs(nb, nh, H, r, L, L_cap, seed=seed, act_dt=dt, C_dt=C_dt or dt,
                             fill=L - 1, q_gain=q_gain)
    x = _normal(seed, (T_X,), (nb, E), 1.0 / np.sqrt(E))
    A_K = _normal(seed, (T_AK,), (E, nh * r), 1.0 / np.sqrt(r))
    A_V = _normal(seed, (T_AV,), (E, nh * r), 1.0 / np.sqrt(r))
    inp.E = E
    inp.x, inp.x_dt = _store(x, dt), dt
    inp.A_K, inp.A_V, inp.A_dt = _store(A_K, dt), _store(A_V, dt), dt
    inp.pos = (L - 1).astype(np.int32)
    return inp


def add_score_shift(inp: DecodeInputs, shift: float = 1000.0) -> DecodeInputs:
    """Rebuild a step's inputs so that every attention score (default scale
    1/sqrt(H)) carries one common offset of about `shift`.

    The last latent column holds the same value c for every token, the
    matching row of B_K maps it onto the first component of q alone, and that
    component is 1:

      * q[b, h, 0] = 1;
      * C_K[..., r-1] = c: 1.0 for f32 / bf16 caches; for an int8 cache code
        127 with every row's fp16 scale set to s0 = fp16(1/127) (so c = 127 s0
        and every row dequantises with the same scale);
      * B_K[h, r-1, :] = (a, 0, ..., 0) with a = shift sqrt(H) / c rounded to
        the factor dtype.

    The offset sigma c a q0 is exactly the same for every token of a head, so
    attention is unchanged by it in exact arithmetic; its value is returned
    in meta["score_shift"] and the input with a = 0 in meta["unshifted"]
    (same tensors otherwise).  The caches keep rows past L[b] as they were.
    Returns a new DecodeInputs; `inp` is not modified."""
    import copy
    out = copy.deepcopy(inp)
    nb, nh, H = out.q.shape
    r = out.r
    one = {"f32": np.float32(1.0), "bf16": np.uint16(0x3F80), "f16": np.float16(1.0)}
    out.q[:, :, 0] = one[out.q_dt]
    if out.C_dt == "i8":
        s0 = np.float16(1.0 / 127.0)
        c = 127.0 * float(s0)
        out.s_K[...] = s0
        out.C_K[..., r - 1] = 127
    else:
        c = 1.0
        out.C_K[..., r - 1] = one[out.C_dt]
    a32 = np.float32(shift * np.sqrt(H) / c)
    a_store = _store(np.array([a32], np.float32), out.B_dt)[0]
    out.B_K[:, r - 1, :] = 0
    twin = copy.deepcopy(out)
    out.B_K[:, r - 1, 0] = a_store
    a_val = float(np.asarray([a_store]).view(np.float32)[0]) if out.B_dt == "f32" else (
        float(np.float16(a_store)) if out.B_dt == "f16" else
        float((np.uint32(a_store) << np.uint32(16)).view(np.float32)))
    out.meta = dict(out.meta, score_shift=c * a_val / np.sqrt(H), unshifted=twin)
    return out


# ---------------------------------------------------------------------------
# W8A8 projection inputs
# ---------------------------------------------------------------------------
T_XO, T_XQ, T_SX, T_AQ, T_SA = range(20, 25)


def make_w8a8_activations(nb, E, *, seed, outlier_channels=0.01, outlier_mul=20.0, dt="bf16"):
    """Token activations x [nb, E] ~ N(0, 1)/sqrt(E) with a few outlier
    channels (the same seeded 1 % of the E columns scaled by outlier_mul in
    every token), the structure the pages' rotation is meant to smooth."""
    x = _normal(seed, (T_X,), (nb, E), 1.0 / np.sqrt(E))
    cols = _rng(seed, T_XO).random(E) < outlier_channels
    x[:, cols] *= np.float32(outlier_mul)
    return _store(x, dt)


def make_w8a8_codes(nb, E, N, *, seed):
    """Synthetic integer operands of the W8A8 product: token codes xq [nb, E],
    per-token scales sx [nb], transposed factor codes AqT [N, E] and
    per-column scales sA [N].  Codes are uniform in [-127, 127]; scales are
    positive and spread over a few octaves."""
    xq = _rng(seed, T_XQ).integers(-127, 128, size=(nb, E), dtype=np.int8)
    AqT = _rng(seed, T_AQ).integers(-127, 128, size=(N, E), dtype=np.int8)
    sx = (np.exp2(_rng(seed, T_SX).uniform(-12, -8, size=nb))).astype(np.float32)
    sA = (np.exp2(_rng(seed, T_SA).uniform(-10, -6, size=N))).astype(np.float32)
    return xq, sx, AqT, sA


T_WP, T_WU, T_WV, T_WS, T_F = range(30, 35)


def make_projection_weights(E, nh, H, *, seed, spectrum="gaussian", rank=None):
    """A projection W fp32 [E, nh*H] whose column block h is head h's slice.

    spectrum = "gaussian": i.i.d. N(0, 1)/sqrt(E) entries (singular values
    packed in a Marchenko-Pastur band); "powerlaw": W_h = U diag(s) V^T with
    Haar-random orthonormal U [E, k], V [H, k], k = min(E, H) (QR of Gaussian
    draws, signs fixed by the diagonal of R) and s_i = (i + 1)^(-1/2), a smoothly decaying
    spectrum with distinct values; "lowrank": (E x rank) @ (rank x H)
    Gaussian product, so W_h has rank `rank` exactly."""
    W = np.zeros((E, nh * H), np.float32)
    for h in range(nh):
        if spectrum == "gaussian":
            Wh = _rng(seed, T_WP, h).standard_normal((E, H)) / np.sqrt(E)
        elif spectrum == "powerlaw":
            def haar(key, m, n):
                Q, R = np.linalg.qr(_rng(seed, key, h).standard_normal((m, n)))
                return Q * np.sign(np.diag(R))
            k = min(E, H)
            s = (np.arange(k) + 1.0) ** -0.5
            Wh = (haar(T_WU, E, k) * s) @ haar(T_WV, H, k).T
        elif spectrum == "lowrank":
            g = _rng(seed, T_WS, h)
            Wh = g.standard_normal((E, rank)) @ g.standard_normal((rank, H)) / np.sqrt(E * rank)
        else:
            raise ValueError(spectrum)
        W[:, h * H:(h + 1) * H] = Wh
    return W


def make_fisher_weights(E, nh, H, *, seed, sigma=1.0):
    """Importance weights F fp32 [E, nh*H], laid out like W: log-normal,
    exp(N(0, sigma^2)), positive with a heavy upper tail (diagonal Fisher
    information is a mean of squared gradients)."""
    return np.exp(sigma * _rng(seed, T_F).standard_normal((E, nh * H))).astype(np.float32)


T_SQ, T_SCK, T_SCV, T_SBK, T_SBV = range(40, 45)


@dataclass
class SharedInputs:
    """One decode step of the conventional (whole-matrix) factorisation: a
    latent of rank R shared by all heads, and factors B [R, nh*H] whose
    column block h maps it to head h's keys (values)."""
    nb: int
    nh: int
    H: int
    R: int
    L_cap: int
    q: np.ndarray            # [nb, nh, H]
    C_K: np.ndarray          # [nb, L_cap, R]
    C_V: np.ndarray
    B_K: np.ndarray          # [R, nh*H]
    B_V: np.ndarray
    L: np.ndarray            # int32 [nb]
    dt: str = "bf16"         # storage dtype of every tensor above except L


def make_shared_inputs(nb, nh, H, R, L, L_cap, *, seed, dt="bf16", q_gain=1.0) -> SharedInputs:
    """Draw a shared-latent decode step: latents N(0, 1)/sqrt(R), factors
    N(0, 1)/sqrt(H), q N(0, 1) q_gain/sqrt(H), so a reconstructed key has
    the per-entry variance (1/H) of the per-head workloads.  Cache rows at or
    beyond L[b] are zero."""
    L = np.broadcast_to(np.asarray(L, dtype=np.int32), (nb,)).copy()
    q = np.stack([_normal(seed, (T_SQ, b), (nh, H), q_gain / np.sqrt(H)) for b in range(nb)])

    def lat(tid):
        out = np.zeros((nb, L_cap, R), np.float32)
        for b in range(nb):
            n = int(min(max(L[b], 0), L_cap))
            out[b, :n] = _normal(seed, (tid, b), (n, R), 1.0 / np.sqrt(R))
        return out

    C_K, C_V = lat(T_SCK), lat(T_SCV)
    B_K = _normal(seed, (T_SBK,), (R, nh * H), 1.0 / np.sqrt(H))
    B_V = _normal(seed, (T_SBV,), (R, nh * H), 1.0 / np.sqrt(H))
    return SharedInputs(nb=nb, nh=nh, H=H, R=R, L_cap=L_cap, q=_store(q, dt), C_K=_store(C_K, dt),
                        C_V=_store(C_V, dt), B_K=_store(B_K, dt), B_V=_store(B_V, dt), L=L, dt=dt)
