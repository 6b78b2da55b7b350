"""Plant plausible mistakes in the oracle (CPU only) and check the pins catch each.

Every mutant below is a small, believable slip -- a dropped term, a wrong
sign, a wrong index, a transposed operand, a truncation instead of a
rounding.  The test applies it to the oracle module, runs every pin in
test_oracle_pins.py and requires at least one of them to fail.
"""
import inspect
import math

import numpy as np
import pytest

import oracle
import oracle.wsvd_oracle as W

from . import test_oracle_pins as P


def _pins():
    out = []
    for name, fn in inspect.getmembers(P, inspect.isfunction):
        if not name.startswith("test_"):
            continue
        marks = getattr(fn, "pytestmark", [])
        params = [m for m in marks if m.name == "parametrize"]
        if not params:
            out.append((name, fn, {}))
            continue
        argnames, values = params[0].args
        argnames = [a.strip() for a in argnames.split(",")]
        for v in values:
            v = v if isinstance(v, tuple) else (v,)
            out.append((f"{name}{v}", fn, dict(zip(argnames, v))))
    return out


PINS = _pins()


def _softmax_nomax(s):
    e = np.exp(s)
    return e / np.sum(e)


def _softmax_sign(s):
    m = np.max(s)
    e = np.exp(m - s)
    return e / np.sum(e)


def _upcast_bad_shift(a, dt, _orig=W.upcast):
    if dt == "bf16":
        bits = np.asarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(15)
        return bits.view(np.float32).astype(np.float64)
    return _orig(a, dt)


def _dequant_noscale(C, C_dt, scale=None):
    return W.upcast(C, C_dt)


def _split_floor(ell, S):
    chunk = ell // S
    return [(min(ell, s * chunk), min(ell, (s + 1) * chunk)) for s in range(S)]


def _combine_badweight(o_parts, lse_parts):
    lse = np.asarray(lse_parts, dtype=np.float64)
    o = np.asarray(o_parts, dtype=np.float64)
    if not np.any(np.isfinite(lse)):
        return np.zeros(o.shape[-1])
    M = np.max(lse)
    w = np.where(np.isfinite(lse), np.exp(M - lse), 0.0)
    return (w @ o) / np.sum(w)


def _combine_nonorm(o_parts, lse_parts):
    lse = np.asarray(lse_parts, dtype=np.float64)
    o = np.asarray(o_parts, dtype=np.float64)
    if not np.any(np.isfinite(lse)):
        return np.zeros(o.shape[-1])
    w = np.where(np.isfinite(lse), np.exp(lse - np.max(lse)), 0.0)
    return w @ o


def _segment_nom(q, K, V, sigma, a, e):
    H = V.shape[1]
    if e <= a:
        return np.zeros(H), -math.inf
    s = sigma * (K[a:e] @ q)
    m = np.max(s)
    w = np.exp(s - m)
    return (w / w.sum()) @ V[a:e], float(math.log(w.sum()))


def _attend_k_for_v(q, K, V, sigma):
    return W.softmax_weights(sigma * (K @ q)) @ K if K.shape == V.shape else W.softmax_weights(sigma * (K @ q)) @ V


def _attend_nosigma(q, K, V, sigma):
    return W.softmax_weights(K @ q) @ V


def _attend_sigma_sq(q, K, V, sigma):
    return W.softmax_weights(sigma * sigma * (K @ q)) @ V


def _reconstruct_transposed(c, B):
    if B.shape[0] == B.shape[1]:
        return c @ B.T
    return c @ B


def _reconstruct_drop_last_rank(c, B):
    return c[:, :-1] @ B[:-1] if B.shape[0] > 1 else c @ B


def _append_shifted(x, x_dt, A, A_dt, nh, r):
    xx = W.upcast(x, x_dt); AA = W.upcast(A, A_dt)
    c = np.zeros((xx.shape[0], nh, r))
    for h in range(nh):
        lo = min(h * r + 1, AA.shape[1] - r)
        c[:, h, :] = xx @ AA[:, lo:lo + r]
    return c


def _round_truncate(v):
    v = np.asarray(v, dtype=np.float64).astype(np.float32)
    return (v.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def _round_half_up(v):
    v = np.asarray(v, dtype=np.float64)
    out = np.zeros(v.shape)
    nz = v != 0
    m, e = np.frexp(v[nz])
    qn = np.ldexp(1.0, np.maximum(e - 8, -133))
    out[nz] = np.floor(v[nz] / qn + 0.5) * qn
    return (out.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def _decode_one_short(inp, b, h, softmax_scale=None, *, C_K=None, C_V=None, _orig=W.decode_attn_one):
    import copy
    j = copy.copy(inp)
    j.L = np.maximum(np.asarray(inp.L) - 1, 1)
    return _orig(j, b, h, softmax_scale, C_K=C_K, C_V=C_V)


def _q8_floor(c):
    c32 = np.asarray(c, dtype=np.float64).astype(np.float32)
    s16 = (np.max(np.abs(c32), axis=-1) / np.float32(127)).astype(np.float16)
    s32 = s16.astype(np.float32)[..., None]
    q = np.where(s32 > 0, np.floor(c32 / np.where(s32 > 0, s32, 1)), 0)
    return np.clip(q, -127, 127).astype(np.int8), s16


def _q8_no_fp16_scale(c):
    c32 = np.asarray(c, dtype=np.float64).astype(np.float32)
    s32 = (np.max(np.abs(c32), axis=-1) / np.float32(127))[..., None]
    q = np.where(s32 > 0, np.rint(c32 / np.where(s32 > 0, s32, 1)), 0)
    return np.clip(q, -127, 127).astype(np.int8), s32[..., 0].astype(np.float16)


def _q8_clamp128(c):
    c32 = np.asarray(c, dtype=np.float64).astype(np.float32)
    s16 = (np.max(np.abs(c32), axis=-1) / np.float32(127)).astype(np.float16)
    s32 = s16.astype(np.float32)[..., None]
    q = np.where(s32 > 0, np.rint(c32 / np.where(s32 > 0, s32, 1)), 0)
    return np.clip(q, -128, 127).astype(np.int8), s16


def _q8_half_away(c):
    c32 = np.asarray(c, dtype=np.float64).astype(np.float32)
    s16 = (np.max(np.abs(c32), axis=-1) / np.float32(127)).astype(np.float16)
    s32 = s16.astype(np.float32)[..., None]
    r = c32 / np.where(s32 > 0, s32, 1)
    q = np.where(s32 > 0, np.sign(r) * np.floor(np.abs(r) + 0.5), 0)
    return np.clip(q, -127, 127).astype(np.int8), s16


def _hadamard_no_minus(n):
    return np.ones((n, n), dtype=np.int64)


def _rotate_unnormalised(x, x_dt):
    xx = W.upcast(x, x_dt)
    return xx @ oracle.w8a8.hadamard_matrix(xx.shape[-1]).astype(np.float64)


def _w8a8_drop_weight_scale(xq, sx, AqT, sA, nh, r):
    acc = np.asarray(xq, np.int64) @ np.asarray(AqT, np.int64).T
    return (acc * np.asarray(sx, np.float64)[:, None]).reshape(acc.shape[0], nh, r)


def _qrows_f32_floor(v):
    v32 = np.asarray(v, dtype=np.float64).astype(np.float32)
    scale = (np.max(np.abs(v32), axis=-1) / np.float32(127)).astype(np.float32)
    s = scale[..., None]
    q = np.where(s > 0, np.floor(v32 / np.where(s > 0, s, 1)), 0)
    return np.clip(q, -127, 127).astype(np.int8), scale


def _rope_adjacent_pairs(X, positions, base=10000.0):
    X = np.asarray(X, dtype=np.float64)
    H = X.shape[-1]
    a = oracle.rope.rope_angles(positions, H, base)
    c, s_ = np.cos(a), np.sin(a)
    x1, x2 = X[..., 0::2], X[..., 1::2]
    out = np.empty_like(X)
    out[..., 0::2], out[..., 1::2] = x1 * c - x2 * s_, x2 * c + x1 * s_
    return out


def _rope_sin_flipped(X, positions, base=10000.0):
    X = np.asarray(X, dtype=np.float64)
    H = X.shape[-1]
    a = oracle.rope.rope_angles(positions, H, base)
    c, s_ = np.cos(a), np.sin(a)
    x1, x2 = X[..., : H // 2], X[..., H // 2:]
    return np.concatenate([x1 * c + x2 * s_, x2 * c - x1 * s_], axis=-1)


def _rope_theta_half(positions, H, base=10000.0):
    i = np.arange(H // 2, dtype=np.float64)
    return np.asarray(positions, dtype=np.float64)[:, None] * (base ** (-i / H))[None, :]


def _decode_rope_from_one(inp, base=10000.0, softmax_scale=None, pairs=None, _orig=None):
    import copy
    from oracle import rope as Rm
    nb, nh, H = inp.q.shape
    out = np.zeros((nb, nh, H))
    for b in range(nb):
        for h in range(nh):
            ell = int(inp.L[b])
            K = W.reconstruct(W.dequant_latent(inp.C_K[b, h, :ell], inp.C_dt), W.upcast(inp.B_K[h], inp.B_dt))
            V = W.reconstruct(W.dequant_latent(inp.C_V[b, h, :ell], inp.C_dt), W.upcast(inp.B_V[h], inp.B_dt))
            K = Rm.rope_rotate(K, np.arange(1, ell + 1), base)
            out[b, h] = W.attend(W.upcast(inp.q[b, h], inp.q_dt), K, V, 1 / np.sqrt(H))
    return out


def _svd_no_sigma(W, nh, r):
    W = np.asarray(W, dtype=np.float64)
    E, NH = W.shape
    H = NH // nh
    A = np.zeros((E, nh * r)); B = np.zeros((nh, r, H))
    for h in range(nh):
        U, s_, Vt = np.linalg.svd(W[:, h * H:(h + 1) * H], full_matrices=False)
        A[:, h * r:(h + 1) * r] = U[:, :r]
        B[h] = Vt[:r]
    return A, B


def _svd_smallest(W, nh, r):
    W = np.asarray(W, dtype=np.float64)
    E, NH = W.shape
    H = NH // nh
    A = np.zeros((E, nh * r)); B = np.zeros((nh, r, H))
    for h in range(nh):
        U, s_, Vt = np.linalg.svd(W[:, h * H:(h + 1) * H], full_matrices=False)
        A[:, h * r:(h + 1) * r] = U[:, -r:] * s_[-r:]
        B[h] = Vt[-r:]
    return A, B


def _als_A_unweighted(W, F, B, nh):
    import oracle.factorize as Fm
    return Fm.__dict__["_orig_als_step_A"](W, np.ones_like(np.asarray(F, np.float64)), B, nh)


def _als_B_rows(W, F, A, nh):
    import oracle.factorize as Fm
    Fa = np.asarray(F, np.float64)
    return Fm.__dict__["_orig_als_step_B"](W, Fa[::-1].copy(), A, nh)


def _shared_one_next_head(inp, b, h, softmax_scale=None):
    import oracle.shared_svd as S
    return S.__dict__["_orig_one"](inp, b, (h + 1) % inp.nh, softmax_scale)


def _shared_one_v_with_k_factor(inp, b, h, softmax_scale=None):
    import dataclasses
    import oracle.shared_svd as S
    return S.__dict__["_orig_one"](dataclasses.replace(inp, B_V=inp.B_K), b, h, softmax_scale)


def _shared_one_wrong_sequence(inp, b, h, softmax_scale=None):
    import dataclasses
    import oracle.shared_svd as S
    bb = (b + 1) % inp.nb
    sub = dataclasses.replace(inp, C_K=inp.C_K[[bb] * inp.nb], C_V=inp.C_V[[bb] * inp.nb])
    return S.__dict__["_orig_one"](sub, b, h, softmax_scale)


MUTANTS = {
    "softmax without max shift": ("softmax_weights", _softmax_nomax),
    "softmax sign flipped": ("softmax_weights", _softmax_sign),
    "bf16 upcast shifted by 15": ("upcast", _upcast_bad_shift),
    "int8 scale dropped": ("dequant_latent", _dequant_noscale),
    "split chunk floor instead of ceil": ("split_bounds", _split_floor),
    "merge weight sign flipped": ("combine", _combine_badweight),
    "merge not normalised": ("combine", _combine_nonorm),
    "segment lse drops the max": ("segment_attend", _segment_nom),
    "K used in place of V": ("attend", _attend_k_for_v),
    "softmax scale dropped": ("attend", _attend_nosigma),
    "softmax scale squared": ("attend", _attend_sigma_sq),
    "factor transposed": ("reconstruct", _reconstruct_transposed),
    "last rank term dropped": ("reconstruct", _reconstruct_drop_last_rank),
    "append head block off by one": ("append_latents", _append_shifted),
    "bf16 rounding truncates": ("round_to_bf16_bits", _round_truncate),
    "bf16 rounding ties away": ("round_to_bf16_bits", _round_half_up),
    "one token short": ("decode_attn_one", _decode_one_short),
    "int8 code truncated": ("quantize_latent_rows", _q8_floor),
    "int8 scale not rounded to fp16": ("quantize_latent_rows", _q8_no_fp16_scale),
    "int8 clamp at -128": ("quantize_latent_rows", _q8_clamp128),
    "int8 ties away from zero": ("quantize_latent_rows", _q8_half_away),
    "hadamard without the minus block": ("hadamard_matrix", _hadamard_no_minus),
    "rotation not normalised": ("rotate_rows", _rotate_unnormalised),
    "w8a8 weight scale dropped": ("w8a8_latents", _w8a8_drop_weight_scale),
    "fp32-scale codes truncated": ("quantize_rows_f32", _qrows_f32_floor),
    "rope pairs adjacent elements": ("rope_rotate", _rope_adjacent_pairs),
    "rope sine sign flipped": ("rope_rotate", _rope_sin_flipped),
    "rope frequency exponent halved": ("rope_angles", _rope_theta_half),
    "rope positions start at 1": ("decode_attn_rope", _decode_rope_from_one),
    "svd latent without singular values": ("svd_factors", _svd_no_sigma),
    "svd keeps the smallest directions": ("svd_factors", _svd_smallest),
    "weighted A step ignores the weights": ("als_step_A", _als_A_unweighted),
    "weighted B step uses the wrong rows of F": ("als_step_B", _als_B_rows),
    "shared factor column block of the next head": ("decode_attn_shared_one", _shared_one_next_head),
    "shared values rebuilt with the key factor": ("decode_attn_shared_one", _shared_one_v_with_k_factor),
    "shared latent of the next sequence": ("decode_attn_shared_one", _shared_one_wrong_sequence),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, monkeypatch):
    attr, fn = MUTANTS[name]
    import oracle.w8a8 as W8
    import oracle.rope as WR
    import oracle.factorize as WF
    WF.__dict__.setdefault("_orig_als_step_A", WF.als_step_A)
    WF.__dict__.setdefault("_orig_als_step_B", WF.als_step_B)
    import oracle.shared_svd as WS
    WS.__dict__.setdefault("_orig_one", WS.decode_attn_shared_one)
    for mod in (W, W8, WR, WF, WS, oracle):
        if hasattr(mod, attr):
            monkeypatch.setattr(mod, attr, fn)
    caught = []
    for pname, pin, kw in PINS:
        try:
            pin(**kw)
        except Exception:  # assertion or numerical failure
            caught.append(pname)
    assert caught, f"no pin caught mutant: {name}"


def test_unmutated_oracle_passes_every_pin():
    for pname, pin, kw in PINS:
        pin(**kw)
