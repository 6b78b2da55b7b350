"""Pins of the fp64 oracle against facts that do not come from the oracle.

Each test ties one part of the oracle to a closed form, a library routine,
an exact invariant, or hand-checked values, so a dropped term, wrong sign,
wrong index or transposed operand fails at least one of them (see
test_oracle_mutants.py, which plants such mistakes and checks that).
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import scipy.linalg
import scipy.special
import torch

import oracle as O
from rank_kv_cache_flash_amd.inputs import DecodeInputs

RNG = np.random.default_rng(12345)


def _inp_f64(q, CK, CV, BK, BV, L=None, s_K=None, s_V=None, C_dt="f64"):
    """Wrap float64 arrays as a one-sequence DecodeInputs ([1, nh, ...])."""
    q = np.asarray(q)[None] if q.ndim == 2 else np.asarray(q)
    CK = CK[None] if CK.ndim == 3 else CK
    CV = CV[None] if CV.ndim == 3 else CV
    nb, nh, L_cap, r = CK.shape
    H = q.shape[-1]
    L = np.full(nb, L_cap, np.int32) if L is None else np.asarray(L, np.int32)
    return DecodeInputs(nb=nb, nh=nh, H=H, r=r, L_cap=L_cap, q=q, q_dt="f64", C_K=CK, C_V=CV,
                        C_dt=C_dt, B_K=BK, B_V=BV, B_dt="f64", L=L, out_dt="f64",
                        s_K=s_K, s_V=s_V)


def _sdpa(q, K, V, sigma):
    """torch's scaled_dot_product_attention in float64 on the CPU."""
    qt = torch.tensor(q, dtype=torch.float64).reshape(1, 1, 1, -1)
    Kt = torch.tensor(K, dtype=torch.float64).reshape(1, 1, K.shape[0], -1)
    Vt = torch.tensor(V, dtype=torch.float64).reshape(1, 1, V.shape[0], -1)
    o = torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt, scale=sigma)
    return o.reshape(-1).numpy()


# ---------------------------------------------------------------------------
# storage dtypes
# ---------------------------------------------------------------------------
def test_bf16_bit_patterns():
    pats = np.array([0x3F80, 0xBF80, 0x4000, 0x3F00, 0x4049, 0x0001, 0x7F7F, 0x8000, 0x0080],
                    dtype=np.uint16)
    want = [1.0, -1.0, 2.0, 0.5, 3.140625, 2.0 ** -133, (2 - 2.0 ** -7) * 2.0 ** 127, -0.0,
            2.0 ** -126]
    got = O.upcast(pats, "bf16")
    for g, w in zip(got, want):
        assert g == w and math.copysign(1, g) == math.copysign(1, w)


def test_bf16_upcast_matches_torch():
    bits = RNG.integers(0, 2 ** 16, size=4096, dtype=np.uint16)
    bits = bits[((bits >> 7) & 0xFF) != 0xFF]          # finite patterns only
    t = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64)
    np.testing.assert_array_equal(O.upcast(bits, "bf16"), t.numpy())


def test_round_to_bf16_ties_by_hand():
    one = 1.0
    cases = {
        one + 2.0 ** -8: 0x3F80,                   # halfway 1 .. 1+2^-7 -> even (1.0)
        one + 3 * 2.0 ** -8: 0x3F82,               # halfway 1+2^-7 .. 1+2^-6 -> even
        one + 2.0 ** -8 + 2.0 ** -30: 0x3F81,      # just above the tie
        -(one + 2.0 ** -8 - 2.0 ** -40): 0xBF80,   # just below the tie, negative
        2.0 ** -133 * 0.5: 0x0000,                 # half the smallest subnormal -> even (0)
        2.0 ** -133 * 1.5: 0x0002,                 # 1.5 ulp subnormal -> even (2 ulp)
        0.0: 0x0000,
    }
    for v, bits in cases.items():
        assert int(O.round_to_bf16_bits(np.array([v]))[0]) == bits, (v, hex(bits))


def test_round_to_bf16_matches_torch_on_float32_values():
    x = (RNG.standard_normal(20000) * np.exp(RNG.uniform(-30, 30, 20000))).astype(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(O.round_to_bf16_bits(x.astype(np.float64)), want)


def test_int8_dequant_exact():
    codes = RNG.integers(-127, 128, size=(3, 5, 16)).astype(np.int8)
    scales = (RNG.uniform(1e-4, 3.0, size=(3, 5))).astype(np.float16)
    got = O.dequant_latent(codes, "i8", scales)
    for idx in np.ndindex(codes.shape):
        exact = Fraction(int(codes[idx])) * Fraction(float(scales[idx[:-1]]))
        assert Fraction(got[idx]) == exact


# ---------------------------------------------------------------------------
# attention special cases
# ---------------------------------------------------------------------------
def test_identity_factor_is_textbook_attention():
    """r = H and B = I: the method reduces to plain attention (library SDPA)."""
    H, L = 16, 37
    q = RNG.standard_normal((2, H))
    CK = RNG.standard_normal((2, L, H))
    CV = RNG.standard_normal((2, L, H))
    I = np.stack([np.eye(H)] * 2)
    inp = _inp_f64(q, CK, CV, I, I)
    sigma = 1 / math.sqrt(H)
    out = O.decode_attn(inp)
    for h in range(2):
        np.testing.assert_allclose(out[0, h], _sdpa(q[h], CK[h], CV[h], sigma), rtol=0, atol=1e-13)


@pytest.mark.parametrize("H,r", [(12, 5), (8, 8)])
def test_scaled_selection_factor_reconstructs_by_indexing(H, r):
    """B with one nonzero per row: K's columns are scaled copies of the
    latent's columns (no matmul needed); then compare with library SDPA.
    The square case uses a cyclic shift, so a transposed factor differs."""
    L = 23
    perm = (np.arange(r) + 1) % H if r == H else RNG.permutation(H)[:r]
    d = RNG.uniform(0.5, 2.0, r) * RNG.choice([-1, 1], r)
    BK = np.zeros((r, H)); BK[np.arange(r), perm] = d
    perm2 = (np.arange(r) + 3) % H if r == H else RNG.permutation(H)[:r]
    d2 = RNG.uniform(0.5, 2.0, r)
    BV = np.zeros((r, H)); BV[np.arange(r), perm2] = d2
    CK = RNG.standard_normal((1, L, r)); CV = RNG.standard_normal((1, L, r))
    q = RNG.standard_normal((1, H))
    K = np.zeros((L, H)); K[:, perm] = CK[0] * d
    V = np.zeros((L, H)); V[:, perm2] = CV[0] * d2
    inp = _inp_f64(q, CK, CV, BK[None], BV[None])
    np.testing.assert_allclose(O.decode_attn(inp)[0, 0], _sdpa(q[0], K, V, 1 / math.sqrt(H)),
                               rtol=0, atol=1e-13)


def test_rank_one_closed_form():
    """r = 1: k_t = c_t b, v_t = d_t g  =>  out = softmax(sigma c (b.q)) . d  * g."""
    H, L = 8, 19
    c = RNG.standard_normal(L); dv = RNG.standard_normal(L)
    b = RNG.standard_normal(H); g = RNG.standard_normal(H); q = RNG.standard_normal(H)
    sigma = 0.7
    p = scipy.special.softmax(sigma * c * float(np.dot(b, q)))
    want = float(np.dot(p, dv)) * g
    inp = _inp_f64(q[None], c[None, :, None], dv[None, :, None], b[None, None, :], g[None, None, :])
    np.testing.assert_allclose(O.decode_attn(inp, softmax_scale=sigma)[0, 0], want, atol=1e-14)


def test_two_tokens_logistic():
    H, r = 6, 3
    BK = RNG.standard_normal((r, H)); BV = RNG.standard_normal((r, H))
    CK = RNG.standard_normal((2, r)); CV = RNG.standard_normal((2, r))
    q = RNG.standard_normal(H)
    k0, k1 = [sum(CK[t, i] * BK[i] for i in range(r)) for t in (0, 1)]
    v0, v1 = [sum(CV[t, i] * BV[i] for i in range(r)) for t in (0, 1)]
    sigma = 1 / math.sqrt(H)
    d = sigma * (float(np.dot(k0, q)) - float(np.dot(k1, q)))
    want = scipy.special.expit(d) * v0 + scipy.special.expit(-d) * v1
    inp = _inp_f64(q[None], CK[None], CV[None], BK[None], BV[None])
    np.testing.assert_allclose(O.decode_attn(inp)[0, 0], want, atol=1e-14)


def test_single_token_returns_its_value_row():
    H, r = 10, 4
    BV = RNG.standard_normal((r, H)); cv = RNG.standard_normal(r)
    v0 = [sum(cv[i] * BV[i, j] for i in range(r)) for j in range(H)]
    inp = _inp_f64(RNG.standard_normal((1, H)), RNG.standard_normal((1, 1, r)), cv[None, None, :],
                   RNG.standard_normal((1, r, H)), BV[None])
    np.testing.assert_allclose(O.decode_attn(inp)[0, 0], v0, rtol=0, atol=1e-14)


def test_zero_query_gives_mean_value():
    H, r, L = 10, 4, 29
    BV = RNG.standard_normal((r, H)); CV = RNG.standard_normal((L, r))
    mean = [sum(sum(CV[t, i] * BV[i, j] for i in range(r)) for t in range(L)) / L for j in range(H)]
    inp = _inp_f64(np.zeros((1, H)), RNG.standard_normal((1, L, r)), CV[None],
                   RNG.standard_normal((1, r, H)), BV[None])
    np.testing.assert_allclose(O.decode_attn(inp)[0, 0], mean, atol=1e-14)


def test_dominant_token_is_selected():
    """One score 1000 above the rest: out is that token's value row, no overflow."""
    H, L = 8, 50
    I = np.eye(H)
    CK = RNG.standard_normal((L, H)) * 0.1
    CK[17] = 0.0; CK[17, 0] = 1000.0 * math.sqrt(H)
    q = np.zeros(H); q[0] = 1.0
    CV = RNG.standard_normal((L, H))
    out = O.decode_attn(_inp_f64(q[None], CK[None], CV[None], I[None], I[None]))[0, 0]
    np.testing.assert_allclose(out, CV[17], rtol=0, atol=1e-12)
    assert np.all(np.isfinite(out))


def test_softmax_weights_sum_shift_and_overflow():
    s = RNG.standard_normal(1000) * 5
    p = O.softmax_weights(s)
    assert abs(p.sum() - 1.0) < 1e-14 and np.all(p > 0)
    np.testing.assert_allclose(O.softmax_weights(s + 1000.0), p, rtol=1e-12)
    np.testing.assert_allclose(p, scipy.special.softmax(s), rtol=1e-13)
    big = O.softmax_weights(s * 1e4)
    assert np.all(np.isfinite(big)) and abs(big.sum() - 1) < 1e-14


def test_token_permutation_invariance():
    H, r, L = 16, 8, 41
    inp = _inp_f64(RNG.standard_normal((1, H)), RNG.standard_normal((1, L, r)),
                   RNG.standard_normal((1, L, r)), RNG.standard_normal((1, r, H)),
                   RNG.standard_normal((1, r, H)))
    perm = RNG.permutation(L)
    inp2 = _inp_f64(inp.q[0], inp.C_K[0][:, perm], inp.C_V[0][:, perm], inp.B_K, inp.B_V)
    np.testing.assert_allclose(O.decode_attn(inp2), O.decode_attn(inp), atol=1e-14)


def test_hadamard_rotation_is_absorbed():
    """c -> c S, B -> S^T B with S an orthonormal Hadamard leaves out unchanged."""
    H, r, L = 32, 16, 33
    S = scipy.linalg.hadamard(r) / math.sqrt(r)
    CK = RNG.standard_normal((1, L, r)); CV = RNG.standard_normal((1, L, r))
    BK = RNG.standard_normal((1, r, H)); BV = RNG.standard_normal((1, r, H))
    q = RNG.standard_normal((1, H))
    a = O.decode_attn(_inp_f64(q, CK, CV, BK, BV))
    b = O.decode_attn(_inp_f64(q, (CK[0] @ S)[None], (CV[0] @ S)[None], (S.T @ BK[0])[None],
                              (S.T @ BV[0])[None]))
    np.testing.assert_allclose(a, b, atol=1e-12)


def test_factor_product_associativity():
    """(c B) q == c (B q): reconstruct-then-dot equals the folded query."""
    H, r, L = 24, 8, 15
    c = RNG.standard_normal((L, r)); B = RNG.standard_normal((r, H)); q = RNG.standard_normal(H)
    K = O.reconstruct(c, B)
    qf = [sum(B[i, j] * q[j] for j in range(H)) for i in range(r)]
    want = [sum(c[t, i] * qf[i] for i in range(r)) for t in range(L)]
    np.testing.assert_allclose(K @ q, want, atol=1e-12)


def test_brute_force_tiny():
    """Everything in pure-Python loops with math.exp on a 2-head toy."""
    nh, H, r, L = 2, 3, 2, 4
    q = RNG.standard_normal((nh, H)); CK = RNG.standard_normal((nh, L, r))
    CV = RNG.standard_normal((nh, L, r)); BK = RNG.standard_normal((nh, r, H))
    BV = RNG.standard_normal((nh, r, H))
    out = O.decode_attn(_inp_f64(q, CK, CV, BK, BV))
    sig = 1 / math.sqrt(H)
    for h in range(nh):
        K = [[sum(CK[h, t, i] * BK[h, i, j] for i in range(r)) for j in range(H)] for t in range(L)]
        V = [[sum(CV[h, t, i] * BV[h, i, j] for i in range(r)) for j in range(H)] for t in range(L)]
        s = [sig * sum(K[t][j] * q[h, j] for j in range(H)) for t in range(L)]
        m = max(s)
        w = [math.exp(x - m) for x in s]
        z = sum(w)
        o = [sum(w[t] * V[t][j] for t in range(L)) / z for j in range(H)]
        np.testing.assert_allclose(out[0, h], o, atol=1e-14)


# ---------------------------------------------------------------------------
# splits and the merge
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("ell,S", [(1, 1), (10, 1), (10, 2), (10, 3), (10, 7), (10, 10), (10, 13),
                                   (1088, 8), (257, 4)])
def test_split_bounds_partition(ell, S):
    b = O.split_bounds(ell, S)
    assert len(b) == S
    covered = [t for (a, e) in b for t in range(a, e)]
    assert covered == list(range(ell))
    chunk = -(-ell // S)
    assert all(e - a <= chunk for a, e in b)


@pytest.mark.parametrize("S", [1, 2, 3, 7, 41, 50])
def test_split_merge_equals_single_pass(S):
    H, r, L = 16, 8, 41
    q = RNG.standard_normal(H) * 3
    K = RNG.standard_normal((L, r)) @ RNG.standard_normal((r, H))
    V = RNG.standard_normal((L, r)) @ RNG.standard_normal((r, H))
    parts = [O.segment_attend(q, K, V, 0.25, a, e) for a, e in O.split_bounds(L, S)]
    o = np.array([p[0] for p in parts]); lse = np.array([p[1] for p in parts])
    np.testing.assert_allclose(O.combine(o, lse), O.attend(q, K, V, 0.25), atol=1e-13)
    # lse of the whole range, merged by log-sum-exp of the parts
    s = 0.25 * (K @ q)
    assert abs(scipy.special.logsumexp(lse[np.isfinite(lse)]) - scipy.special.logsumexp(s)) < 1e-12


def test_segment_lse_is_logsumexp():
    s_full = RNG.standard_normal(30)
    K = np.eye(30); q = s_full.copy(); V = RNG.standard_normal((30, 4))
    o, lse = O.segment_attend(q, K, V, 1.0, 5, 17)
    assert abs(lse - scipy.special.logsumexp(s_full[5:17])) < 1e-13
    np.testing.assert_allclose(o, scipy.special.softmax(s_full[5:17]) @ V[5:17], atol=1e-14)
    o0, l0 = O.segment_attend(q, K, V, 1.0, 9, 9)
    assert l0 == -math.inf and not o0.any()


def test_combine_closed_forms():
    a = RNG.standard_normal(5); b = RNG.standard_normal(5)
    np.testing.assert_allclose(O.combine(np.stack([a, b]), np.array([2.0, 2.0])), (a + b) / 2, atol=1e-15)
    np.testing.assert_allclose(O.combine(np.stack([a, b]), np.array([-math.inf, 7.0])), b, atol=0)
    w = scipy.special.expit(1.5)   # lse difference 1.5 -> logistic weight
    np.testing.assert_allclose(O.combine(np.stack([a, b]), np.array([1.5, 0.0])), w * a + (1 - w) * b,
                               atol=1e-15)
    assert not O.combine(np.stack([a, b]), np.array([-math.inf, -math.inf])).any()


def test_zero_length_and_clamp():
    H, r, L = 8, 4, 6
    inp = _inp_f64(RNG.standard_normal((1, H)), RNG.standard_normal((1, L, r)),
                   RNG.standard_normal((1, L, r)), RNG.standard_normal((1, r, H)),
                   RNG.standard_normal((1, r, H)), L=[0])
    assert not O.decode_attn(inp).any()
    inp.L = np.array([L + 100], np.int32)
    full = O.decode_attn(inp)
    inp.L = np.array([L], np.int32)
    np.testing.assert_array_equal(full, O.decode_attn(inp))


def test_partials_of_decode_match_segments():
    H, r, L = 16, 8, 23
    inp = _inp_f64(RNG.standard_normal((1, H)), RNG.standard_normal((1, L, r)),
                   RNG.standard_normal((1, L, r)), RNG.standard_normal((1, r, H)),
                   RNG.standard_normal((1, r, H)))
    o, lse = O.decode_partials_one(inp, 0, 0, 4)
    np.testing.assert_allclose(O.combine(o, lse), O.decode_attn(inp)[0, 0], atol=1e-13)
    assert O.split_bounds(L, 4) == [(0, 6), (6, 12), (12, 18), (18, 23)]


# ---------------------------------------------------------------------------
# append
# ---------------------------------------------------------------------------
def test_append_brute_force_and_associativity():
    nb, E, nh, r, H = 3, 7, 2, 3, 5
    x = RNG.standard_normal((nb, E)); A = RNG.standard_normal((E, nh * r))
    c = O.append_latents(x, "f64", A, "f64", nh, r)
    for b in range(nb):
        for h in range(nh):
            for i in range(r):
                want = sum(x[b, e] * A[e, h * r + i] for e in range(E))
                assert abs(c[b, h, i] - want) < 1e-13
    B = RNG.standard_normal((r, H))
    for h in range(nh):
        np.testing.assert_allclose(c[:, h] @ B, x @ (A[:, h * r:(h + 1) * r] @ B), atol=1e-12)


def test_apply_append_writes_rounded_row_at_pos():
    from rank_kv_cache_flash_amd.inputs import make_ragged_step_inputs
    inp = make_ragged_step_inputs(3, 2, 16, 8, 32, 4, 9, 12, seed=7)
    CK, CV, cK, cV = O.apply_append(inp)
    for b in range(3):
        p = int(inp.pos[b])
        assert p == inp.L[b] - 1
        np.testing.assert_array_equal(CK[b, :, p], O.round_to_bf16_bits(cK[b]))
        np.testing.assert_array_equal(np.delete(CK[b], p, axis=1), np.delete(inp.C_K[b], p, axis=1))
        # rounded row within half a bf16 ulp of the exact latent
        back = O.upcast(CK[b, :, p], "bf16")
        ulp = np.ldexp(1.0, np.frexp(np.abs(cK[b]))[1] - 8)
        assert np.all(np.abs(back - cK[b]) <= ulp / 2 + 1e-300)


# ---------------------------------------------------------------------------
# int8 latent rows (symmetric absmax, fp16 scale): hand-worked values
# ---------------------------------------------------------------------------
def test_int8_rows_hand_worked():
    # absmax 1: 1/127 = 0.0078740... rounds to fp16 1032 * 2^-17; then
    # 0.5 / s = 63.504 -> 64, 1 / s = 127.008 -> 127, 0.25 / s = 31.752 -> 32.
    codes, scale = O.quantize_latent_rows(np.array([[0.5, -1.0, 0.25, 0.0]]))
    assert float(scale[0]) == 1032 * 2.0 ** -17
    assert codes.tolist() == [[64, -127, 32, 0]]
    assert codes.dtype == np.int8 and scale.dtype == np.float16


def test_int8_rows_ties_go_to_even():
    # absmax 127 * 2^-7 makes the scale exactly 2^-7: ratios 2.5 and 3.5 and -0.5 are ties.
    s = 2.0 ** -7
    codes, scale = O.quantize_latent_rows(np.array([[127 * s, 2.5 * s, 3.5 * s, -0.5 * s, -1.5 * s]]))
    assert float(scale[0]) == s
    assert codes.tolist() == [[127, 2, 4, 0, -2]]


def test_int8_rows_zero_row_and_clamp():
    # zero row: scale 0, codes 0
    codes, scale = O.quantize_latent_rows(np.zeros((2, 3)))
    assert np.all(scale == 0) and np.all(codes == 0)
    # absmax / 127 = 1.4 * 2^-24 rounds down to the smallest fp16 subnormal 2^-24,
    # so the largest entries sit at 177.8 scales: they clamp to +-127, 2^-24 itself is code 1.
    t = 2.0 ** -24
    codes, scale = O.quantize_latent_rows(np.array([[127 * 1.4 * t, -127 * 1.4 * t, 0.0, t]]))
    assert float(scale[0]) == t
    assert codes.tolist() == [[127, -127, 0, 1]]


def test_int8_rows_error_bound():
    # With normal (not subnormal) fp16 scales, code * scale is within half a scale of the
    # value (plus fp32 rounding) and the absmax entry maps to +-127.
    rng = np.random.default_rng(7)
    c = rng.standard_normal((50, 48)) * np.exp(rng.uniform(-4, 4, (50, 1)))
    codes, scale = O.quantize_latent_rows(c)
    s = scale.astype(np.float64)[:, None]
    err = np.abs(codes * s - c)
    assert np.all(err <= 0.5 * s * (1 + 1e-6) + np.abs(c) * 2.0 ** -23)
    assert np.all(scale >= np.float16(2.0 ** -14))
    assert np.all(np.abs(codes).max(axis=1) == 127)


def test_apply_append_int8_writes_codes_and_scales_at_pos():
    from rank_kv_cache_flash_amd import inputs as I
    inp = I.make_ragged_step_inputs(3, 2, 64, 16, 256, 3, 9, 9, seed=8, C_dt="i8")
    inp.pos[2] = 9                                       # out of range: row left alone
    CK, CV, sK, sV, cK, cV = O.apply_append_int8(inp)
    for b in range(2):
        p = int(inp.pos[b])
        for h in range(2):
            deq = CK[b, h, p].astype(np.float64) * float(sK[b, h, p])
            assert np.all(np.abs(deq - cK[b, h]) <= 0.5 * float(sK[b, h, p]) * (1 + 1e-6) + 1e-12)
            assert np.abs(CV[b, h, p]).max() == 127
        # every other row untouched
        keep = np.ones(inp.L_cap, bool); keep[p] = False
        assert np.array_equal(CK[b][:, keep], inp.C_K[b][:, keep])
        assert np.array_equal(sK[b][:, keep], np.asarray(inp.s_K[b])[:, keep])
    assert np.array_equal(CK[2], inp.C_K[2]) and np.array_equal(sV[2], np.asarray(inp.s_V[2]))


# ---------------------------------------------------------------------------
# W8A8 projection: Hadamard rotation, per-row fp32-scale codes, integer product
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("n", [1, 2, 4, 8, 64])
def test_hadamard_matrix_is_sylvester(n):
    h = O.hadamard_matrix(n)
    assert np.array_equal(h, scipy.linalg.hadamard(n))
    assert np.array_equal(h @ h.T, n * np.eye(n, dtype=np.int64))


def test_rotation_hand_worked_and_orthogonal():
    # H_4 = [[1,1,1,1],[1,-1,1,-1],[1,1,-1,-1],[1,-1,-1,1]]; [1,2,3,4] H_4 = [10,-2,-4,0]; / sqrt(4)
    assert np.allclose(O.rotate_rows(np.array([[1.0, 2.0, 3.0, 4.0]]), "f64"), [[5.0, -1.0, -2.0, 0.0]], atol=0)
    x = RNG.standard_normal((3, 256))
    xr = O.rotate_rows(x, "f64")
    assert np.allclose(np.linalg.norm(xr, axis=1), np.linalg.norm(x, axis=1), rtol=1e-12)
    assert np.allclose(O.rotate_rows(xr, "f64"), x, atol=1e-12)       # H_E / sqrt(E) squares to I


def test_quantize_rows_f32_hand_worked():
    # scale fp32(1/127); 0.5 / scale rounds to 63.5 in fp32 and the tie goes to 64;
    # 1 / scale = 127.0000005 -> 127; 0.25 / scale -> 31.75 -> 32.
    codes, scale = O.quantize_rows_f32(np.array([[0.5, -1.0, 0.25, 0.0]]))
    assert scale.dtype == np.float32 and scale[0] == np.float32(1.0) / np.float32(127.0)
    assert codes.tolist() == [[64, -127, 32, 0]]
    s = 2.0 ** -7                                   # exact scale: 2.5, 3.5, -0.5, -1.5 are ties
    codes, scale = O.quantize_rows_f32(np.array([[127 * s, 2.5 * s, 3.5 * s, -0.5 * s, -1.5 * s]]))
    assert scale[0] == s and codes.tolist() == [[127, 2, 4, 0, -2]]
    codes, scale = O.quantize_rows_f32(np.zeros((1, 5)))
    assert scale[0] == 0 and not codes.any()


def test_prepare_factor_of_identity():
    # A = I_4: A' = H_4 / 2, every column is +-1/2, so scale 1/254 and codes 127 * sign pattern of H_4.
    AqT, sA = O.prepare_factor(np.eye(4), "f64")
    assert np.array_equal(AqT.astype(np.int64), 127 * scipy.linalg.hadamard(4).T)
    assert np.all(sA == np.float32(0.5) / np.float32(127.0))


def test_w8a8_latents_brute_force():
    xq = RNG.integers(-127, 128, (3, 8)).astype(np.int8)
    AqT = RNG.integers(-127, 128, (6, 8)).astype(np.int8)
    sx = np.array([0.5, 0.25, 2.0], np.float32)
    sA = np.linspace(0.1, 0.6, 6).astype(np.float32)
    got = O.w8a8_latents(xq, sx, AqT, sA, nh=2, r=3)
    for b in range(3):
        for n in range(6):
            acc = sum(int(xq[b, e]) * int(AqT[n, e]) for e in range(8))
            assert got[b, n // 3, n % 3] == acc * float(sx[b]) * float(sA[n])


def test_w8a8_exact_case_and_error_bound():
    # x = 1/2 everywhere rotates to (1, 0, 0, 0): codes exact; with A = I the pipeline returns x.
    xq, sx = O.quantize_activations(np.full((1, 4), 0.5), "f64")
    assert xq.tolist() == [[127, 0, 0, 0]]
    AqT, sA = O.prepare_factor(np.eye(4), "f64")
    c = O.w8a8_latents(xq, sx, AqT, sA, nh=1, r=4)
    assert np.allclose(c.reshape(1, 4), 0.5, rtol=1e-7)
    # random data: |w8a8 - x.A| within the two half-step quantisation errors
    E, N = 256, 24
    x = RNG.standard_normal((4, E)) / 16
    A = RNG.standard_normal((E, N)) / 4
    xq, sx = O.quantize_activations(x, "f64")
    AqT, sA = O.prepare_factor(A, "f64")
    c = O.w8a8_latents(xq, sx, AqT, sA, nh=2, r=12).reshape(4, N)
    xr = O.rotate_rows(x, "f64")
    Ar = (scipy.linalg.hadamard(E) @ A) / np.sqrt(E)
    bound = (sx[:, None] / 2) @ np.abs(Ar).sum(0)[None, :] + np.abs(xr).sum(1)[:, None] * (sA[None, :] / 2) * (1 + 1e-6)
    assert np.all(np.abs(c - x @ A) <= bound * 1.01 + 1e-12)


# ---------------------------------------------------------------------------
# rotary position step on reconstructed keys
# ---------------------------------------------------------------------------
def test_rope_hand_worked():
    # H = 4, base 16: theta = (1, 16^-1/2 = 1/4).  At t = 2 pi pair (0, 2) turns a full circle
    # and pair (1, 3) a quarter: (x1, x3) -> (-x3, x1).
    got = O.rope_rotate(np.array([[1.0, 2.0, 3.0, 4.0]]), [2 * math.pi], base=16.0)
    assert np.allclose(got, [[1.0, -4.0, 3.0, 2.0]], atol=1e-12)
    # t = 0 is the identity
    x = RNG.standard_normal((3, 8))
    assert np.array_equal(O.rope_rotate(x, [0, 0, 0]), x)


def test_rope_rotation_properties():
    H = 64
    q = RNG.standard_normal(H)
    k = RNG.standard_normal(H)
    X = RNG.standard_normal((5, H))
    t = np.array([0, 3, 17, 250, 4095])
    R = O.rope_rotate(X, t)
    assert np.allclose(np.linalg.norm(R, axis=1), np.linalg.norm(X, axis=1), rtol=1e-12)
    assert np.allclose(O.rope_rotate(R, t + 5), O.rope_rotate(X, 2 * t + 5), atol=1e-9)
    for m, n in [(10, 3), (1000, 999), (7, 7)]:
        lhs = O.rope_rotate(q[None], [m]) @ O.rope_rotate(k[None], [n]).T
        rhs = O.rope_rotate(q[None], [m - n]) @ k[None].T
        assert np.allclose(lhs, rhs, rtol=1e-9, atol=1e-9)


def test_rope_matches_explicit_plane_rotations():
    # each pair (i, i + H/2) is an explicit 2x2 rotation by t * base^(-2 i / H)
    H, base = 8, 100.0
    x = RNG.standard_normal(H)
    for t in (1, 6, 33):
        want = np.empty(H)
        for i in range(H // 2):
            a = t * base ** (-2.0 * i / H)
            rot = np.array([[math.cos(a), -math.sin(a)], [math.sin(a), math.cos(a)]])
            want[i], want[i + H // 2] = rot @ np.array([x[i], x[i + H // 2]])
        assert np.allclose(O.rope_rotate(x[None], [t], base=base)[0], want, atol=1e-12)


def test_rope_decode_one_token_and_brute_force():
    rng = np.random.default_rng(31)
    nh, H, r, L = 2, 8, 4, 5
    q = rng.standard_normal((nh, H))
    CK, CV = rng.standard_normal((nh, L, r)), rng.standard_normal((nh, L, r))
    BK, BV = rng.standard_normal((nh, r, H)), rng.standard_normal((nh, r, H))
    inp = _inp_f64(q, CK, CV, BK, BV)
    got = O.decode_attn_rope(inp, base=50.0)
    for h in range(nh):
        K = O.rope_rotate(CK[h] @ BK[h], np.arange(L), base=50.0)
        s = (K @ q[h]) / math.sqrt(H)
        p = np.exp(s - s.max()); p /= p.sum()
        assert np.allclose(got[0, h], p @ (CV[h] @ BV[h]), rtol=1e-12, atol=1e-12)
    # one cached token sits at position 0: no rotation, same as the plain decode
    inp1 = _inp_f64(q, CK[:, :1], CV[:, :1], BK, BV)
    assert np.allclose(O.decode_attn_rope(inp1), O.decode_attn(inp1), atol=1e-12)


# ---------------------------------------------------------------------------
# offline per-head factorisation (truncated SVD; weighted alternating least squares)
# ---------------------------------------------------------------------------
def test_svd_factors_eckart_young():
    rng = np.random.default_rng(41)
    E, nh, H, r = 40, 2, 8, 3
    W = rng.standard_normal((E, nh * H))
    A, B = O.svd_factors(W, nh, r)
    for h in range(nh):
        Wh = W[:, h * H:(h + 1) * H]
        err = np.sum((Wh - A[:, h * r:(h + 1) * r] @ B[h]) ** 2)
        lam = np.sort(np.linalg.eigvalsh(Wh.T @ Wh))[::-1]       # squared singular values
        assert np.isclose(err, lam[r:].sum(), rtol=1e-10)
        assert np.allclose(B[h] @ B[h].T, np.eye(r), atol=1e-12)
    A, B = O.svd_factors(W, nh, H)                               # full rank: exact
    assert np.allclose(np.concatenate([A[:, h * H:(h + 1) * H] @ B[h] for h in range(nh)], axis=1), W, atol=1e-12)


def test_svd_factors_hand_and_low_rank():
    A, B = O.svd_factors(np.array([[3.0, 0.0], [0.0, 1.0], [0.0, 0.0]]), 1, 1)
    assert np.allclose(A @ B[0], [[3.0, 0.0], [0.0, 0.0], [0.0, 0.0]], atol=1e-12)
    rng = np.random.default_rng(42)
    X, Y = rng.standard_normal((30, 4)), rng.standard_normal((4, 6))
    A, B = O.svd_factors(X @ Y, 1, 4)
    assert np.allclose(A @ B[0], X @ Y, atol=1e-10)


def test_weighted_als_properties():
    rng = np.random.default_rng(43)
    E, nh, H, r = 24, 2, 6, 2
    W = rng.standard_normal((E, nh * H))
    F = rng.uniform(0.1, 3.0, (E, nh * H))
    A, B = O.svd_factors(W, nh, r)
    objs = [O.weighted_objective(W, F, A, B, nh)]
    for _ in range(4):
        A = O.als_step_A(W, F, B, nh)
        objs.append(O.weighted_objective(W, F, A, B, nh))
        # the A step is a minimiser: moving any row makes it worse
        for _ in range(3):
            D = np.zeros_like(A)
            D[rng.integers(E), rng.integers(nh * r)] = 1e-3
            assert np.all(O.weighted_objective(W, F, A + D, B, nh) >= objs[-1] - 1e-12)
        B = O.als_step_B(W, F, A, nh)
        objs.append(O.weighted_objective(W, F, A, B, nh))
    objs = np.array(objs)
    assert np.all(np.diff(objs, axis=0) <= 1e-12)              # never increases
    # unit weights: the truncated SVD is a fixed point of the alternation
    A0, B0 = O.svd_factors(W, nh, r)
    A1, B1 = O.weighted_factors(W, np.ones_like(W), A0, B0, nh, 1)
    for h in range(nh):
        assert np.allclose(A1[:, h * r:(h + 1) * r] @ B1[h], A0[:, h * r:(h + 1) * r] @ B0[h], atol=1e-10)


def test_weighted_als_recovers_low_rank():
    rng = np.random.default_rng(44)
    E, H, r = 30, 7, 2
    W = rng.standard_normal((E, r)) @ rng.standard_normal((r, H))
    F = rng.uniform(0.2, 5.0, (E, H))
    A, B = O.weighted_factors(W, F, rng.standard_normal((E, r)), rng.standard_normal((1, r, H)), 1, 60)
    assert O.weighted_objective(W, F, A, B, 1)[0] <= 1e-12 * np.sum(F * W * W)


# ---------------------------------------------------------------------------
# conventional (shared-latent) factorisation
# ---------------------------------------------------------------------------
def _shared_from_per_head(inp):
    """Embed per-head latents and factors in one shared latent of rank
    R = nh r: latent columns [h r, (h + 1) r) hold head h's latent, and the
    factor is block diagonal (head h's rows only feed head h's columns)."""
    from rank_kv_cache_flash_amd.inputs import SharedInputs
    nb, nh, H, r, Lc = inp.nb, inp.nh, inp.H, inp.r, inp.L_cap
    C_K = np.zeros((nb, Lc, nh * r), np.float32)
    C_V = np.zeros_like(C_K)
    B_K = np.zeros((nh * r, nh * H), np.float32)
    B_V = np.zeros_like(B_K)
    for h in range(nh):
        C_K[:, :, h * r:(h + 1) * r] = inp.C_K[:, h]
        C_V[:, :, h * r:(h + 1) * r] = inp.C_V[:, h]
        B_K[h * r:(h + 1) * r, h * H:(h + 1) * H] = inp.B_K[h]
        B_V[h * r:(h + 1) * r, h * H:(h + 1) * H] = inp.B_V[h]
    return SharedInputs(nb=nb, nh=nh, H=H, R=nh * r, L_cap=Lc, q=np.asarray(inp.q, np.float32), C_K=C_K, C_V=C_V,
                        B_K=B_K, B_V=B_V, L=inp.L, dt="f32")


def test_shared_block_diagonal_equals_per_head():
    from rank_kv_cache_flash_amd.inputs import make_decode_inputs
    inp = make_decode_inputs(3, 4, 8, 3, np.array([7, 0, 1], np.int32), 8, seed=51, act_dt="f32", C_dt="f32",
                             q_gain=6.0)
    got = O.decode_attn_shared(_shared_from_per_head(inp))
    assert np.allclose(got, O.decode_attn(inp), rtol=0, atol=1e-12)
    assert not got[1].any()


def test_shared_identity_factors_equal_library_attention():
    """R = nh H and B = I: head h's keys are latent columns [h H, (h + 1) H)."""
    from rank_kv_cache_flash_amd.inputs import SharedInputs
    rng = np.random.default_rng(52)
    nb, nh, H, ell = 2, 3, 4, 6
    R = nh * H
    q = rng.standard_normal((nb, nh, H)).astype(np.float32)
    C_K = rng.standard_normal((nb, ell, R)).astype(np.float32)
    C_V = rng.standard_normal((nb, ell, R)).astype(np.float32)
    I = np.eye(R, dtype=np.float32)
    inp = SharedInputs(nb=nb, nh=nh, H=H, R=R, L_cap=ell, q=q, C_K=C_K, C_V=C_V, B_K=I, B_V=I,
                       L=np.array([ell, ell], np.int32), dt="f32")
    got = O.decode_attn_shared(inp)
    for b in range(nb):
        for h in range(nh):
            Q = torch.tensor(q[b, h], dtype=torch.float64).view(1, 1, 1, H)
            K = torch.tensor(C_K[b, :, h * H:(h + 1) * H], dtype=torch.float64).view(1, 1, ell, H)
            V = torch.tensor(C_V[b, :, h * H:(h + 1) * H], dtype=torch.float64).view(1, 1, ell, H)
            ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V).view(H).numpy()
            assert np.allclose(got[b, h], ref, rtol=0, atol=1e-12)


def test_shared_brute_force_loops():
    from rank_kv_cache_flash_amd.inputs import SharedInputs
    rng = np.random.default_rng(53)
    nb, nh, H, R, ell = 2, 2, 3, 5, 4
    q = rng.standard_normal((nb, nh, H)).astype(np.float32)
    C_K = rng.standard_normal((nb, ell, R)).astype(np.float32)
    C_V = rng.standard_normal((nb, ell, R)).astype(np.float32)
    B_K = rng.standard_normal((R, nh * H)).astype(np.float32)
    B_V = rng.standard_normal((R, nh * H)).astype(np.float32)
    Ls = [4, 3]
    inp = SharedInputs(nb=nb, nh=nh, H=H, R=R, L_cap=ell, q=q, C_K=C_K, C_V=C_V, B_K=B_K, B_V=B_V,
                       L=np.array(Ls, np.int32), dt="f32")
    got = O.decode_attn_shared(inp)
    for b in range(nb):
        for h in range(nh):
            scores = []
            for t in range(Ls[b]):
                acc = 0.0
                for j in range(H):
                    k = sum(float(C_K[b, t, i]) * float(B_K[i, h * H + j]) for i in range(R))
                    acc += float(q[b, h, j]) * k
                scores.append(acc / math.sqrt(H))
            m = max(scores)
            w = [math.exp(s - m) for s in scores]
            for j in range(H):
                num = sum(w[t] * sum(float(C_V[b, t, i]) * float(B_V[i, h * H + j]) for i in range(R))
                          for t in range(Ls[b]))
                assert abs(got[b, h, j] - num / sum(w)) <= 1e-12
