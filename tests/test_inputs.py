"""The seeded generators and the byte model (CPU)."""
import numpy as np
import pytest

from rank_kv_cache_flash_amd import inputs as I
from rank_kv_cache_flash_amd.configs import CONFIGS


def test_deterministic_and_keyed_per_sequence():
    a = I.make_decode_inputs(3, 2, 16, 8, 10, 12, seed=5)
    b = I.make_decode_inputs(3, 2, 16, 8, 10, 12, seed=5)
    c = I.make_decode_inputs(5, 2, 16, 8, 10, 12, seed=5)
    for k in ("q", "C_K", "C_V", "B_K", "B_V"):
        np.testing.assert_array_equal(getattr(a, k), getattr(b, k))
    np.testing.assert_array_equal(a.C_K, c.C_K[:3])
    np.testing.assert_array_equal(a.q, c.q[:3])
    d = I.make_decode_inputs(3, 2, 16, 8, 10, 12, seed=6)
    assert not np.array_equal(a.C_K, d.C_K)
    # rows past L are zero
    assert not a.C_K[:, :, 10:].any()


def test_bf16_storage_rounding_matches_torch():
    import torch
    x = np.random.default_rng(0).standard_normal(10000).astype(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(I.f32_to_bf16_bits(x), want)


def test_value_scales():
    inp = I.make_decode_inputs(2, 4, 128, 32, 512, 512, seed=3, act_dt="f32", C_dt="f32")
    assert abs(inp.q.std() * np.sqrt(128) - 1) < 0.05
    assert abs(inp.C_K.std() * np.sqrt(32) - 1) < 0.02
    assert abs(inp.B_V.std() * np.sqrt(128) - 1) < 0.05


def test_int8_rows_properties():
    g = np.random.default_rng(1)
    c = (g.standard_normal((50, 64, 32)) / np.sqrt(32)).astype(np.float32)
    c[3, 5] = 0.0
    codes, sc = I._int8_rows(c)
    assert codes.dtype == np.int8 and sc.dtype == np.float16
    assert np.abs(codes.astype(int)).max() <= 127
    assert sc[3, 5] == 0 and not codes[3, 5].any()
    nz = sc.astype(np.float32) > 0
    top = np.abs(codes.astype(int)).max(-1)
    assert np.all(top[nz] >= 126)
    deq = codes.astype(np.float64) * sc.astype(np.float64)[..., None]
    err = np.abs(deq - c)
    # half a step, plus the clamp when the fp16 scale rounded down
    assert np.all(err <= sc.astype(np.float64)[..., None] * 0.5 + 1e-3 * np.abs(c).max(-1, keepdims=True))


def test_int8_cache_outliers():
    inp = I.make_decode_inputs(2, 4, 128, 32, 256, 256, seed=9, C_dt="i8", outlier_p=0.01,
                               outlier_mul=20.0)
    assert inp.C_K.dtype == np.int8 and inp.s_K.shape == (2, 4, 256)
    assert np.all(inp.s_K.astype(np.float32) > 0)
    m = I._rng(9, I.T_MK, 0).random((4, 256, 32), dtype=np.float32) < np.float32(0.01)
    assert 0.007 < m.mean() < 0.013
    # rows holding an outlier have a much larger scale than rows without
    has = m.any(-1)
    s = inp.s_K[0].astype(np.float32)
    assert np.median(s[has]) > 5 * np.median(s[~has])


def test_ragged_step_inputs():
    inp = I.make_ragged_step_inputs(6, 2, 16, 8, 32, 4, 9, 12, seed=11)
    assert np.all((inp.L >= 4) & (inp.L <= 9))
    np.testing.assert_array_equal(inp.pos, inp.L - 1)
    for b in range(6):
        assert not inp.C_K[b, :, inp.L[b] - 1:].any()
        assert inp.C_K[b, :, : inp.L[b] - 1].any()
    assert inp.x.shape == (6, 32) and inp.A_K.shape == (32, 16)


def test_byte_model_matches_hand_totals():
    assert CONFIGS[1].decode_bytes() == 165_888
    assert CONFIGS[2].decode_bytes() == 4_997_120
    assert CONFIGS[3].decode_bytes() == 538_181_632
    assert CONFIGS[4].decode_bytes() == 143_654_912
    c5 = CONFIGS[5]
    assert c5.append_bytes() == 26_083_328
    L = c5.draw_L()
    assert c5.decode_bytes(L) == 6_144 * int(L.sum()) + 786_432 + 1_048_576
    assert np.all((L >= 1024) & (L <= 8192))


@pytest.mark.parametrize("C_dt,act", [("f32", "f32"), ("bf16", "bf16"), ("i8", "bf16")])
def test_score_shift_construction(C_dt, act):
    """add_score_shift: every score of a head moves by one constant of about
    1000 (scores written out here as sigma * sum_i c_i (B_K q)_i from the
    stored values, independently of the oracle), and the oracle's output is
    unchanged by it (softmax is shift invariant; an oracle without its max
    subtraction would overflow at these scores)."""
    import oracle as O
    L = np.array([300, 1, 0, 129], np.int32)
    inp = I.make_decode_inputs(4, 3, 128, 32, L, 300, seed=11, act_dt=act, C_dt=C_dt, q_gain=4.0 * 128)
    sh = I.add_score_shift(inp)
    tw = sh.meta["unshifted"]
    assert 990.0 < sh.meta["score_shift"] < 1010.0
    assert not np.array_equal(inp.q, sh.q)            # the input was copied, not changed in place

    def scores(x, b, h):
        n = int(x.L[b])
        c = O.upcast(x.C_K[b, h, :n], x.C_dt)
        if x.C_dt == "i8":
            c = c * O.upcast(x.s_K[b, h, :n], "f16")[:, None]
        qp = O.upcast(x.B_K[h], x.B_dt) @ O.upcast(x.q[b, h], x.q_dt)      # [r]
        return np.array([sum(c[t, i] * qp[i] for i in range(x.r)) for t in range(n)]) / np.sqrt(128)

    for b, h in ((0, 0), (0, 2), (1, 1), (3, 2)):
        d = scores(sh, b, h) - scores(tw, b, h)
        np.testing.assert_allclose(d, sh.meta["score_shift"], rtol=1e-12)
    a, t = O.decode_attn(sh), O.decode_attn(tw)
    assert np.all(np.isfinite(a))
    assert np.max(np.abs(a - t)) <= 1e-9 * np.max(np.abs(t))
    assert not a[2].any()                               # L = 0 still gives a zero row
