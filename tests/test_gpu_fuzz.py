"""Seeded random shapes across the supported space, every output element
against the fp64 oracle: the folded decode (all cache and activation dtypes,
split counts, output dtypes, softmax scales), the rotary-key decode, the
shared-latent decode, the dense baseline, the appends and the stand-alone
merge.  Each case is drawn from its own seed and printed before it runs."""
import numpy as np
import pytest

import oracle as O
from rank_kv_cache_flash_amd import inputs as I

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 2e-2, "i8": 2e-2}


@pytest.fixture(scope="module")
def W():
    from rank_kv_cache_flash_amd import wsvd
    wsvd.lib()
    return wsvd


def rel(g, ref):
    return float(np.max(np.abs(np.asarray(g, np.float64) - ref)) / max(np.max(np.abs(ref)), 1e-300))


def draw_lengths(g, nb, L_cap):
    L = g.integers(0, L_cap + 1, size=nb).astype(np.int32)
    L[g.integers(0, nb)] = L_cap                       # at least one full cache
    return L


@pytest.mark.parametrize("seed", range(30))
def test_folded_decode_random_shapes(W, seed):
    g = np.random.default_rng(5000 + seed)
    H = int(g.choice([64, 128]))
    r = int(g.choice([16, 32, 48, 64]))
    C_dt = str(g.choice(["f32", "bf16", "i8"]))
    act = "f32" if C_dt == "f32" else str(g.choice(["bf16", "f16"]))
    nb, nh = int(g.integers(1, 7)), int(g.integers(1, 10))
    L_cap = int(g.integers(1, 700))
    L = draw_lengths(g, nb, L_cap)
    S = [None, 1, 2, 5, 17][int(g.integers(0, 5))]
    S = None if S is not None and S > L_cap else S
    scale = None if g.random() < 0.5 else float(g.uniform(0.02, 0.3))
    gain = float(g.choice([1.0, 4.0 * H]))
    out_f32 = bool(g.random() < 0.3)
    print(f"[case] folded seed={seed} H={H} r={r} C={C_dt} act={act} nb={nb} nh={nh} L_cap={L_cap} S={S} "
          f"scale={scale} gain={gain} out_f32={out_f32}", flush=True)
    inp = I.make_decode_inputs(nb, nh, H, r, L, L_cap, seed=5100 + seed, act_dt=act, C_dt=C_dt,
                               outlier_p=0.01 if C_dt == "i8" else 0.0, outlier_mul=20.0, q_gain=gain)
    d = W.device_inputs(inp)
    out, _, _ = W.decode_attn(d["q"], d["C_K"], d["C_V"], d["B_K"], d["B_V"], d["L"], s_K=d.get("s_K"),
                              s_V=d.get("s_V"), n_splits=S, softmax_scale=scale,
                              out_dtype=torch.float32 if out_f32 else None)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    ref = O.decode_attn(inp, softmax_scale=scale)
    tol = TOL[C_dt] if (C_dt != "f32" or out_f32 or act == "f32") else TOL["bf16"]
    e = rel(got, ref)
    print(f"[parity] folded seed={seed}: {e:.3e} (tol {tol})", flush=True)
    assert np.all(np.isfinite(got)) and e <= tol
    assert not got[L == 0].any()


@pytest.mark.parametrize("seed", range(10))
def test_rope_decode_random_shapes(W, seed):
    g = np.random.default_rng(5200 + seed)
    H = int(g.choice([64, 128]))
    r = int(g.choice([32, 64]))
    nb, nh = int(g.integers(1, 6)), int(g.integers(1, 9))
    L_cap = int(g.integers(1, 900))
    L = draw_lengths(g, nb, L_cap)
    S = [None, 1, 3][int(g.integers(0, 3))]
    S = None if S is not None and S > L_cap else S
    gain = float(g.choice([1.0, 4.0 * H]))
    print(f"[case] rope seed={seed} H={H} r={r} nb={nb} nh={nh} L_cap={L_cap} S={S} gain={gain}", flush=True)
    inp = I.make_decode_inputs(nb, nh, H, r, L, L_cap, seed=5300 + seed, act_dt="bf16", C_dt="bf16", q_gain=gain)
    d = W.device_inputs(inp)
    c, s_ = W.rope_tables(L_cap, H)
    out, _, _ = W.decode_attn_rope(d["q"], d["C_K"], d["C_V"], d["B_K"], d["B_V"], d["L"], c, s_, n_splits=S)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    e = rel(got, O.decode_attn_rope(inp))
    print(f"[parity] rope seed={seed}: {e:.3e}", flush=True)
    assert e <= TOL["bf16"]
    assert not got[L == 0].any()


@pytest.mark.parametrize("seed", range(8))
def test_shared_decode_random_shapes(W, seed):
    g = np.random.default_rng(5400 + seed)
    H = int(g.choice([64, 128]))
    R = int(g.choice([512, 1024, 2048]))
    nb, nh = int(g.integers(1, 11)), int(g.integers(1, 6))
    L_cap = int(g.integers(1, 400))
    L = draw_lengths(g, nb, L_cap)
    S = [None, 1, 4][int(g.integers(0, 3))]
    S = None if S is not None and S > L_cap else S
    print(f"[case] shared seed={seed} H={H} R={R} nb={nb} nh={nh} L_cap={L_cap} S={S}", flush=True)
    inp = I.make_shared_inputs(nb, nh, H, R, L, L_cap, seed=5500 + seed, q_gain=4.0 * H)
    d = W.shared_device_inputs(inp)
    out = W.shared_decode_attn(d["q"], d["C_K"], d["C_V"], d["B_K"], d["B_V"], d["L"], n_splits=S)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    e = rel(got, O.decode_attn_shared(inp))
    print(f"[parity] shared seed={seed}: {e:.3e}", flush=True)
    assert e <= TOL["bf16"]
    assert not got[L == 0].any()


@pytest.mark.parametrize("seed", range(12))
def test_append_random_shapes(W, seed):
    """Seeded random appends (bf16 and int8 caches), including out-of-range
    positions, with the same checks as the fixed-shape append tests."""
    from .test_gpu_parity import _append_case, _append_int8_case
    g = np.random.default_rng(5600 + seed)
    nb = int(g.integers(1, 71))
    nh = int(g.integers(1, 9))
    H = int(g.choice([64, 128]))
    r = int(g.choice([16, 32, 48, 64]))
    C_dt = str(g.choice(["bf16", "i8"]))
    if C_dt == "i8" and r == 48:
        r = 32
    E = int(g.choice([256, 512, 1024, 2048, 4096]))
    L_cap = int(g.integers(2, 60))
    print(f"[case] append seed={seed} nb={nb} nh={nh} H={H} r={r} E={E} C={C_dt} L_cap={L_cap}", flush=True)
    inp = I.make_ragged_step_inputs(nb, nh, H, r, E, 1, L_cap, L_cap, seed=5700 + seed, C_dt=C_dt)
    if C_dt == "i8":
        if nb > 1:
            inp.pos[0] = L_cap      # out of range: skipped
        _append_int8_case(W, inp)
    else:
        _append_case(W, inp)


@pytest.mark.parametrize("seed", range(8))
def test_dense_random_shapes(W, seed):
    """The Flash-Decoding baseline over full bf16 K / V on seeded random shapes:
    the oracle with r = H and identity factors (pinned against library SDPA)."""
    from .test_gpu_parity import _dense_case
    g = np.random.default_rng(5800 + seed)
    H = int(g.choice([64, 128]))
    nb, nh = int(g.integers(1, 7)), int(g.integers(1, 9))
    L_cap = int(g.integers(1, 700))
    L = draw_lengths(g, nb, L_cap)
    S = [None, 1, 2, 5][int(g.integers(0, 4))]
    S = None if S is not None and S > L_cap else S
    gain = float(g.choice([1.0, 4.0 * H]))
    print(f"[case] dense seed={seed} H={H} nb={nb} nh={nh} L_cap={L_cap} S={S} gain={gain}", flush=True)
    inp = _dense_case(nb, nh, H, L, L_cap, seed=5900 + seed, q_gain=gain)
    d = W.device_inputs(inp)
    out = W.dense_decode_attn(d["q"], d["C_K"], d["C_V"], d["L"], n_splits=S)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    e = rel(got, O.decode_attn(inp))
    print(f"[parity] dense seed={seed}: {e:.3e}", flush=True)
    assert e <= TOL["bf16"]
    assert not got[L == 0].any()


@pytest.mark.parametrize("seed", range(10))
def test_append_w8a8_random_shapes(W, seed):
    """Seeded random W8A8 appends (int8 activations and factors, bf16 or int8
    caches), with the exact-code checks of the fixed-shape W8A8 tests."""
    from .test_gpu_w8a8 import _w8_case
    g = np.random.default_rng(6000 + seed)
    nb = int(g.integers(1, 81))
    nh = int(g.integers(1, 9))
    C_dt = str(g.choice(["bf16", "i8"]))
    r = int(g.choice([16, 32, 64] if C_dt == "i8" else [16, 32, 48, 64]))
    E = int(g.choice([512, 1024, 1536, 2048, 2560, 4096]))
    L_cap = int(g.integers(2, 40))
    print(f"[case] w8a8 append seed={seed} nb={nb} nh={nh} r={r} E={E} C={C_dt} L_cap={L_cap}", flush=True)
    _w8_case(W, nb, E, nh, r, C_dt, seed=6100 + seed, L_cap=L_cap)


@pytest.mark.parametrize("seed", range(8))
def test_combine_random_shapes(W, seed):
    """wsvd_combine_splits on seeded random partials (split counts on both
    sides of the one-round-trip path, empty splits with lse = -inf, whole rows
    of empty splits) against the oracle's merge, fp32 output."""
    g = np.random.default_rng(6200 + seed)
    H = int(g.choice([64, 128]))
    nb, nh = int(g.integers(1, 9)), int(g.integers(1, 9))
    S = [1, 2, 3, 5, 8, 9, 64, 300][seed]      # both sides of the eight-split path
    o = g.standard_normal((nb, nh, S, H)).astype(np.float32)
    lse = (g.standard_normal((nb, nh, S)) * 20.0).astype(np.float32)
    empty = g.random((nb, nh, S)) < 0.2
    lse[empty] = -np.inf
    o[empty] = 0.0
    lse[0, 0, :] = -np.inf                       # one row with every split empty
    o[0, 0] = 0.0
    print(f"[case] combine seed={seed} H={H} nb={nb} nh={nh} S={S}", flush=True)
    out = W.combine_splits(torch.from_numpy(o).cuda(), torch.from_numpy(lse).cuda(), out_dtype=torch.float32)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    ref = np.stack([np.stack([O.combine(o[b, h], lse[b, h]) for h in range(nh)]) for b in range(nb)])
    e = rel(got, ref)
    print(f"[parity] combine seed={seed}: {e:.3e}", flush=True)
    assert e <= TOL["f32"]
    assert not got[0, 0].any()
