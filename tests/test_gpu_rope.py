"""GPU parity of the decode with a rotary position step (keys rebuilt on matrix
cores, rotated to their token positions) against the fp64 oracle."""
import numpy as np
import pytest

import oracle as O
from rank_kv_cache_flash_amd import inputs as I

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = 2e-2   # bf16 inputs and outputs (the same bar as the folded decode)


@pytest.fixture(scope="module")
def W():
    from rank_kv_cache_flash_amd import wsvd
    wsvd.lib()
    return wsvd


def rel(g, ref):
    return float(np.max(np.abs(np.asarray(g, np.float64) - ref)) / max(np.max(np.abs(ref)), 1e-300))


def run(W, inp, base=10000.0, n_splits=None, tables=None):
    d = W.device_inputs(inp)
    H = inp.q.shape[-1]
    c, s = tables if tables is not None else W.rope_tables(inp.L_cap, H, base)
    out, o_part, lse = W.decode_attn_rope(d["q"], d["C_K"], d["C_V"], d["B_K"], d["B_V"], d["L"], c, s,
                                          n_splits=n_splits)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), d


@pytest.mark.parametrize("L_cap,H", [(300, 128), (8192, 64)])
def test_rope_tables(W, L_cap, H):
    c, s = W.rope_tables(L_cap, H, 10000.0)
    torch.cuda.synchronize()
    ang = O.rope_angles(np.arange(L_cap), H, 10000.0)
    assert np.max(np.abs(c.cpu().numpy() - np.cos(ang))) <= 6e-8
    assert np.max(np.abs(s.cpu().numpy() - np.sin(ang))) <= 6e-8


@pytest.mark.parametrize("H,r", [(128, 32), (128, 64), (64, 32), (64, 64)])
@pytest.mark.parametrize("S", [None, 1, 3])
def test_rope_decode_ragged(W, H, r, S):
    L = np.array([300, 1, 0, 257, 129], np.int32)
    inp = I.make_decode_inputs(5, 3, H, r, L, 300, seed=1200 + H + r, act_dt="bf16", C_dt="bf16", q_gain=4.0 * H)
    g, _ = run(W, inp, n_splits=S)
    ref = O.decode_attn_rope(inp)
    e = rel(g, ref)
    print(f"[parity] rope H={H} r={r} S={S}: max|err|/max|ref| = {e:.3e}", flush=True)
    assert e <= TOL
    assert np.all(g[2] == 0)                     # L = 0 rows are zero


def test_rope_decode_llava_layer(W):
    """The LLaVA-7B-shaped layer (1 x 32 heads, H 128, r 32, 1088 tokens) with rotated keys."""
    inp = I.make_decode_inputs(1, 32, 128, 32, 1088, 1088, seed=1300, act_dt="bf16", C_dt="bf16", q_gain=4.0 * 128)
    g, _ = run(W, inp)
    e = rel(g, O.decode_attn_rope(inp))
    print(f"[parity] rope llava layer: max|err|/max|ref| = {e:.3e}", flush=True)
    assert e <= TOL


def test_rope_decode_long_positions(W):
    """Positions up to 8000: the tables and the three angle steps per lane stay accurate."""
    inp = I.make_decode_inputs(2, 4, 128, 64, 8000, 8192, seed=1400, act_dt="bf16", C_dt="bf16", q_gain=300.0 * 128)
    g, _ = run(W, inp)
    e = rel(g, O.decode_attn_rope(inp))
    print(f"[parity] rope long positions (peaked): max|err|/max|ref| = {e:.3e}", flush=True)
    assert e <= TOL


def test_rope_with_zero_angles_equals_folded_decode(W):
    """cos = 1, sin = 0 everywhere turns the rotation off: the rebuilt-key kernel
    must then agree with the folded kernel and with the plain oracle."""
    inp = I.make_decode_inputs(3, 4, 128, 32, np.array([500, 77, 1], np.int32), 512, seed=1500, act_dt="bf16",
                               C_dt="bf16", q_gain=4.0 * 128)
    c = torch.ones(512, 64, dtype=torch.float32, device="cuda")
    s = torch.zeros_like(c)
    g, d = run(W, inp, tables=(c, s))
    folded, _, _ = W.decode_attn(d["q"], d["C_K"], d["C_V"], d["B_K"], d["B_V"], d["L"])
    torch.cuda.synchronize()
    ref = O.decode_attn(inp)
    assert rel(g, ref) <= TOL
    assert rel(g, folded.float().cpu().numpy().astype(np.float64)) <= TOL


def test_rope_decode_large_grid(W):
    """64 x 8 heads x 4 splits = 2048 blocks: partials merged in a second launch."""
    L = (np.arange(64, dtype=np.int32) * 37) % 300 + 1
    inp = I.make_decode_inputs(64, 8, 64, 32, L, 300, seed=1600, act_dt="bf16", C_dt="bf16", q_gain=4.0 * 64)
    g, _ = run(W, inp, n_splits=4)
    assert rel(g, O.decode_attn_rope(inp)) <= TOL


@pytest.mark.parametrize("nb", [64, 65])
def test_rope_decode_large_grid_ragged(W, nb):
    """2048+ blocks over ragged lengths with ties and an empty sequence
    (partials merged in a second launch)."""
    rng = np.random.default_rng(1700 + nb)
    L = rng.integers(1, 301, nb).astype(np.int32)
    L[::7] = L[0]
    L[3] = 0
    inp = I.make_decode_inputs(nb, 8, 64, 32, L, 300, seed=1700 + nb, act_dt="bf16", C_dt="bf16",
                               q_gain=4.0 * 64)
    g, _ = run(W, inp, n_splits=4)
    e = rel(g, O.decode_attn_rope(inp))
    print(f"[parity] rope large grid nb={nb}: max|err|/max|ref| = {e:.3e}", flush=True)
    assert e <= TOL
    assert np.all(g[3] == 0)
