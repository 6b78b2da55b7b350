"""GPU parity of the W8A8 append (Hadamard S1 rotation, int8 operands) against the oracle.

Where fp32 arithmetic decides an integer code, GPU and oracle take the
decision in fp32, but on fp32 values reached by different roundings (the
GPU's butterfly transform or dot, the oracle's exact value rounded once).
Codes are therefore compared exactly except at elements whose exact value
lies within the arithmetic's error bound of a rounding boundary, where
either neighbour is correct; every bound is derived in the test.
"""
import numpy as np
import pytest

import oracle as O
from rank_kv_cache_flash_amd import inputs as I

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

U32 = 2.0 ** -24          # fp32 unit roundoff


@pytest.fixture(scope="module")
def W():
    from rank_kv_cache_flash_amd import wsvd
    wsvd.lib()
    return wsvd


def dev(a, dt):
    from rank_kv_cache_flash_amd import wsvd
    return wsvd.to_device(a, dt)


def near_boundary(v, scale, eps):
    """|v| / scale within eps / scale (plus fp32 rounding of the division) of k + 1/2."""
    t = np.abs(v) / scale
    frac = t - np.floor(t)
    return np.abs(frac - 0.5) <= eps / scale + 4 * U32 * t


def check_codes(gq, gs, v_exact, eps, what):
    """GPU codes / scales of rows of v_exact against the oracle's quantiser.

    eps bounds |GPU fp32 value - exact value| per row."""
    oq, os_ = O.quantize_rows_f32(v_exact)
    os_ = os_.astype(np.float64)
    gs = np.asarray(gs, np.float64)
    assert np.all(np.abs(gs - os_) <= eps / 127 + 2 * U32 * os_), f"{what}: scale"
    d = np.abs(gq.astype(np.int32) - oq.astype(np.int32))
    assert d.max() <= 1, f"{what}: code off by {d.max()}"
    # the scale's own uncertainty moves the boundary by at most |v| |ds| / s^2 <= 127 |ds| / s
    slack = eps[:, None] + np.abs(v_exact) * (eps[:, None] / 127 + 2 * U32 * os_[:, None]) / os_[:, None]
    amb = near_boundary(v_exact, os_[:, None], slack)
    bad = (d == 1) & ~amb
    assert not bad.any(), f"{what}: {int(bad.sum())} codes differ away from a rounding boundary"
    frac = float(np.mean(d == 0))
    print(f"[parity] {what}: codes equal {frac:.5f}, differing only at {int(d.sum())} near-boundary elements",
          flush=True)
    return frac


@pytest.mark.parametrize("nb,E", [(9, 4096), (3, 256), (5, 8192), (64, 4096)])
def test_quantize_activations(W, nb, E):
    x = I.make_w8a8_activations(nb, E, seed=600 + E + nb)
    xq, sx = W.w8a8_quantize_activations(dev(x, "bf16"))
    torch.cuda.synchronize()
    xr = O.rotate_rows(x, "bf16")
    # pairwise-summation bound of the log2(E)-pass transform, then the exact 2^-k scaling (E = 4^j) or one rounding
    eps = np.log2(E) * U32 * np.abs(O.upcast(x, "bf16")).sum(axis=1) / np.sqrt(E) + 2 * U32 * np.abs(xr).max(axis=1)
    check_codes(xq.cpu().numpy(), sx.cpu().numpy(), xr, eps, f"activations nb={nb} E={E}")


def test_quantize_activations_zero_row(W):
    x = I.make_w8a8_activations(3, 512, seed=5)
    x[1] = 0
    xq, sx = W.w8a8_quantize_activations(dev(x, "bf16"))
    torch.cuda.synchronize()
    assert float(sx[1]) == 0.0 and not xq[1].any()


@pytest.mark.parametrize("E,N", [(4096, 192), (512, 64), (2048, 40)])
def test_prepare_factor(W, E, N):
    A = I._store(I._normal(700 + E, (I.T_AK,), (E, N), 1.0 / np.sqrt(32)), "bf16")
    AqT, sA = W.w8a8_prepare_factor(dev(A, "bf16"))
    torch.cuda.synchronize()
    rot = (O.hadamard_matrix(E).astype(np.float64) @ O.upcast(A, "bf16")) / np.sqrt(E)
    eps = np.log2(E) * U32 * np.abs(O.upcast(A, "bf16")).sum(axis=0) / np.sqrt(E) + 2 * U32 * np.abs(rot).max(axis=0)
    check_codes(AqT.cpu().numpy(), sA.cpu().numpy(), rot.T, eps, f"factor E={E} N={N}")


def _w8_case(W, nb, E, nh, r, C_dt, seed, L_cap=24):
    xq, sx, AqT_K, sA_K = I.make_w8a8_codes(nb, E, nh * r, seed=seed)
    _, _, AqT_V, sA_V = I.make_w8a8_codes(nb, E, nh * r, seed=seed + 1)
    pos = (np.arange(nb) * 7 % L_cap).astype(np.int32)
    g = {k: torch.from_numpy(v).cuda() for k, v in
         dict(xq=xq, sx=sx, AK=AqT_K, sK=sA_K, AV=AqT_V, sV=sA_V, pos=pos).items()}
    tdt = {"bf16": torch.bfloat16, "i8": torch.int8}[C_dt]
    C_K = torch.zeros(nb, nh, L_cap, r, dtype=tdt, device="cuda")
    C_V = torch.zeros_like(C_K)
    s_K = torch.zeros(nb, nh, L_cap, dtype=torch.float16, device="cuda") if C_dt == "i8" else None
    s_V = torch.zeros_like(s_K) if s_K is not None else None
    W.append_latent_w8a8(g["xq"], g["sx"], g["AK"], g["sK"], g["AV"], g["sV"], g["pos"], C_K, C_V, s_K=s_K,
                         s_V=s_V)
    torch.cuda.synchronize()
    for A, sA, C, S, tag in ((AqT_K, sA_K, C_K, s_K, "K"), (AqT_V, sA_V, C_V, s_V, "V")):
        c = O.w8a8_latents(xq, sx, A, sA, nh, r)             # exact
        bound = 3 * U32 * np.abs(c)                            # fp32: int -> float, two products
        Cn = C.cpu().float().numpy() if C_dt == "bf16" else C.cpu().numpy()
        rows = Cn[np.arange(nb), :, pos]                       # [nb, nh, r]
        if C_dt == "bf16":
            gv = rows.astype(np.float64)
            half_ulp = np.ldexp(1.0, np.frexp(np.abs(gv))[1] - 9)
            assert np.all(np.abs(gv - c) <= half_ulp + bound), f"w8a8 append {tag}: bf16 rows"
        else:
            gc = rows
            gs = S.cpu().numpy()[np.arange(nb), :, pos].astype(np.float64)
            rq, rs = O.quantize_latent_rows(c)
            ulp = np.spacing(rs).astype(np.float64)
            assert np.all(np.abs(gs - rs.astype(np.float64)) <= ulp), f"w8a8 append {tag}: scales"
            deq = gc.astype(np.float64) * gs[..., None]
            assert np.all(np.abs(deq - c) <= 0.5 * gs[..., None] * (1 + 1e-6) + bound + 1e-30), f"{tag}: codes"
            assert np.abs(gc.astype(np.int32) - rq.astype(np.int32)).max() <= 1
        # nothing else written
        mask = np.ones((nb, nh, L_cap), bool)
        mask[np.arange(nb), :, pos] = False
        assert not C.cpu().float().numpy()[mask].any()


@pytest.mark.parametrize("nb,E,nh,r,C_dt", [
    (70, 4096, 4, 32, "bf16"),     # two row tiles, E split 4 ways (two stages per slice)
    (5, 512, 3, 16, "bf16"),       # one stage, ragged column tile
    (9, 1536, 2, 64, "i8"),        # three stages in one slice (no split)
    (9, 4608, 2, 64, "bf16"),      # nine stages in one slice: four pairs, then one
    (7, 2560, 4, 32, "i8"),        # five stages in one slice
    (64, 4096, 32, 48, "bf16"),    # the LLaVA-7B-layer step's shape
    (32, 4096, 32, 32, "i8"),      # the int8-cache workload's shape
])
def test_append_w8a8_exact_codes(W, nb, E, nh, r, C_dt):
    _w8_case(W, nb, E, nh, r, C_dt, seed=800 + nb + r)


def test_w8a8_pipeline_then_decode(W):
    """x, A -> (GPU) prepare, rotate + quantise, integer append, decode; the
    oracle runs the same pipeline from the same x and A."""
    nb, nh, H, r, E = 8, 4, 128, 32, 4096
    inp = I.make_ragged_step_inputs(nb, nh, H, r, E, 100, 300, 300, seed=909)
    inp.x = I.make_w8a8_activations(nb, E, seed=910)
    d = W.device_inputs(inp)
    AK, sAK = W.w8a8_prepare_factor(d["A_K"])
    AV, sAV = W.w8a8_prepare_factor(d["A_V"])
    xq, sx = W.w8a8_quantize_activations(d["x"])
    W.append_latent_w8a8(xq, sx, AK, sAK, AV, sAV, d["pos"], d["C_K"], d["C_V"])
    out, _, _ = W.decode_attn(d["q"], d["C_K"], d["C_V"], d["B_K"], d["B_V"], d["L"])
    torch.cuda.synchronize()
    # oracle pipeline
    oxq, osx = O.quantize_activations(inp.x, "bf16")
    ok = {}
    for tag, A in (("K", inp.A_K), ("V", inp.A_V)):
        AqT, sA = O.prepare_factor(A, "bf16")
        ok[tag] = O.w8a8_latents(oxq, osx, AqT, sA, nh, r)
    CK, CV = inp.C_K.copy(), inp.C_V.copy()
    for b in range(nb):
        p = int(inp.pos[b])
        CK[b, :, p] = O.round_to_bf16_bits(ok["K"][b])
        CV[b, :, p] = O.round_to_bf16_bits(ok["V"][b])
    ref = O.decode_attn(inp, C_K=CK, C_V=CV)
    g = out.float().cpu().numpy().astype(np.float64)
    err = float(np.max(np.abs(g - ref)) / np.max(np.abs(ref)))
    print(f"[parity] w8a8 pipeline + decode: max|err|/max|ref| = {err:.3e} (tol 0.02)", flush=True)
    assert err <= 2e-2
    # Appended rows: the GPU's codes may differ from the oracle's only at near-boundary elements;
    # each flipped x code moves latent n by s_x s_A |AqT[n, e]| (+1 if that code flipped too), each
    # flipped A code by s_x s_A (|xq[b, e]| + 1); scales differ by at most their fp32 bounds.
    xr = O.rotate_rows(inp.x, "bf16")
    ex = np.log2(E) * U32 * np.abs(O.upcast(inp.x, "bf16")).sum(1) / np.sqrt(E) + 2 * U32 * np.abs(xr).max(1)
    amb_x = near_boundary(xr, osx[:, None].astype(np.float64),
                          ex[:, None] + np.abs(xr) * (ex[:, None] / 127 + 2 * U32 * osx[:, None]) / osx[:, None])
    for tag, A, C in (("K", inp.A_K, d["C_K"]), ("V", inp.A_V, d["C_V"])):
        AqT, sA = O.prepare_factor(A, "bf16")
        rot = ((O.hadamard_matrix(E).astype(np.float64) @ O.upcast(A, "bf16")) / np.sqrt(E)).T
        ea = np.log2(E) * U32 * np.abs(O.upcast(A, "bf16")).sum(0) / np.sqrt(E) + 2 * U32 * np.abs(rot).max(1)
        sa64 = sA.astype(np.float64)
        amb_a = near_boundary(rot, sa64[:, None], ea[:, None] + np.abs(rot) * (ea[:, None] / 127 + 2 * U32 * sa64[:, None]) / sa64[:, None])
        flips = amb_x.astype(np.float64) @ (np.abs(AqT.astype(np.float64)) + 1).T \
            + (np.abs(oxq.astype(np.float64)) + 1) @ amb_a.astype(np.float64).T
        c = ok[tag].reshape(nb, nh * r)
        rel_s = ex / 127 / osx + 2 * U32                  # scale uncertainty, relative
        bound = (osx[:, None] * sa64[None, :] * flips + (rel_s[:, None] + (ea / 127 / sa64)[None, :] + 5 * U32) * np.abs(c))
        gv = C.cpu().float().numpy()[np.arange(nb), :, inp.pos].astype(np.float64).reshape(nb, nh * r)
        half_ulp = np.ldexp(1.0, np.frexp(np.abs(gv))[1] - 9)
        diff = np.abs(gv - c)
        assert np.all(diff <= half_ulp + bound), f"w8a8 pipeline latents {tag}"
        print(f"[parity] w8a8 pipeline {tag} latents: max|gpu - oracle| / max|oracle| = "
              f"{float(diff.max() / np.abs(c).max()):.3e}; near-boundary codes x {int(amb_x.sum())}, "
              f"A {int(amb_a.sum())}", flush=True)


@pytest.mark.parametrize("E,nh,r", [(512, 1, 64), (4096, 1, 64), (4096, 2, 32)])
def test_append_w8a8_identifies_every_k(W, E, nh, r):
    """One-hot token codes pick one k per row and the factor codes encode k and
    n, so every entry of the integer product is known exactly; covers shapes
    with few output tiles, where the E split is deepest."""
    nb, N = 64, nh * r
    xq = np.zeros((nb, E), np.int8)
    xq[np.arange(nb), (3 * np.arange(nb) + 5) % E] = 1
    AqT = ((np.arange(E)[None, :] + 7 * np.arange(N)[:, None]) % 101).astype(np.int8)
    ones_x, ones_a = np.ones(nb, np.float32), np.ones(N, np.float32)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    C_K = torch.zeros(nb, nh, 1, r, dtype=torch.float32, device="cuda")
    C_V = torch.zeros_like(C_K)
    W.append_latent_w8a8(t(xq), t(ones_x), t(AqT), t(ones_a), t(-AqT), t(ones_a), t(np.zeros(nb, np.int32)), C_K, C_V)
    torch.cuda.synchronize()
    exact = (xq.astype(np.int64) @ AqT.astype(np.int64).T).reshape(nb, nh, r)
    assert np.array_equal(C_K.cpu().numpy()[:, :, 0, :], exact)
    assert np.array_equal(C_V.cpu().numpy()[:, :, 0, :], -exact)
