"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Bar: max|gpu - ref| / max|ref| <= 1e-5 for the fp32 workload and <= 2e-2
for bf16 / int8 workloads, over the whole output tensor.  The full-size
workloads run in the launch configuration the benchmark times (automatic
splits); the oracle computes every (b, h) row of them, one row at a time
(rows in parallel threads).
"""
import math

import numpy as np
import pytest

import oracle as O
from rank_kv_cache_flash_amd import inputs as I
from rank_kv_cache_flash_amd.configs import CONFIGS
from tests.golden import make_golden as G

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 2e-2, "f16": 2e-2, "i8": 2e-2}


@pytest.fixture(scope="module")
def W():
    from rank_kv_cache_flash_amd import wsvd
    wsvd.lib()
    return wsvd


def oracle_all(inp, C_K=None, C_V=None, softmax_scale=None):
    """out [nb, nh, H] from the oracle's single-row function for every (b, h),
    rows spread over threads (BLAS kept to one thread per worker)."""
    from concurrent.futures import ThreadPoolExecutor

    from threadpoolctl import threadpool_limits
    nb, nh, H = inp.q.shape
    pairs = [(b, h) for b in range(nb) for h in range(nh)]
    with threadpool_limits(1), ThreadPoolExecutor(I._workers()) as ex:
        rows = list(ex.map(lambda p: O.decode_attn_one(inp, p[0], p[1], softmax_scale, C_K=C_K, C_V=C_V), pairs))
    return np.stack(rows).reshape(nb, nh, H)


def rel_err(gpu, ref):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.max(np.abs(ref))
    return float(np.max(np.abs(gpu - ref)) / (den if den > 0 else 1.0))


def run_decode(W, inp, n_splits=None, out_dtype=None, softmax_scale=None, poison=False, partials_only=False):
    d = W.device_inputs(inp)
    ws = None
    if poison:
        nb, nh, H = inp.q.shape
        need = W.decode_workspace_bytes(nb, nh, H, inp.L_cap, n_splits or 0)
        ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")  # NaN bytes
        ws[:W.decode_counter_bytes(nb, nh)] = 0  # counters start at zero
    out, o_part, lse = W.decode_attn(d["q"], d["C_K"], d["C_V"], d["B_K"], d["B_V"], d["L"], s_K=d.get("s_K"),
                                     s_V=d.get("s_V"), n_splits=n_splits, out_dtype=out_dtype,
                                     softmax_scale=softmax_scale, workspace=ws, partials_only=partials_only)
    torch.cuda.synchronize()
    return out, o_part, lse


def f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def check(name, gpu, ref, tol):
    e = rel_err(gpu, ref)
    print(f"[parity] {name}: max|err|/max|ref| = {e:.3e} (tol {tol:g})", flush=True)
    assert np.all(np.isfinite(gpu)), name
    assert e <= tol, f"{name}: {e} > {tol}"


# ---------------------------------------------------------------------------
# tiny fp32 workload (batch 1, 4 heads, H 64, r 16, L 256)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("S", [None, 1, 2, 3, 7, 64, 256])
def test_config1_fp32(W, S):
    inp = CONFIGS[1].make()
    out, _, _ = run_decode(W, inp, n_splits=S)
    ref = O.decode_attn(inp)
    check(f"config1 S={S}", f64(out), ref, TOL["f32"])
    check(f"config1 S={S} vs stored", f64(out).reshape(-1), G.read("config1_out"), TOL["f32"])


def test_config1_peaked_and_huge(W):
    c = CONFIGS[1]
    for gain in (4.0 * c.H, 300.0 * c.H):
        inp = c.make(q_gain=gain)
        out, _, _ = run_decode(W, inp)
        check(f"config1 q_gain={gain}", f64(out), O.decode_attn(inp), TOL["f32"])
    out, _, _ = run_decode(W, c.make(q_gain=4.0 * c.H))
    check("config1 peaked vs stored", f64(out).reshape(-1), G.read("config1_peaked_out"), TOL["f32"])


@pytest.mark.parametrize("S", [3, 7])
def test_config1_partials_match_segments(W, S):
    inp = CONFIGS[1].make(q_gain=2.0 * CONFIGS[1].H)
    _, o_part, lse = run_decode(W, inp, n_splits=S, partials_only=True)
    o_part, lse = f64(o_part), f64(lse)
    for h in range(inp.nh):
        ro, rl = O.decode_partials_one(inp, 0, h, S)
        check(f"partials h={h} S={S}", o_part[0, h], ro, TOL["f32"])
        fin = np.isfinite(rl)
        assert np.array_equal(np.isfinite(lse[0, h]), fin)
        assert np.max(np.abs(lse[0, h][fin] - rl[fin])) < 1e-5 * max(1.0, np.max(np.abs(rl[fin])))


def test_config1_stored_partials(W):
    inp = CONFIGS[1].make()
    _, o_part, lse = run_decode(W, inp, n_splits=3, partials_only=True)
    check("stored partials o", f64(o_part).reshape(-1), G.read("config1_split3_o"), TOL["f32"])
    assert np.max(np.abs(f64(lse).reshape(-1) - G.read("config1_split3_lse"))) < 1e-5


def test_combine_entry_point_matches_decode(W):
    inp = CONFIGS[1].make()
    out, _, _ = run_decode(W, inp, n_splits=5)
    _, o_part, lse = run_decode(W, inp, n_splits=5, partials_only=True)
    out2 = W.combine_splits(o_part.contiguous(), lse.contiguous(), out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)


def test_nan_poisoned_workspace_and_determinism(W):
    inp = CONFIGS[1].make()
    a, _, _ = run_decode(W, inp, n_splits=7, poison=True)
    b, _, _ = run_decode(W, inp, n_splits=7)
    assert torch.isfinite(a).all()
    assert torch.equal(a, b)


def test_merge_counters_reset_and_reuse(W):
    """One workspace reused across calls and shapes: the counters come back to zero."""
    inp = CONFIGS[2].make(q_gain=4.0 * CONFIGS[2].H)
    d = W.device_inputs(inp)
    nb, nh, H = inp.q.shape
    ws = W.decode_workspace(nb, nh, H, inp.L_cap, 0)
    nctr = W.decode_counter_bytes(nb, nh)
    ref = O.decode_attn(inp)
    outs = []
    for _ in range(5):
        out, _, _ = W.decode_attn(d["q"], d["C_K"], d["C_V"], d["B_K"], d["B_V"], d["L"], workspace=ws)
        outs.append(out)
    torch.cuda.synchronize()
    assert not ws[:nctr].any(), "merge counters must be zero after every call"
    for o in outs:
        assert torch.equal(o, outs[0])
    check("config 2 reused workspace", f64(outs[0]), ref, TOL["bf16"])


def test_workspace_reused_across_split_counts(W):
    """One zero-filled workspace serves S = 5 and then S = 3 (and back) with an
    output: the counters sit at byte 0 for every split count, so partials of
    one call never land on counters of the next."""
    inp = CONFIGS[2].make(q_gain=4.0 * CONFIGS[2].H)
    d = W.device_inputs(inp)
    nb, nh, H = inp.q.shape
    need = max(W.decode_workspace_bytes(nb, nh, H, inp.L_cap, S) for S in (5, 3))
    ws = W._zero_filled(torch.zeros(need, dtype=torch.uint8, device="cuda"))
    ref = O.decode_attn(inp)
    outs = {}
    for S in (5, 3, 5, 3):
        out, _, _ = W.decode_attn(d["q"], d["C_K"], d["C_V"], d["B_K"], d["B_V"], d["L"], n_splits=S, workspace=ws)
        torch.cuda.synchronize()
        assert not ws[:W.decode_counter_bytes(nb, nh)].any(), f"counters not zero after S={S}"
        if S in outs:
            assert torch.equal(out, outs[S]), f"S={S} changed between calls"
        outs[S] = out
        check(f"config 2 shared workspace S={S}", f64(out), ref, TOL["bf16"])


def test_one_split_with_output_leaves_partials_alone(W):
    """S = 1 with an output: rows go straight to out and the partial area of the
    workspace keeps whatever it held (here a NaN fill); the output equals the
    partials-only run's o_part, rounded once."""
    L = np.array([300, 1, 0, 257], np.int32)
    inp = I.make_decode_inputs(4, 3, 128, 32, L, 300, seed=4500, act_dt="bf16", C_dt="bf16", q_gain=4.0 * 128)
    d = W.device_inputs(inp)
    nb, nh, H = inp.q.shape
    need = W.decode_workspace_bytes(nb, nh, H, inp.L_cap, 1)
    nctr = W.decode_counter_bytes(nb, nh)
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")
    ws[:nctr] = 0
    out, _, _ = W.decode_attn(d["q"], d["C_K"], d["C_V"], d["B_K"], d["B_V"], d["L"], n_splits=1, workspace=ws,
                              out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert bool((ws[nctr:] == 0xFF).all()), "partials must not be written with S = 1 and an output"
    _, o_part, lse = W.decode_attn(d["q"], d["C_K"], d["C_V"], d["B_K"], d["B_V"], d["L"], n_splits=1,
                                   partials_only=True)
    torch.cuda.synchronize()
    assert torch.equal(out, o_part[:, :, 0, :])
    check("one split, direct output", f64(out), O.decode_attn(inp), TOL["bf16"])


# ---------------------------------------------------------------------------
# small cases spanning several tiles, ragged tails, every (H, r, cache dtype)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("H,r", [(64, 16), (64, 32), (64, 48), (64, 64), (128, 16), (128, 32), (128, 48), (128, 64)])
@pytest.mark.parametrize("C_dt", ["f32", "bf16", "i8"])
def test_small_all_shapes(W, H, r, C_dt):
    act = "f32" if C_dt == "f32" else "bf16"
    L = np.array([300, 1, 0, 257, 129], np.int32)
    inp = I.make_decode_inputs(5, 3, H, r, L, 300, seed=77 + H + r, act_dt=act, C_dt=C_dt,
                               outlier_p=0.01 if C_dt == "i8" else 0.0, outlier_mul=20.0, q_gain=2.0 * H)
    ref = O.decode_attn(inp)
    for S in (None, 1, 3):
        out, _, _ = run_decode(W, inp, n_splits=S)
        g = f64(out)
        check(f"H={H} r={r} C={C_dt} S={S}", g, ref, TOL[C_dt])
        assert not g[2].any(), "L = 0 must give a zero row"


def test_length_clamp_and_single_token(W):
    L = np.array([1, 40, 4000], np.int32)   # last one exceeds L_cap = 64
    inp = I.make_decode_inputs(3, 4, 128, 32, L, 64, seed=5, act_dt="bf16", C_dt="bf16", fill=np.minimum(L, 64))
    out, _, _ = run_decode(W, inp, n_splits=4)
    check("clamp/single", f64(out), O.decode_attn(inp), TOL["bf16"])


def test_mixed_dtypes_and_scale(W):
    inp = I.make_decode_inputs(2, 4, 128, 64, 333, 333, seed=8, act_dt="f16", C_dt="bf16")
    inp.B_K = I.f32_to_bf16_bits(O.upcast(inp.B_K, "f16").astype(np.float32))
    inp.B_V = I.f32_to_bf16_bits(O.upcast(inp.B_V, "f16").astype(np.float32))
    inp.B_dt = "bf16"
    out, _, _ = run_decode(W, inp, out_dtype=torch.float32, softmax_scale=0.3)
    check("q f16 / B bf16 / out f32, sigma 0.3", f64(out), O.decode_attn(inp, softmax_scale=0.3), TOL["f16"])


def test_int8_zero_rows(W):
    inp = I.make_decode_inputs(2, 2, 128, 32, 100, 100, seed=4, act_dt="bf16", C_dt="i8")
    inp.C_K[0, 1, 10:20] = 0
    inp.s_K[0, 1, 10:20] = np.float16(0)
    inp.C_V[1, 0, :50] = 0
    inp.s_V[1, 0, :50] = np.float16(0)
    out, _, _ = run_decode(W, inp, n_splits=3)
    check("int8 zero rows", f64(out), O.decode_attn(inp), TOL["i8"])


# ---------------------------------------------------------------------------
# the workloads at full size, in the benchmark's launch configuration; every
# output row compared
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("cid", [2, 3, 4])
@pytest.mark.parametrize("peaked", [False, True])
def test_full_size_whole_tensor(W, cid, peaked):
    """Near-uniform (the benchmark's inputs) and peaked (q x 4H, score sd
    about 4) softmax at full size; all nb x nh rows against the oracle."""
    c = CONFIGS[cid]
    inp = c.make(q_gain=4.0 * c.H if peaked else 1.0)
    print(f"[case] config {cid} {'peaked' if peaked else 'uniform'}: {c.describe()}", flush=True)
    out, _, _ = run_decode(W, inp)
    check(f"config {cid} {'peaked' if peaked else 'uniform'} whole tensor ({c.nb * c.nh} rows)", f64(out),
          oracle_all(inp), TOL[c.C_dt])


# ---------------------------------------------------------------------------
# +1000 on every score (a constant latent column mapped onto q), per cache
# dtype.  Softmax is unchanged by it in exact arithmetic; it checks that the
# running max and the rescaling take the common offset out.
# ---------------------------------------------------------------------------
def plain_fp32_attention(inp):
    """Plain attention in torch float32 on the CPU (K = C B materialised in
    fp32, softmax, p V) -- the accuracy fp32 arithmetic reaches on inputs
    whose scores all sit near 1000; used to size the fp32 tolerance there."""
    nb, nh, H = inp.q.shape
    out = np.zeros((nb, nh, H))
    sig = 1.0 / math.sqrt(H)
    for b in range(nb):
        n = int(inp.L[b])
        if n == 0:
            continue
        for h in range(nh):
            def lat(C, sc):
                c = torch.from_numpy(O.upcast(C[b, h, :n], inp.C_dt).astype(np.float32))
                if sc is not None:
                    c = c * torch.from_numpy(O.upcast(sc[b, h, :n], "f16").astype(np.float32))[:, None]
                return c
            K = lat(inp.C_K, inp.s_K) @ torch.from_numpy(O.upcast(inp.B_K[h], inp.B_dt).astype(np.float32))
            V = lat(inp.C_V, inp.s_V) @ torch.from_numpy(O.upcast(inp.B_V[h], inp.B_dt).astype(np.float32))
            q = torch.from_numpy(O.upcast(inp.q[b, h], inp.q_dt).astype(np.float32))
            p = torch.softmax((K @ q) * sig, dim=0)
            out[b, h] = (p @ V).double().numpy()
    return out


@pytest.mark.parametrize("C_dt", ["f32", "bf16", "i8"])
@pytest.mark.parametrize("gain", [1.0, 4.0])
def test_score_shift_1000(W, C_dt, gain):
    H = 128
    act = "f32" if C_dt == "f32" else "bf16"
    L = np.array([300, 1, 0, 257, 129], np.int32)
    base = I.make_decode_inputs(5, 4, H, 32, L, 300, seed=4700 + int(gain), act_dt=act, C_dt=C_dt,
                                outlier_p=0.01 if C_dt == "i8" else 0.0, outlier_mul=20.0, q_gain=gain * H)
    inp = I.add_score_shift(base)
    ref = O.decode_attn(inp)
    assert np.max(np.abs(ref - O.decode_attn(inp.meta["unshifted"]))) <= 1e-9 * np.max(np.abs(ref))
    tol = TOL[C_dt]
    if C_dt == "f32":
        # Scores near 1000 carry fp32 rounding of about 1000 * 2^-24 each, so
        # 1e-5 is out of reach of any fp32 arithmetic here: the bar is four
        # times what plain fp32 attention reaches on the same inputs.
        e32 = rel_err(plain_fp32_attention(inp), ref)
        tol = max(TOL["f32"], 4.0 * e32)
        print(f"[parity] plain fp32 attention at +{inp.meta['score_shift']:.1f}: {e32:.3e}", flush=True)
    for S in (None, 1, 3):
        out, _, _ = run_decode(W, inp, n_splits=S)
        g = f64(out)
        check(f"+{inp.meta['score_shift']:.1f} on every score, C={C_dt} gain={gain} S={S}", g, ref, tol)
        assert not g[2].any()


@pytest.mark.parametrize("cid", [2, 4])
def test_score_shift_1000_full_size(W, cid):
    c = CONFIGS[cid]
    inp = I.add_score_shift(c.make(q_gain=4.0 * c.H))
    out, _, _ = run_decode(W, inp)
    check(f"config {cid} +{inp.meta['score_shift']:.1f} on every score, whole tensor", f64(out), oracle_all(inp),
          TOL[c.C_dt])


@pytest.mark.parametrize("S", [1, 2, 3, 1088])
def test_config2_split_sweep(W, S):
    c = CONFIGS[2]
    inp = c.make(q_gain=4.0 * c.H)
    out, _, _ = run_decode(W, inp, n_splits=S)
    check(f"config 2 S={S}", f64(out), O.decode_attn(inp), TOL["bf16"])


# ---------------------------------------------------------------------------
# append (x . A_Kh into the cache) + decode
# ---------------------------------------------------------------------------
def appended_row_ok(gpu_bits, exact, x, A, nh, r):
    """|gpu - exact| <= half a bf16 ulp of the stored value plus the fp32
    accumulation bound E * 2^-24 * sum_e |x_e A_e| of a length-E dot."""
    xx = O.upcast(x, "bf16")
    AA = O.upcast(A, "bf16")
    E = xx.shape[1]
    mag = np.abs(xx) @ np.abs(AA)                     # [nb, nh*r]
    bound_acc = E * 2.0 ** -24 * mag.reshape(exact.shape)
    g = O.upcast(gpu_bits, "bf16")
    half_ulp = np.ldexp(1.0, np.frexp(np.abs(g))[1] - 9)
    return np.abs(g - exact) <= half_ulp + bound_acc + 1e-30


def bf16_ulp_distance(a_bits, b_bits):
    """Steps between two bf16 bit patterns along the number line (+0 and -0
    are the same point)."""
    def key(u):
        u = np.asarray(u, np.uint16).astype(np.int64)
        return np.where(u & 0x8000, -(u & 0x7FFF), u)
    return np.abs(key(a_bits) - key(b_bits))


def appended_rows_within_one_ulp(gpu_bits, exact, what):
    """The appended-row rule: the stored bf16 value is within one bf16 step of
    the oracle's rounding of the exact latent.  The only admitted exceptions
    are near-cancellations: elements whose exact value is below 2^-10 of the
    largest in their row, where one bf16 step is finer than the rounding of
    an fp32 sum over E terms of the row's size.  Prints the count."""
    ref = O.round_to_bf16_bits(exact)
    dist = bf16_ulp_distance(gpu_bits, ref)
    far = dist > 1
    rowmax = np.max(np.abs(exact), axis=-1, keepdims=True)
    tiny = np.abs(exact) < 2.0 ** -10 * rowmax
    print(f"[parity] {what}: {dist.size} appended elements, {int(np.sum(dist == 0))} equal to the oracle's bf16, "
          f"{int(np.sum(dist == 1))} one step apart, {int(np.sum(far))} further (all near-cancellations: "
          f"{bool(np.all(tiny[far]))}), max steps {int(dist.max())}", flush=True)
    assert np.all(tiny[far]), f"{what}: element more than one bf16 step from the oracle away from zero"
    assert np.mean(far) <= 1e-4, f"{what}: {np.mean(far):.2e} of elements more than one step away"


def _append_case(W, inp):
    d = W.device_inputs(inp)
    W.append_latent(d["x"], d["A_K"], d["A_V"], d["pos"], d["C_K"], d["C_V"])
    torch.cuda.synchronize()
    CK_ref, CV_ref, cK, cV = O.apply_append(inp)
    gK = d["C_K"].view(torch.int16).cpu().numpy().view(np.uint16)
    gV = d["C_V"].view(torch.int16).cpu().numpy().view(np.uint16)
    for b in range(inp.nb):
        p = int(inp.pos[b])
        okK = appended_row_ok(gK[b, :, p], cK[b], inp.x[b:b + 1], inp.A_K, inp.nh, inp.r)
        okV = appended_row_ok(gV[b, :, p], cV[b], inp.x[b:b + 1], inp.A_V, inp.nh, inp.r)
        assert okK.all() and okV.all(), f"appended latent row of sequence {b} outside the rounding bound"
    rows = [b for b in range(inp.nb) if 0 <= int(inp.pos[b]) < inp.L_cap]
    for g, lat, tag in ((gK, cK, "K"), (gV, cV, "V")):
        got = np.stack([g[b, :, int(inp.pos[b])] for b in rows])
        appended_rows_within_one_ulp(got, lat[rows], f"append {tag} nb={inp.nb} nh={inp.nh} r={inp.r} E={inp.E}")
    # untouched rows stay untouched
    mask = np.ones(gK.shape[:3], bool)
    for b in range(inp.nb):
        mask[b, :, int(inp.pos[b])] = False
    assert np.array_equal(gK[mask], inp.C_K[mask]) and np.array_equal(gV[mask], inp.C_V[mask])
    return d, CK_ref, CV_ref


def test_append_small(W):
    inp = I.make_ragged_step_inputs(5, 4, 128, 48, 512, 3, 40, 40, seed=21)
    inp.pos[3] = 40        # out of range: skipped
    inp.pos[4] = -1        # out of range: skipped
    d = W.device_inputs(inp)
    W.append_latent(d["x"], d["A_K"], d["A_V"], d["pos"], d["C_K"], d["C_V"])
    torch.cuda.synchronize()
    gK = d["C_K"].view(torch.int16).cpu().numpy().view(np.uint16)
    np.testing.assert_array_equal(gK[3:], inp.C_K[3:])
    inp.pos[3] = inp.L[3] - 1
    inp.pos[4] = inp.L[4] - 1
    _append_case(W, inp)


@pytest.mark.parametrize("r", [16, 32, 64])
def test_append_ranks(W, r):
    inp = I.make_ragged_step_inputs(7, 8, 64, r, 768, 2, 30, 30, seed=30 + r)
    _append_case(W, inp)


@pytest.mark.parametrize("nb,nh,r,E,stages", [(130, 32, 32, 8192, 16), (9, 4, 32, 2560, 5)])
def test_append_long_slices(W, nb, nh, r, E, stages):
    """E-slices longer than the four stages a block keeps in flight.  130 x 32
    heads at r 32 make 96 tiles, so E = 8192 goes into 2 slices of 16 stages:
    the steady-state loop (each stage requested right after one is consumed),
    the prologue and the tail, with three 64-row tiles (the last ragged).
    9 x 4 heads, E = 2560: 2 slices of 5 stages (the tail's refill path)."""
    ks = E // 256 // stages
    assert W.append_workspace_bytes(nb, E, nh, r) >= (-(-nh * r // 64)) * 2 * (-(-nb // 64)) * ks * 64 * 64 * 4
    inp = I.make_ragged_step_inputs(nb, nh, 64, r, E, 2, 16, 16, seed=90 + stages)
    _append_case(W, inp)


def test_append_row_tiles_and_reuse(W):
    """70 sequences (two 64-row tiles, the second ragged), E split into 4
    slices of two stages each; three calls on one workspace.  Equal inputs
    give equal bits, and the third call (new token) is only right if every
    tile counter came back to zero."""
    inp = I.make_ragged_step_inputs(70, 4, 64, 32, 2048, 2, 20, 20, seed=77)
    d = W.device_inputs(inp)
    ws = W.append_workspace(70, 2048, 4, 32)
    assert W.append_workspace_bytes(70, 2048, 4, 32) > 0
    W.append_latent(d["x"], d["A_K"], d["A_V"], d["pos"], d["C_K"], d["C_V"], workspace=ws)
    first = d["C_K"].clone(), d["C_V"].clone()
    W.append_latent(d["x"], d["A_K"], d["A_V"], d["pos"], d["C_K"], d["C_V"], workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(first[0], d["C_K"]) and torch.equal(first[1], d["C_V"])
    # a different token through the same workspace
    inp2 = I.make_ragged_step_inputs(70, 4, 64, 32, 2048, 2, 20, 20, seed=78)
    d2 = W.device_inputs(inp2)
    W.append_latent(d2["x"], d2["A_K"], d2["A_V"], d2["pos"], d2["C_K"], d2["C_V"], workspace=ws)
    torch.cuda.synchronize()
    _, _, cK, cV = O.apply_append(inp2)
    gK = d2["C_K"].view(torch.int16).cpu().numpy().view(np.uint16)
    gV = d2["C_V"].view(torch.int16).cpu().numpy().view(np.uint16)
    for b in range(inp2.nb):
        p = int(inp2.pos[b])
        assert appended_row_ok(gK[b, :, p], cK[b], inp2.x[b:b + 1], inp2.A_K, inp2.nh, inp2.r).all()
        assert appended_row_ok(gV[b, :, p], cV[b], inp2.x[b:b + 1], inp2.A_V, inp2.nh, inp2.r).all()


# ---------------------------------------------------------------------------
# append into int8 caches (absmax rows, fp16 scales)
# ---------------------------------------------------------------------------
def int8_rows_check(codes, scales, exact, x, A, nh, r, what):
    """GPU int8 rows vs the oracle's quantiser on the exact latent.

    The GPU rounds its own fp32 dot (length E), so near a rounding boundary
    its decision may fall on the other side of the oracle's; the bound on
    that is the fp32 accumulation bound E 2^-24 sum_e |x_e A_e|.  Checked:
    scales within one fp16 ulp of the oracle's, every code within half a
    scale (plus that bound) of the exact value, codes within 1 of the
    oracle's and equal to them almost everywhere."""
    ref_codes, ref_scales = O.quantize_latent_rows(exact)
    xx, AA = O.upcast(x, "bf16"), O.upcast(A, "bf16")
    bound = xx.shape[1] * 2.0 ** -24 * (np.abs(xx) @ np.abs(AA)).reshape(exact.shape)
    sg = np.asarray(scales, np.float16).astype(np.float64)
    sr = ref_scales.astype(np.float64)
    ulp = np.spacing(ref_scales.astype(np.float16)).astype(np.float64)
    assert np.all(np.abs(sg - sr) <= ulp), f"{what}: scale off by more than one fp16 ulp"
    deq = codes.astype(np.float64) * sg[..., None]
    assert np.all(np.abs(deq - exact) <= 0.5 * sg[..., None] * (1 + 1e-6) + bound + 1e-30), f"{what}: code error"
    d = np.abs(codes.astype(np.int32) - ref_codes.astype(np.int32))
    assert d.max() <= 1, f"{what}: code differs by {d.max()}"
    assert np.mean(d == 0) >= 0.99, f"{what}: only {np.mean(d == 0):.4f} of codes equal"
    return float(np.mean(d == 0))


def _append_int8_case(W, inp, workspace=None):
    d = W.device_inputs(inp)
    W.append_latent(d["x"], d["A_K"], d["A_V"], d["pos"], d["C_K"], d["C_V"], s_K=d["s_K"], s_V=d["s_V"],
                    workspace=workspace)
    torch.cuda.synchronize()
    CK, CV, sK, sV, cK, cV = O.apply_append_int8(inp)
    gK, gV = d["C_K"].cpu().numpy(), d["C_V"].cpu().numpy()
    hK = d["s_K"].cpu().numpy().astype(np.float16)
    hV = d["s_V"].cpu().numpy().astype(np.float16)
    eq = []
    rows = [b for b in range(inp.nb) if 0 <= int(inp.pos[b]) < inp.L_cap]
    for lat, g, hs, A, tag in ((cK, gK, hK, inp.A_K, "K"), (cV, gV, hV, inp.A_V, "V")):
        gc = np.stack([g[b, :, int(inp.pos[b])] for b in rows])
        gs = np.stack([hs[b, :, int(inp.pos[b])] for b in rows])
        eq.append(int8_rows_check(gc, gs, lat[rows], inp.x[rows], A, inp.nh, inp.r, f"int8 append {tag}"))
    # untouched rows stay untouched
    mask = np.ones(gK.shape[:3], bool)
    for b in rows:
        mask[b, :, int(inp.pos[b])] = False
    assert np.array_equal(gK[mask], inp.C_K[mask]) and np.array_equal(gV[mask], inp.C_V[mask])
    assert np.array_equal(hK[mask], np.asarray(inp.s_K)[mask]) and np.array_equal(hV[mask], np.asarray(inp.s_V)[mask])
    print(f"[parity] int8 append nb={inp.nb} r={inp.r} E={inp.E}: codes equal to the oracle's: {min(eq):.5f}",
          flush=True)
    return d, CK, CV, sK, sV


def test_append_int8_small(W):
    inp = I.make_ragged_step_inputs(5, 4, 128, 32, 512, 3, 40, 40, seed=41, C_dt="i8")
    inp.pos[3] = 40      # out of range: skipped
    inp.pos[4] = -1
    _append_int8_case(W, inp)


@pytest.mark.parametrize("r,E,nb", [(16, 768, 7), (32, 2048, 70), (64, 1024, 9)])
def test_append_int8_ranks(W, r, E, nb):
    inp = I.make_ragged_step_inputs(nb, 4, 128, r, E, 2, 20, 20, seed=50 + r, C_dt="i8")
    _append_int8_case(W, inp)


def test_append_int8_then_decode(W):
    """The int8-cache workload's shapes end to end: the new token's latents are
    quantised on the GPU into int8 rows, then the fused decode attends over
    the cache; the oracle does both steps itself."""
    inp = I.make_ragged_step_inputs(32, 32, 128, 32, 4096, 1024, 2048, 2048, seed=404, C_dt="i8")
    d, CK, CV, sK, sV = _append_int8_case(W, inp)
    out, _, _ = W.decode_attn(d["q"], d["C_K"], d["C_V"], d["B_K"], d["B_V"], d["L"], s_K=d["s_K"], s_V=d["s_V"])
    torch.cuda.synchronize()
    g = f64(out)
    import copy
    ref_inp = copy.copy(inp)
    ref_inp.s_K, ref_inp.s_V = sK, sV
    check("int8 append + decode, whole tensor", g, oracle_all(ref_inp, C_K=CK, C_V=CV), TOL["i8"])


@pytest.mark.parametrize("peaked", [False, True])
def test_config5_full_step(W, peaked):
    """The full step at full size (append x.A_Kh at pos = L - 1, then the
    decode, automatic splits with the second-launch merge): appended rows to
    one bf16 step, every output row against the oracle's own append +
    attention."""
    c = CONFIGS[5]
    inp = c.make(q_gain=4.0 * c.H if peaked else 1.0)
    tag = "peaked" if peaked else "uniform"
    print(f"[case] config 5 {tag}: {c.describe()} sum L = {int(inp.L.sum())}", flush=True)
    d, CK_ref, CV_ref = _append_case(W, inp)
    out, _, _ = W.decode_attn(d["q"], d["C_K"], d["C_V"], d["B_K"], d["B_V"], d["L"])
    torch.cuda.synchronize()
    check(f"config 5 {tag} whole tensor ({c.nb * c.nh} rows)", f64(out), oracle_all(inp, C_K=CK_ref, C_V=CV_ref),
          TOL["bf16"])


def test_merge_across_xcds_repeated(W):
    """Many splits of one (b, h) land on every XCD (3 heads, so blocks of a
    head do not share an XCD); the in-kernel merge must equal the separate
    merge entry point bit for bit on every call."""
    inp = I.make_decode_inputs(2, 3, 128, 32, 2000, 2000, seed=99, act_dt="bf16", C_dt="bf16", q_gain=300.0)
    d = W.device_inputs(inp)
    ws = W.decode_workspace(2, 3, 128, 2000, 64)
    _, o_part, lse = W.decode_attn(d["q"], d["C_K"], d["C_V"], d["B_K"], d["B_V"], d["L"], n_splits=64,
                                   partials_only=True, workspace=ws)
    ref = W.combine_splits(o_part.clone(), lse.clone(), out_dtype=torch.bfloat16)
    outs = []
    for _ in range(20):
        out, _, _ = W.decode_attn(d["q"], d["C_K"], d["C_V"], d["B_K"], d["B_V"], d["L"], n_splits=64,
                                  workspace=ws)
        outs.append(out)
    torch.cuda.synchronize()
    for o in outs:
        assert torch.equal(o, ref)
    check("merge across XCDs", f64(ref), O.decode_attn(inp), TOL["bf16"])


# ---------------------------------------------------------------------------
# dense Flash-Decoding baseline: the oracle with r = H and identity factors
# ---------------------------------------------------------------------------
def _dense_case(nb, nh, H, L, L_cap, seed, q_gain=1.0):
    inp = I.make_decode_inputs(nb, nh, H, H, L, L_cap, seed=seed, act_dt="bf16", C_dt="bf16", q_gain=q_gain)
    eye = np.zeros((nh, H, H), np.uint16)
    eye[:, np.arange(H), np.arange(H)] = 0x3F80          # bf16 1.0
    inp.B_K = eye
    inp.B_V = eye.copy()
    return inp


@pytest.mark.parametrize("H", [64, 128])
@pytest.mark.parametrize("S", [None, 1, 3])
def test_dense_baseline_matches_oracle(W, H, S):
    L = np.array([300, 1, 0, 257, 129], np.int32)
    inp = _dense_case(5, 3, H, L, 300, seed=55 + H, q_gain=2.0 * H)
    d = W.device_inputs(inp)
    out = W.dense_decode_attn(d["q"], d["C_K"], d["C_V"], d["L"], n_splits=S)
    torch.cuda.synchronize()
    g = f64(out)
    check(f"dense H={H} S={S}", g, O.decode_attn(inp), TOL["bf16"])
    assert not g[2].any()


def test_dense_baseline_full_llava_layer(W):
    """LLaVA-7B layer shape (1 x 32 heads, H = 128, L = 1088) with full K / V."""
    inp = _dense_case(1, 32, 128, 1088, 1088, seed=2002, q_gain=4.0 * 128)
    d = W.device_inputs(inp)
    out = W.dense_decode_attn(d["q"], d["C_K"], d["C_V"], d["L"])
    torch.cuda.synchronize()
    check("dense llava layer", f64(out), O.decode_attn(inp), TOL["bf16"])


def test_large_grid_merges_in_second_launch(W):
    """64 x 8 heads x 4 splits = 2048 blocks: the partials are merged by the
    merge kernel in a second launch.  Same result as the oracle, as the
    stand-alone merge of the same partials, and as a one-launch grid."""
    L = (np.arange(64, dtype=np.int32) * 37) % 300 + 1
    inp = I.make_decode_inputs(64, 8, 64, 16, L, 300, seed=4100, act_dt="bf16", C_dt="bf16", q_gain=2.0 * 64)
    out, o_part, lse = run_decode(W, inp, n_splits=4)
    check("large grid S=4", f64(out), O.decode_attn(inp), TOL["bf16"])
    merged = W.combine_splits(o_part.contiguous(), lse.contiguous(), out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(out, merged)
    small = I.make_decode_inputs(8, 8, 64, 16, L[:8], 300, seed=4100, act_dt="bf16", C_dt="bf16", q_gain=2.0 * 64)
    out8, _, _ = run_decode(W, small, n_splits=4)          # 256 blocks: merged in-kernel
    check("small grid S=4", f64(out8), O.decode_attn(small), TOL["bf16"])


@pytest.mark.parametrize("nb", [2, 64, 65, 200, 256, 257])
def test_large_grid_ragged_many_sequences(W, nb):
    """Grids of 2048 blocks or more over 2..257 sequences (so from 256 heads
    down to 2): ragged lengths with ties, empty sequences and lengths past
    L_cap, a NaN-poisoned workspace (a partial left unwritten would show), and
    the whole output against the oracle."""
    S = 4
    nh = -(-2048 // (S * nb))
    L_cap = 64
    rng = np.random.default_rng(5000 + nb)
    L = rng.integers(0, L_cap + 1, nb).astype(np.int32)
    L[rng.integers(0, nb, max(1, nb // 8))] = 0
    L[rng.integers(0, nb, max(1, nb // 8))] = L_cap + 40
    assert nb * nh * S >= 2048
    inp = I.make_decode_inputs(nb, nh, 64, 16, L, L_cap, seed=5100 + nb, act_dt="bf16", C_dt="bf16",
                               fill=np.minimum(L, L_cap), q_gain=2.0 * 64)
    out, _, _ = run_decode(W, inp, n_splits=S, poison=True)
    g = f64(out)
    check(f"large grid nb={nb} nh={nh}", g, O.decode_attn(inp), TOL["bf16"])
    assert not g[L == 0].any(), "L = 0 must give zero rows"


def test_dense_baseline_large_grid(W):
    """2048 split blocks: the dense baseline also merges in a second launch."""
    L = (np.arange(64, dtype=np.int32) * 37) % 300 + 1
    inp = _dense_case(64, 8, 64, L, 300, seed=4200, q_gain=2.0 * 64)
    d = W.device_inputs(inp)
    out = W.dense_decode_attn(d["q"], d["C_K"], d["C_V"], d["L"], n_splits=4)
    torch.cuda.synchronize()
    check("dense large grid", f64(out), O.decode_attn(inp), TOL["bf16"])


@pytest.mark.parametrize("C_dt", ["bf16", "i8"])
def test_long_context(W, C_dt):
    """One sequence of 65536 tokens, 4 heads: the automatic rule gives 64
    splits of 1024 tokens; a near-uniform and a peaked query."""
    for gain in (1.0, 40.0 * 128):
        inp = I.make_decode_inputs(1, 4, 128, 32, 65536, 65536, seed=4300, act_dt="bf16", C_dt=C_dt,
                                   outlier_p=0.01 if C_dt == "i8" else 0.0, outlier_mul=20.0, q_gain=gain)
        out, _, _ = run_decode(W, inp)
        check(f"long context {C_dt} gain={gain}", f64(out), O.decode_attn(inp), TOL[C_dt])


@pytest.mark.parametrize("C_dt", ["f32", "bf16", "i8"])
@pytest.mark.parametrize("S", [None, 1, 3])
def test_rows_past_length_may_hold_any_bits(W, C_dt, S):
    """Cache rows at or past L[b] (and their int8 scales) filled with NaN bit
    patterns: the result must equal the run on clean rows bit for bit."""
    L = np.array([300, 5, 0, 130, 1], np.int32)
    inp = I.make_decode_inputs(5, 4, 128, 32, L, 300, seed=4400, act_dt="f32" if C_dt == "f32" else "bf16",
                               C_dt=C_dt, q_gain=4.0 * 128)
    d = W.device_inputs(inp)
    clean, _, _ = W.decode_attn(d["q"], d["C_K"], d["C_V"], d["B_K"], d["B_V"], d["L"], s_K=d.get("s_K"),
                                s_V=d.get("s_V"), n_splits=S)
    torch.cuda.synchronize()
    clean = clean.clone()
    keys = ["C_K", "C_V"] + (["s_K", "s_V"] if C_dt == "i8" else [])
    for k in keys:
        u = d[k].view(torch.uint8).view(5, 4, 300, -1)
        for b in range(5):
            u[b, :, int(L[b]):, :] = 0xFF
    poisoned, _, _ = W.decode_attn(d["q"], d["C_K"], d["C_V"], d["B_K"], d["B_V"], d["L"], s_K=d.get("s_K"),
                                   s_V=d.get("s_V"), n_splits=S)
    torch.cuda.synchronize()
    assert torch.isfinite(poisoned).all()
    assert torch.equal(poisoned, clean)
    check(f"rows past L poisoned {C_dt} S={S}", f64(poisoned), O.decode_attn(inp), TOL[C_dt])


@pytest.mark.parametrize("C_dt", ["f32", "bf16"])
def test_largest_row_offsets(W, C_dt):
    """One head whose cache rows end just below 2 GiB, the most the host
    accepts for one sequence (the kernel's row offsets are 32-bit).  All rows
    are zero except two marked ones, at a third of the cache and at its last
    row; q points at the last marked key (score 30).  Expected: the oracle's
    attention over the two marked rows merged with the zero rows (score 0,
    value 0, log-sum-exp log(count))."""
    H = r = 64
    es = 4 if C_dt == "f32" else 2
    L_cap = (1 << 31) // (r * es) - 1
    act = "f32" if C_dt == "f32" else "bf16"
    small = I.make_decode_inputs(1, 1, H, r, 2, 2, seed=4600, act_dt=act, C_dt=C_dt)
    from oracle import wsvd_oracle as WO
    sig = WO._sigma(H, None)
    K = WO.reconstruct(WO.dequant_latent(small.C_K[0, 0], small.C_dt), WO.upcast(small.B_K[0], small.B_dt))
    V = WO.reconstruct(WO.dequant_latent(small.C_V[0, 0], small.C_dt), WO.upcast(small.B_V[0], small.B_dt))
    qd = 30.0 / sig * K[1] / float(K[1] @ K[1])
    small.q[0, 0] = WO.round_to_bf16_bits(qd) if act == "bf16" else qd.astype(np.float32)
    q = WO.upcast(small.q[0, 0], small.q_dt)
    o_m, lse_m = WO.segment_attend(q, K, V, sig, 0, 2)
    ref = WO.combine(np.stack([o_m, np.zeros(H)]), np.array([lse_m, math.log(L_cap - 2)]))

    d = W.device_inputs(small)
    pos = [L_cap // 3, L_cap - 1]
    print(f"[case] largest offsets {C_dt}: L_cap={L_cap}, marked rows {pos}", flush=True)
    C_K = torch.zeros((1, 1, L_cap, r), dtype=d["C_K"].dtype, device="cuda")
    C_V = torch.zeros_like(C_K)
    for i, p in enumerate(pos):
        C_K[0, 0, p] = d["C_K"][0, 0, i]
        C_V[0, 0, p] = d["C_V"][0, 0, i]
    L = torch.tensor([L_cap], dtype=torch.int32, device="cuda")
    outs = []
    for S in (None, 3):
        out, _, _ = W.decode_attn(d["q"], C_K, C_V, d["B_K"], d["B_V"], L, n_splits=S, out_dtype=torch.float32)
        outs.append(out)
    torch.cuda.synchronize()
    del C_K, C_V
    torch.cuda.empty_cache()
    for S, out in zip((None, 3), outs):
        check(f"largest row offsets {C_dt} S={S}", f64(out)[0, 0], ref, TOL[C_dt])
