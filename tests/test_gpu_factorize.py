"""GPU parity of the offline per-head factorisation (truncated SVD and the
weighted alternating least squares half-steps) against the fp64 oracle."""
import numpy as np
import pytest

import oracle as O
from rank_kv_cache_flash_amd import inputs as I

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

# fp32 outputs of fp64 arithmetic: a few units of fp32 rounding, scaled by
# the largest magnitude involved.
TOL = 1e-5


@pytest.fixture(scope="module")
def W_():
    from rank_kv_cache_flash_amd import wsvd
    wsvd.lib()
    return wsvd


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    return t.cpu().numpy().astype(np.float64)


def relmax(g, ref):
    return float(np.max(np.abs(g - ref)) / max(np.max(np.abs(ref)), 1e-300))


def svd_gpu(W_, W, nh, r):
    A, B, s, sw = W_.factorize_svd(dev(W), nh, r)
    torch.cuda.synchronize()
    return host(A), host(B), host(s), sw.cpu().numpy()


def check_svd(W, nh, r, A, B, sig, sweeps, *, gap_ok=True):
    E, NH = W.shape
    H = NH // nh
    W64 = W.astype(np.float64)
    A_o, B_o = O.svd_factors(W64, nh, r)
    assert np.all(sweeps > 0), sweeps                      # every head converged
    for h in range(nh):
        Wh = W64[:, h * H:(h + 1) * H]
        s_ref = np.zeros(H)
        s_ref[:min(E, H)] = np.linalg.svd(Wh, compute_uv=False)
        smax = max(s_ref[0], 1e-300)
        assert np.max(np.abs(sig[h] - s_ref)) <= TOL * smax  # all H singular values, descending
        Bh, Ah = B[h], A[:, h * r:(h + 1) * r]
        assert np.max(np.abs(Bh @ Bh.T - np.eye(r))) <= 2 * TOL   # orthonormal rows
        idx = np.argmax(np.abs(Bh), axis=1)
        assert np.all(Bh[np.arange(r), idx] > 0)                    # sign convention
        assert relmax(Ah, Wh @ Bh.T) <= TOL                          # A_h = W_h B_h^T
        # Eckart-Young: the residual energy is the discarded spectrum.
        res = np.sum((Wh - Ah @ Bh) ** 2)
        assert abs(res - np.sum(s_ref[r:] ** 2)) <= 1e-4 * np.sum(s_ref ** 2)
        if gap_ok:
            # Unique rank-r projection: the product matches the oracle's.
            assert relmax(Ah @ Bh, A_o[:, h * r:(h + 1) * r] @ B_o[h]) <= 10 * TOL
            # Rows agree with the oracle's right singular vectors up to sign.
            d = np.minimum(np.abs(Bh - B_o[h]).max(1), np.abs(Bh + B_o[h]).max(1))
            assert d.max() <= 1e-4, d.max()


@pytest.mark.parametrize("E,nh,H,r,spectrum", [
    (300, 3, 64, 16, "gaussian"),
    (1000, 2, 128, 32, "powerlaw"),
    (777, 2, 128, 64, "gaussian"),
    (64, 1, 64, 64, "powerlaw"),        # r = H: the factors are a rotation of W
    (96, 2, 128, 48, "powerlaw"),       # E < H: rank E heads
])
def test_svd_matches_oracle(W_, E, nh, H, r, spectrum):
    W = I.make_projection_weights(E, nh, H, seed=2000 + E + r, spectrum=spectrum)
    A, B, sig, sw = svd_gpu(W_, W, nh, r)
    print(f"[parity] svd E={E} nh={nh} H={H} r={r} {spectrum}: sweeps {sw.tolist()}", flush=True)
    check_svd(W, nh, r, A, B, sig, sw)


def test_svd_llava_layer(W_):
    """The key projection of a LLaVA-7B layer: E 4096, 32 heads of 128, rank 32."""
    W = I.make_projection_weights(4096, 32, 128, seed=2100, spectrum="powerlaw")
    A, B, sig, sw = svd_gpu(W_, W, 32, 32)
    print(f"[parity] svd llava layer: sweeps max {sw.max()}", flush=True)
    check_svd(W, 32, 32, A, B, sig, sw)


def test_svd_rank_deficient_and_zero_heads(W_):
    """Head 0 has rank 5 < r, head 1 is zero: the factors still reproduce W,
    B keeps orthonormal rows (completed), and the trailing spectrum is ~0."""
    E, H, r = 256, 64, 16
    W = np.zeros((E, 2 * H), np.float32)
    W[:, :H] = I.make_projection_weights(E, 1, H, seed=2200, spectrum="lowrank", rank=5)
    A, B, sig, sw = svd_gpu(W_, W, 2, r)
    W64 = W.astype(np.float64)
    for h in range(2):
        Wh, Ah, Bh = W64[:, h * H:(h + 1) * H], A[:, h * r:(h + 1) * r], B[h]
        assert np.max(np.abs(Bh @ Bh.T - np.eye(r))) <= 2 * TOL
        assert np.max(np.abs(Ah @ Bh - Wh)) <= TOL * max(np.abs(Wh).max(), 1.0)
    assert np.max(sig[0, 5:]) <= 1e-5 * sig[0, 0]
    assert np.all(sig[1] == 0) and np.all(A[:, r:] == 0)
    # The zero head's rows come from the completion: unit vectors e_0 .. e_{r-1}.
    assert np.array_equal(B[1], np.eye(r, H))


def test_svd_known_factors(W_):
    """W_h = U diag(s) V^T with chosen orthonormal U, V and distinct s: the
    singular values come back as s and the rows of B as the columns of V."""
    E, H, r = 512, 64, 16
    g = np.random.default_rng(2300)
    U, _ = np.linalg.qr(g.standard_normal((E, H)))
    V, _ = np.linalg.qr(g.standard_normal((H, H)))
    s = np.linspace(3.0, 0.5, H)
    W = ((U * s) @ V.T).astype(np.float32)
    A, B, sig, sw = svd_gpu(W_, W, 1, r)
    assert np.max(np.abs(sig[0] - s)) <= 1e-5 * s[0]
    Vr = V[:, :r].T
    d = np.minimum(np.abs(B[0] - Vr).max(1), np.abs(B[0] + Vr).max(1))
    assert d.max() <= 1e-4


def test_svd_deterministic(W_):
    W = dev(I.make_projection_weights(1024, 4, 128, seed=2400, spectrum="gaussian"))
    outs = [W_.factorize_svd(W, 4, 32) for _ in range(2)]
    torch.cuda.synchronize()
    for a, b in zip(*outs):
        assert torch.equal(a, b)


def als_inputs(E, nh, H, r, seed):
    W = I.make_projection_weights(E, nh, H, seed=seed, spectrum="powerlaw")
    F = I.make_fisher_weights(E, nh, H, seed=seed)
    A0, B0 = O.svd_factors(W.astype(np.float64), nh, r)
    return W, F, A0.astype(np.float32), B0.astype(np.float32)


@pytest.mark.parametrize("E,nh,H,r", [(200, 3, 64, 16), (300, 2, 128, 32), (150, 2, 128, 48), (257, 2, 128, 64),
                                      (100, 1, 64, 64)])
def test_weighted_updates_match_oracle(W_, E, nh, H, r):
    W, F, A0, B0 = als_inputs(E, nh, H, r, 2500 + E + r)
    A = host(W_.weighted_update_A(dev(W), dev(F), dev(B0)))
    A_ref = O.als_step_A(W, F, B0.astype(np.float64), nh)
    eA = relmax(A, A_ref)
    B = host(W_.weighted_update_B(dev(W), dev(F), dev(A0), nh))
    B_ref = O.als_step_B(W, F, A0.astype(np.float64), nh)
    eB = relmax(B, B_ref)
    print(f"[parity] weighted E={E} nh={nh} H={H} r={r}: A {eA:.2e} B {eB:.2e}", flush=True)
    assert eA <= TOL and eB <= TOL


def test_weighted_uniform_weights_reduce_to_projection(W_):
    """F = 1 and orthonormal B: the weighted A step is the plain least-squares
    fit W_h B_h^T, i.e. the SVD's own latent."""
    E, nh, H, r = 512, 2, 128, 32
    W = I.make_projection_weights(E, nh, H, seed=2600, spectrum="powerlaw")
    A_svd, B_svd, _, _ = W_.factorize_svd(dev(W), nh, r)
    A = W_.weighted_update_A(dev(W), torch.ones((E, nh * H), dtype=torch.float32, device="cuda"), B_svd)
    torch.cuda.synchronize()
    assert relmax(host(A), host(A_svd)) <= TOL


def test_weighted_iterations_descend_like_oracle(W_):
    """Three (A, B) rounds on the GPU: the weighted objective never rises, and
    the final product matches three oracle rounds."""
    E, nh, H, r = 256, 2, 64, 16
    W, F, A0, B0 = als_inputs(E, nh, H, r, 2700)
    Wd, Fd, B = dev(W), dev(F), dev(B0)
    obj = [O.weighted_objective(W, F, A0.astype(np.float64), B0.astype(np.float64), nh).sum()]
    for _ in range(3):
        A = W_.weighted_update_A(Wd, Fd, B)
        B = W_.weighted_update_B(Wd, Fd, A, nh)
        torch.cuda.synchronize()
        obj.append(O.weighted_objective(W, F, host(A), host(B), nh).sum())
    assert all(b <= a * (1 + 1e-6) for a, b in zip(obj, obj[1:])), obj
    A_o, B_o = O.weighted_factors(W, F, A0, B0, nh, 3)
    for h in range(nh):
        P = host(A)[:, h * r:(h + 1) * r] @ host(B)[h]
        Po = A_o[:, h * r:(h + 1) * r] @ B_o[h]
        assert relmax(P, Po) <= 1e-4


def test_weighted_llava_layer_sampled(W_):
    """E 4096, 32 heads of 128, rank 32: sampled rows of the A step and two
    heads of the B step against the oracle."""
    E, nh, H, r = 4096, 32, 128, 32
    W, F, A0, B0 = als_inputs(E, nh, H, r, 2800)
    Wd, Fd = dev(W), dev(F)
    A = host(W_.weighted_update_A(Wd, Fd, dev(B0)))
    B = host(W_.weighted_update_B(Wd, Fd, dev(A0), nh))
    rows = np.random.default_rng(0).choice(E, 64, replace=False)
    A_ref = O.als_step_A(W[rows], F[rows], B0.astype(np.float64), nh)
    assert relmax(A[rows], A_ref) <= TOL
    for h in (0, 31):
        sl = slice(h * H, (h + 1) * H)
        B_ref = O.als_step_B(W[:, sl], F[:, sl], A0[:, h * r:(h + 1) * r].astype(np.float64), 1)
        assert relmax(B[h], B_ref[0]) <= TOL
