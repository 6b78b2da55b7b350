"""GPU parity of the conventional shared-latent decode (the ablation the
per-head path is measured against) with the fp64 oracle."""
import numpy as np
import pytest

import oracle as O
from rank_kv_cache_flash_amd import inputs as I

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = 2e-2   # bf16 inputs and outputs, as for the per-head decode


@pytest.fixture(scope="module")
def W():
    from rank_kv_cache_flash_amd import wsvd
    wsvd.lib()
    return wsvd


def rel(g, ref):
    return float(np.max(np.abs(np.asarray(g, np.float64) - ref)) / max(np.max(np.abs(ref)), 1e-300))


def run(W, inp, n_splits=None, out_dtype=None):
    d = W.shared_device_inputs(inp)
    out = W.shared_decode_attn(d["q"], d["C_K"], d["C_V"], d["B_K"], d["B_V"], d["L"], n_splits=n_splits,
                               out_dtype=out_dtype)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("H,R", [(64, 512), (128, 1024), (128, 2048), (64, 2048)])
@pytest.mark.parametrize("S", [None, 1, 3])
def test_shared_ragged(W, H, R, S):
    L = np.array([300, 1, 0, 257], np.int32)
    inp = I.make_shared_inputs(4, 3, H, R, L, 300, seed=3000 + H + R, q_gain=4.0 * H)
    g = run(W, inp, n_splits=S)
    e = rel(g, O.decode_attn_shared(inp))
    print(f"[parity] shared H={H} R={R} S={S}: {e:.3e}", flush=True)
    assert e <= TOL
    assert not g[2].any()


def test_shared_peaked_and_fp32_out(W):
    inp = I.make_shared_inputs(2, 4, 128, 1024, np.array([500, 77], np.int32), 512, seed=3100, q_gain=300.0 * 128)
    g = run(W, inp, out_dtype=torch.float32)
    e = rel(g, O.decode_attn_shared(inp))
    print(f"[parity] shared peaked: {e:.3e}", flush=True)
    assert e <= TOL


def test_shared_many_sequences(W):
    """Ten sequences: two merge groups, the second one partial."""
    L = np.arange(10, dtype=np.int32) * 13 + 1
    inp = I.make_shared_inputs(10, 2, 128, 512, L, 130, seed=3200, q_gain=4.0 * 128)
    g = run(W, inp, n_splits=2)
    assert rel(g, O.decode_attn_shared(inp)) <= TOL


def test_shared_llava_layer_sampled(W):
    """One sequence, 32 heads of 128, shared rank 1024 (the per-head workload's
    cache size at r = 32), 1088 tokens; eight heads against the oracle."""
    inp = I.make_shared_inputs(1, 32, 128, 1024, 1088, 1088, seed=3300, q_gain=4.0 * 128)
    g = run(W, inp)
    pairs = [(0, h) for h in (0, 5, 9, 14, 18, 23, 27, 31)]
    ref = O.decode_attn_shared(inp, pairs=pairs)
    e = rel(np.stack([g[p] for p in pairs]), np.stack([ref[p] for p in pairs]))
    print(f"[parity] shared llava layer: {e:.3e}", flush=True)
    assert e <= TOL


def test_shared_block_diagonal_matches_per_head_kernel(W):
    """Per-head latents placed side by side in a shared latent of rank nh r
    with a block-diagonal factor: the shared-latent kernel, the per-head
    kernel and the per-head oracle agree."""
    nb, nh, H, r = 2, 16, 128, 64
    L = np.array([400, 129], np.int32)
    ph = I.make_decode_inputs(nb, nh, H, r, L, 400, seed=3400, act_dt="bf16", C_dt="bf16", q_gain=4.0 * H)
    R = nh * r
    C_K = np.zeros((nb, 400, R), np.uint16)
    C_V = np.zeros_like(C_K)
    B_K = np.zeros((R, nh * H), np.uint16)
    B_V = np.zeros_like(B_K)
    for h in range(nh):
        C_K[:, :, h * r:(h + 1) * r] = ph.C_K[:, h]
        C_V[:, :, h * r:(h + 1) * r] = ph.C_V[:, h]
        B_K[h * r:(h + 1) * r, h * H:(h + 1) * H] = ph.B_K[h]
        B_V[h * r:(h + 1) * r, h * H:(h + 1) * H] = ph.B_V[h]
    sh = I.SharedInputs(nb=nb, nh=nh, H=H, R=R, L_cap=400, q=ph.q, C_K=C_K, C_V=C_V, B_K=B_K, B_V=B_V, L=L)
    g_shared = run(W, sh)
    d = W.device_inputs(ph)
    per_head, _, _ = W.decode_attn(d["q"], d["C_K"], d["C_V"], d["B_K"], d["B_V"], d["L"])
    torch.cuda.synchronize()
    ref = O.decode_attn(ph)
    assert rel(g_shared, ref) <= TOL
    assert rel(g_shared, per_head.float().cpu().numpy().astype(np.float64)) <= TOL
