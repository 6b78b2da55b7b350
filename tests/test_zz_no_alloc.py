"""GPU: wsvd_decode_attn_noalloc (no workspace; the library's static
per-GPU scratch) against wsvd_decode_attn with a workspace, through the C
ABI, on calls in a row with shrinking inputs: bit for bit equal, and within
the oracle's tolerance."""
import numpy as np
import pytest

import oracle as O
from rank_kv_cache_flash_amd import inputs as I
from rank_kv_cache_flash_amd.configs import CONFIGS

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _run_both(W, inp, n_splits=None):
    d = W.device_inputs(inp)
    ref, _, _ = W.decode_attn(d["q"], d["C_K"], d["C_V"], d["B_K"], d["B_V"], d["L"], s_K=d.get("s_K"),
                              s_V=d.get("s_V"), n_splits=n_splits)
    got = W.decode_attn_noalloc(d["q"], d["C_K"], d["C_V"], d["B_K"], d["B_V"], d["L"], s_K=d.get("s_K"),
                                s_V=d.get("s_V"), n_splits=n_splits)
    torch.cuda.synchronize()
    return ref, got


def test_noalloc_matches_workspace_entry_point():
    from rank_kv_cache_flash_amd import wsvd as W
    W.lib()
    L = (np.arange(64, dtype=np.int32) * 37) % 300 + 1
    cases = [
        # 64 x 8 heads x 4 splits = 2048 blocks: partials in the scratch, merged by a second launch
        ("large grid, S=4", I.make_decode_inputs(64, 8, 64, 16, L, 300, seed=4800, act_dt="bf16", C_dt="bf16",
                                                 q_gain=2.0 * 64), 4),
        # the LLaVA-7B layer: 160 blocks, merged in the split kernel
        ("LLaVA-7B layer, automatic splits", CONFIGS[2].make(q_gain=4.0 * 128), None),
        # smaller again, int8 cache, ragged lengths with an empty sequence
        ("int8, 3 x 4 heads", I.make_decode_inputs(3, 4, 128, 32, np.array([300, 0, 77], np.int32), 300,
                                                   seed=4801, act_dt="bf16", C_dt="i8", outlier_p=0.01,
                                                   outlier_mul=20.0, q_gain=4.0 * 128), 3),
    ]
    for name, inp, S in cases:
        print(f"[case] noalloc {name}", flush=True)
        ref, got = _run_both(W, inp, S)
        assert torch.equal(got, ref), f"{name}: no-allocation entry point differs from the workspace one"
        want = O.decode_attn(inp)
        g = got.float().cpu().numpy().astype(np.float64)
        err = float(np.max(np.abs(g - want)) / np.max(np.abs(want)))
        print(f"[parity] noalloc {name}: bitwise equal to wsvd_decode_attn, max|err|/max|ref| = {err:.3e}",
              flush=True)
        assert err <= 2e-2


def test_noalloc_rejects_too_large():
    from rank_kv_cache_flash_amd import wsvd as W
    inp = I.make_decode_inputs(1, 32, 128, 32, 4, 4096, seed=1, act_dt="bf16", C_dt="bf16")
    d = W.device_inputs(inp)
    with pytest.raises(W.WsvdError, match="workspace"):
        W.decode_attn_noalloc(d["q"], d["C_K"], d["C_V"], d["B_K"], d["B_V"], d["L"], n_splits=1100)
