"""Graph replay.  The decode (merged in the kernel, or in a second launch on a
large grid) and the append + decode step are captured once in a HIP graph
and replayed several times, with eager calls on the same workspaces and
other eager work between the replays.  Every replay must equal the eager
call bit for bit: the merge and tile counters are reset by the kernels that
use them, so nothing in the graph clears memory.  The eager result is also
checked against the fp64 oracle."""
import numpy as np
import pytest

import oracle as O
from rank_kv_cache_flash_amd import inputs as I

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL_BF16 = 2e-2
REPLAYS = 4


@pytest.fixture(scope="module")
def W():
    from rank_kv_cache_flash_amd import wsvd
    wsvd.lib()
    return wsvd


def rel(g, ref):
    g = g.float().cpu().numpy().astype(np.float64)
    return float(np.max(np.abs(g - ref)) / max(np.max(np.abs(ref)), 1e-300))


def capture(fn):
    """One untimed call on a side stream, then fn captured into a graph."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _decode_replays(W, inp, n_splits, what):
    d = W.device_inputs(inp)
    nb, nh, H = inp.q.shape
    ws = W.decode_workspace(nb, nh, H, inp.L_cap, n_splits or 0)
    out_g = torch.empty((nb, nh, H), dtype=torch.bfloat16, device="cuda")
    out_e = torch.empty_like(out_g)

    def call(out):
        W.decode_attn(d["q"], d["C_K"], d["C_V"], d["B_K"], d["B_V"], d["L"], n_splits=n_splits, out=out,
                      workspace=ws, stream=torch.cuda.current_stream())

    call(out_e)
    torch.cuda.synchronize()
    e = rel(out_e, O.decode_attn(inp))
    print(f"[parity] graph {what} eager: {e:.3e}", flush=True)
    assert e <= TOL_BF16
    ref = out_e.clone()
    g = capture(lambda: call(out_g))
    for k in range(REPLAYS):
        out_g.fill_(float("nan"))          # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g, ref), f"{what}: replay {k} differs from the eager call"
        call(out_e)                        # an eager call on the same workspace
        torch.cuda.synchronize()
        assert torch.equal(out_e, ref), f"{what}: eager call after replay {k} differs"


def test_graph_decode_merged_in_kernel(W):
    """1 x 32 heads, 1088 tokens, automatic splits: the last block of each
    head merges its splits, then resets the head's counter."""
    print("[case] graph decode nb=1 nh=32 H=128 r=32 L=1088 S=auto", flush=True)
    inp = I.make_decode_inputs(1, 32, 128, 32, 1088, 1088, seed=7100, act_dt="bf16", C_dt="bf16", q_gain=256.0)
    _decode_replays(W, inp, None, "in-kernel merge")


def test_graph_decode_merged_in_second_launch(W):
    """2 x 32 heads x 64 splits = 4096 blocks: the partials are merged by the
    merge kernel, a second node of the graph."""
    print("[case] graph decode nb=2 nh=32 H=128 r=32 L_cap=2048 S=64", flush=True)
    L = np.array([2048, 1500], np.int32)
    inp = I.make_decode_inputs(2, 32, 128, 32, L, 2048, seed=7200, act_dt="bf16", C_dt="bf16", q_gain=256.0)
    _decode_replays(W, inp, 64, "second-launch merge")


@pytest.mark.parametrize("C_dt", ["bf16", "i8"])
def test_graph_append_then_decode(W, C_dt):
    """The whole step (append the new token's latents, then attend) in one
    graph; the caches are restored between replays, and every replay's caches
    and output equal those of the same step run eagerly."""
    print(f"[case] graph append+decode nb=8 nh=8 H=128 r=32 E=1024 C={C_dt}", flush=True)
    inp = I.make_ragged_step_inputs(8, 8, 128, 32, 1024, 20, 300, 300, seed=7300, C_dt=C_dt)
    d = W.device_inputs(inp)
    aws = W.append_workspace(inp.nb, inp.E, inp.nh, inp.r)
    dws = W.decode_workspace(inp.nb, inp.nh, inp.H, inp.L_cap)
    keys = ["C_K", "C_V"] + (["s_K", "s_V"] if C_dt == "i8" else [])
    pristine = {k: d[k].clone() for k in keys}
    out = torch.empty((inp.nb, inp.nh, inp.H), dtype=torch.bfloat16, device="cuda")

    def restore():
        for k in keys:
            d[k].copy_(pristine[k])

    def step():
        st = torch.cuda.current_stream()
        W.append_latent(d["x"], d["A_K"], d["A_V"], d["pos"], d["C_K"], d["C_V"], s_K=d.get("s_K"),
                        s_V=d.get("s_V"), workspace=aws, stream=st)
        W.decode_attn(d["q"], d["C_K"], d["C_V"], d["B_K"], d["B_V"], d["L"], s_K=d.get("s_K"), s_V=d.get("s_V"),
                      out=out, workspace=dws, stream=st)

    step()
    torch.cuda.synchronize()
    ref_out = out.clone()
    ref_cache = {k: d[k].clone() for k in keys}
    if C_dt == "bf16":
        CK, CV, _, _ = O.apply_append(inp)
        e = rel(ref_out, O.decode_attn(inp, C_K=CK, C_V=CV))
        print(f"[parity] graph append+decode eager: {e:.3e}", flush=True)
        assert e <= TOL_BF16
    restore()
    g = capture(step)
    for k in range(REPLAYS):
        restore()
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out), f"replay {k}: output differs from the eager step"
        for key in keys:
            assert torch.equal(d[key], ref_cache[key]), f"replay {k}: {key} differs from the eager step"
