"""The C ABI on the host: the library loads, exports every declared symbol,
and rejects bad arguments with the documented status before launching.

No call here reaches a kernel: each error case fails host validation, which
runs before any HIP call, so these tests need no GPU.
"""
import ctypes
import os
import re

import pytest

torch = pytest.importorskip("torch")

from rank_kv_cache_flash_amd import wsvd  # noqa: E402

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "wsvd.h")

OK, ENULL, ESHAPE, EDTYPE, EUNSUP, EALIGN, EWS, EHIP = 0, -1, -2, -3, -4, -5, -6, -7
F32, BF16, F16, I8 = 0, 1, 2, 3


def declared_symbols():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(wsvd_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(wsvd.LIB_PATH):
        pytest.fail("libwsvd.so is not built (python -m rank_kv_cache_flash_amd.build)")
    return wsvd.lib()


def test_exports_every_declared_symbol(L):
    syms = declared_symbols()
    assert {"wsvd_decode_attn", "wsvd_append_latent", "wsvd_combine_splits"} <= set(syms)
    for s in syms:
        assert hasattr(L, s), f"{s} declared in wsvd.h but not exported"


def test_status_strings_and_version(L):
    for st in (OK, ENULL, ESHAPE, EDTYPE, EUNSUP, EALIGN, EWS, EHIP, -99):
        assert wsvd.status_string(st)
    assert "gfx950" in wsvd.version()


def test_split_rule_and_workspace_sizes(L):
    assert wsvd.decode_num_splits(1, 32, 1088, 5) == 5
    assert wsvd.decode_num_splits(1, 32, 1088, 0) >= 1
    assert wsvd.decode_num_splits(0, 32, 1088, 0) == ESHAPE
    assert wsvd.decode_num_splits(1, 32, 10, 11) == ESHAPE
    for (nb, nh, H, Lc, S) in [(1, 4, 64, 256, 3), (16, 32, 128, 4096, 0), (2, 3, 64, 100, 7)]:
        s = wsvd.decode_num_splits(nb, nh, Lc, S)
        off = wsvd.decode_lse_offset(nb, nh, H, Lc, S)
        ws = wsvd.decode_workspace_bytes(nb, nh, H, Lc, S)
        assert off >= nb * nh * s * H * 4 and off % 256 == 0
        assert ws >= off + nb * nh * s * 4
    assert wsvd.decode_workspace_bytes(0, 1, 64, 1, 0) == 0
    assert wsvd.append_workspace_bytes(64, 4096, 32, 48) % 256 == 0
    assert wsvd.append_workspace_bytes(64, 4096, 32, 48) >= 64 * 2 * 32 * 48 * 4
    assert wsvd.append_workspace_bytes(7, 768, 8, 16) == 0      # no E split: no scratch


# Fake, well-aligned device addresses: validation must reject before use.
# Every helper defaults to a workspace that is too small, so a case that
# passed the check it targets would stop at WSVD_ERR_WORKSPACE instead of
# launching a kernel on fake pointers.
P = 0x7F0000000000
WS = 16


def decode(L, **kw):
    a = dict(nb=1, nh=4, H=64, r=16, L_cap=256, Lp=P, q=P, q_dt=F32, C_K=P, C_V=P, C_dt=F32, s_K=None,
             s_V=None, B_K=P, B_V=P, B_dt=F32, scale=0.0, S=0, ws=P, ws_bytes=WS, out=P, out_dt=F32)
    a.update(kw)
    v = ctypes.c_void_p
    return L.wsvd_decode_attn(a["nb"], a["nh"], a["H"], a["r"], a["L_cap"], v(a["Lp"]), v(a["q"]), a["q_dt"],
                              v(a["C_K"]), v(a["C_V"]), a["C_dt"], v(a["s_K"]), v(a["s_V"]), v(a["B_K"]),
                              v(a["B_V"]), a["B_dt"], a["scale"], a["S"], v(a["ws"]), a["ws_bytes"], v(a["out"]),
                              a["out_dt"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(nb=0), ESHAPE), (dict(nh=-1), ESHAPE), (dict(H=0), ESHAPE), (dict(L_cap=0), ESHAPE),
    (dict(r=128), ESHAPE), (dict(S=-1), ESHAPE), (dict(S=257), ESHAPE),
    (dict(Lp=None), ENULL), (dict(q=None), ENULL), (dict(C_K=None), ENULL), (dict(C_V=None), ENULL),
    (dict(B_K=None), ENULL), (dict(B_V=None), ENULL),
    (dict(C_dt=I8), ENULL), (dict(C_dt=I8, s_K=P), ENULL),
    (dict(q_dt=I8), EDTYPE), (dict(B_dt=7), EDTYPE), (dict(C_dt=F16), EDTYPE), (dict(out_dt=I8), EDTYPE),
    (dict(H=96), EUNSUP), (dict(r=24), EUNSUP), (dict(H=256, r=16), EUNSUP), (dict(r=8), EUNSUP),
    (dict(q=P + 8), EALIGN), (dict(C_K=P + 4), EALIGN), (dict(B_V=P + 2), EALIGN), (dict(out=P + 8), EALIGN),
    (dict(C_dt=I8, s_K=P, s_V=P + 2), EALIGN), (dict(Lp=P + 4), EALIGN),
    (dict(ws=None), EWS), (dict(ws_bytes=16), EWS), (dict(ws=P + 16), EWS),
    # one (b, h)'s rows must stay below 2 GiB (32-bit row offsets in the kernel)
    (dict(nh=1, r=64, L_cap=1 << 23), ESHAPE), (dict(nh=1, r=64, L_cap=(1 << 23) - 1), EWS),
    (dict(nh=1, r=64, C_dt=I8, s_K=P, s_V=P, L_cap=1 << 25), ESHAPE),
])
def test_decode_rejects(L, kw, want):
    assert decode(L, **kw) == want


def test_decode_workspace_boundary(L):
    need = wsvd.decode_workspace_bytes(1, 4, 64, 256, 3)
    assert decode(L, S=3, ws_bytes=need - 1) == EWS


def test_combine_rejects(L):
    v = ctypes.c_void_p
    f = L.wsvd_combine_splits
    assert f(0, 1, 64, 2, v(P), v(P), v(P), F32, None) == ESHAPE
    assert f(1, 1, 64, 0, v(P), v(P), v(P), F32, None) == ESHAPE
    assert f(1, 1, 64, 2, None, v(P), v(P), F32, None) == ENULL
    assert f(1, 1, 64, 2, v(P), v(P), None, F32, None) == ENULL
    assert f(1, 1, 64, 2, v(P), v(P), v(P), I8, None) == EDTYPE
    assert f(1, 1, 96, 2, v(P), v(P), v(P), F32, None) == EUNSUP
    assert f(1, 1, 64, 2, v(P + 4), v(P), v(P), F32, None) == EALIGN


def append(L, **kw):
    a = dict(nb=64, E=4096, nh=32, r=48, L_cap=8192, x=P, x_dt=BF16, A_K=P, A_V=P, A_dt=BF16, pos=P, C_K=P,
             C_V=P, C_dt=BF16, s_K=None, s_V=None, ws=P, ws_bytes=WS)
    a.update(kw)
    v = ctypes.c_void_p
    return L.wsvd_append_latent(a["nb"], a["E"], a["nh"], a["r"], a["L_cap"], v(a["x"]), a["x_dt"], v(a["A_K"]),
                                v(a["A_V"]), a["A_dt"], v(a["pos"]), v(a["C_K"]), v(a["C_V"]), a["C_dt"],
                                v(a["s_K"]), v(a["s_V"]), v(a["ws"]), a["ws_bytes"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(nb=0), ESHAPE), (dict(E=-4), ESHAPE), (dict(L_cap=0), ESHAPE),
    (dict(x=None), ENULL), (dict(A_V=None), ENULL), (dict(pos=None), ENULL), (dict(C_K=None), ENULL),
    (dict(x_dt=F32), EDTYPE), (dict(A_dt=F16), EDTYPE), (dict(C_dt=F16), EDTYPE),
    (dict(C_dt=I8), ENULL), (dict(C_dt=I8, s_K=P), ENULL), (dict(C_dt=I8, s_K=P, s_V=P), EUNSUP),
    (dict(C_dt=I8, s_K=P, s_V=P + 2, r=32), EALIGN), (dict(C_dt=I8, s_K=P, s_V=P, r=32), EWS),
    (dict(r=40), EUNSUP), (dict(E=4000), EUNSUP),
    (dict(s_K=P), ESHAPE),
    (dict(x=P + 2), EALIGN), (dict(A_K=P + 8), EALIGN), (dict(C_V=P + 4), EALIGN),
    (dict(ws=None), EWS), (dict(ws_bytes=100), EWS),
])
def test_append_rejects(L, kw, want):
    assert append(L, **kw) == want


def test_binding_refuses_cpu_tensors(L):
    q = torch.zeros(1, 4, 64)
    c = torch.zeros(1, 4, 256, 16)
    b = torch.zeros(4, 16, 64)
    with pytest.raises(ValueError, match="GPU"):
        wsvd.decode_attn(q, c, c, b, b, torch.zeros(1, dtype=torch.int32))


# Shape and dtype checks run on tensor metadata before the device check, so
# every refusal below is reached with CPU tensors and launches nothing.
def _dec(nb=2, nh=4, H=64, r=16, Lc=256, dt=torch.bfloat16, cdt=torch.bfloat16):
    return dict(q=torch.zeros(nb, nh, H, dtype=dt), C_K=torch.zeros(nb, nh, Lc, r, dtype=cdt),
                C_V=torch.zeros(nb, nh, Lc, r, dtype=cdt), B_K=torch.zeros(nh, r, H, dtype=dt),
                B_V=torch.zeros(nh, r, H, dtype=dt), L=torch.zeros(nb, dtype=torch.int32))


@pytest.mark.parametrize("change,msg", [
    (dict(C_V=torch.zeros(2, 4, 255, 16, dtype=torch.bfloat16)), "C_V must have shape"),
    (dict(C_V=torch.zeros(2, 4, 256, 16, dtype=torch.float32)), "C_V must be one of"),
    (dict(B_K=torch.zeros(4, 32, 64, dtype=torch.bfloat16)), "B_K must have shape"),
    (dict(B_V=torch.zeros(4, 16, 64, dtype=torch.float16)), "B_V must be one of"),
    (dict(L=torch.zeros(2, dtype=torch.int64)), "L must be one of"),
    (dict(L=torch.zeros(3, dtype=torch.int32)), "L must have shape"),
    (dict(out=torch.zeros(2, 4, 32, dtype=torch.bfloat16)), "out must have shape"),
    (dict(q=torch.zeros(2, 4, 64, dtype=torch.int8)), "q must be one of"),
    (dict(s_K=torch.zeros(2, 4, 256, dtype=torch.float16)), "int8 caches only"),
])
def test_binding_refuses_bad_decode_shapes(L, change, msg):
    a = _dec()
    a.update(change)
    out = a.pop("out", None)
    s_K = a.pop("s_K", None)
    with pytest.raises(ValueError, match=msg):
        wsvd.decode_attn(a["q"], a["C_K"], a["C_V"], a["B_K"], a["B_V"], a["L"], out=out, s_K=s_K)
    with pytest.raises(ValueError, match=msg):
        wsvd.PreparedDecode(a["q"], a["C_K"], a["C_V"], a["B_K"], a["B_V"], a["L"], out=out, s_K=s_K,
                            workspace=torch.zeros(16, dtype=torch.uint8))


def test_binding_int8_needs_scales_of_the_cache_shape(L):
    a = _dec(cdt=torch.int8)
    with pytest.raises(ValueError, match="s_K is required"):
        wsvd.decode_attn(**a)
    with pytest.raises(ValueError, match="s_V must have shape"):
        wsvd.decode_attn(**a, s_K=torch.zeros(2, 4, 256, dtype=torch.float16),
                         s_V=torch.zeros(2, 4, 128, dtype=torch.float16))


def test_binding_refuses_bad_rope_dense_combine_shapes(L):
    a = _dec()
    c = torch.zeros(256, 32)
    with pytest.raises(ValueError, match="rope_sin must have shape"):
        wsvd.decode_attn_rope(a["q"], a["C_K"], a["C_V"], a["B_K"], a["B_V"], a["L"], c, torch.zeros(256, 16))
    with pytest.raises(ValueError, match="C_K must be one of"):
        wsvd.decode_attn_rope(a["q"], a["C_K"].float(), a["C_V"].float(), a["B_K"], a["B_V"], a["L"], c, c)
    K = torch.zeros(2, 4, 256, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="V must have shape"):
        wsvd.dense_decode_attn(a["q"], K, K[:, :, :200], a["L"])
    with pytest.raises(ValueError, match="lse_part must have shape"):
        wsvd.combine_splits(torch.zeros(2, 4, 3, 64), torch.zeros(2, 4, 2))


def test_binding_refuses_bad_append_shapes(L):
    bf = torch.bfloat16
    x = torch.zeros(3, 512, dtype=bf)
    A = torch.zeros(512, 4 * 32, dtype=bf)
    C = torch.zeros(3, 4, 64, 32, dtype=bf)
    pos = torch.zeros(3, dtype=torch.int32)
    with pytest.raises(ValueError, match="A_V must have shape"):
        wsvd.append_latent(x, A, A[:, :64], pos, C, C)
    with pytest.raises(ValueError, match="pos must have shape"):
        wsvd.append_latent(x, A, A, pos[:2], C, C)
    with pytest.raises(ValueError, match="C_K must hold 3 sequences"):
        wsvd.append_latent(x, A, A, pos, C[:2], C[:2])
    with pytest.raises(ValueError, match="x must be one of"):
        wsvd.append_latent(x.float(), A, A, pos, C, C)
    xq = torch.zeros(3, 512, dtype=torch.int8)
    Aq = torch.zeros(128, 512, dtype=torch.int8)
    sA = torch.zeros(128)
    with pytest.raises(ValueError, match="AqT_V must have shape"):
        wsvd.append_latent_w8a8(xq, torch.zeros(3), Aq, sA, Aq[:64], sA, pos, C, C)
    with pytest.raises(ValueError, match="sx must have shape"):
        wsvd.append_latent_w8a8(xq, torch.zeros(4), Aq, sA, Aq, sA, pos, C, C)


def test_binding_zero_counter_rule(L):
    """A workspace this module zero-filled remembers how much of it is still
    known to be zero; a call whose counter area reaches past that is refused
    before anything is launched."""
    ws = torch.zeros(4096, dtype=torch.uint8)
    wsvd._zero_filled(ws)
    wsvd._claim_counters(ws, 256, "first call")        # a small batch: partials from byte 256 on
    assert ws._wsvd_zero_bytes == 256
    wsvd._claim_counters(ws, 256, "same size")
    with pytest.raises(ValueError, match="must be zero"):
        wsvd._claim_counters(ws, 512, "larger batch")
    ws2 = wsvd._zero_filled(torch.zeros(4096, dtype=torch.uint8))
    wsvd._claim_counters(ws2, 512, "partials only", needs_zero=False)   # writes past byte 512, merges nothing
    wsvd._claim_counters(ws2, 512, "then with an output")
    with pytest.raises(ValueError, match="must be zero"):
        wsvd._claim_counters(ws2, 768, "larger batch")
    plain = torch.zeros(16, dtype=torch.uint8)          # not from this module: the caller's responsibility
    wsvd._claim_counters(plain, 1 << 20, "unmarked")


def dense(L, **kw):
    a = dict(nb=2, nh=4, H=128, L_cap=256, Lp=P, q=P, q_dt=BF16, K=P, V=P, kv_dt=BF16, S=0, ws=P, ws_bytes=WS,
             out=P, out_dt=BF16)
    a.update(kw)
    v = ctypes.c_void_p
    return L.wsvd_dense_decode_attn(a["nb"], a["nh"], a["H"], a["L_cap"], v(a["Lp"]), v(a["q"]), a["q_dt"], v(a["K"]),
                                    v(a["V"]), a["kv_dt"], 0.0, a["S"], v(a["ws"]), a["ws_bytes"], v(a["out"]),
                                    a["out_dt"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(nb=0), ESHAPE), (dict(L_cap=-1), ESHAPE), (dict(S=-2), ESHAPE),
    (dict(K=None), ENULL), (dict(Lp=None), ENULL),
    (dict(kv_dt=F32), EDTYPE), (dict(kv_dt=I8), EDTYPE), (dict(q_dt=I8), EDTYPE),
    (dict(H=96), EUNSUP), (dict(H=32), EUNSUP),
    (dict(V=P + 4), EALIGN), (dict(q=P + 2), EALIGN),
    ({}, EWS), (dict(ws=None), EWS),
    (dict(nb=1, nh=1, L_cap=1 << 23), ESHAPE), (dict(nb=1, nh=1, L_cap=(1 << 23) - 1), EWS),
])
def test_dense_rejects(L, kw, want):
    assert dense(L, **kw) == want


def test_w8a8_rejects(L):
    v = ctypes.c_void_p
    q = L.wsvd_w8a8_quantize_activations
    assert q(0, 4096, v(P), BF16, v(P), v(P), None) == ESHAPE
    assert q(2, 4096, None, BF16, v(P), v(P), None) == ENULL
    assert q(2, 4096, v(P), I8, v(P), v(P), None) == EDTYPE
    assert q(2, 3000, v(P), BF16, v(P), v(P), None) == EUNSUP       # not a power of two
    assert q(2, 16384, v(P), BF16, v(P), v(P), None) == EUNSUP      # above the LDS limit
    assert q(2, 128, v(P), BF16, v(P), v(P), None) == EUNSUP
    assert q(2, 4096, v(P + 2), BF16, v(P), v(P), None) == EALIGN
    p = L.wsvd_w8a8_prepare_factor
    assert p(4096, 0, v(P), BF16, v(P), v(P), None) == ESHAPE
    assert p(4096, 64, v(P), BF16, None, v(P), None) == ENULL
    assert p(4096, 64, v(P), I8, v(P), v(P), None) == EDTYPE
    assert p(1000, 64, v(P), BF16, v(P), v(P), None) == EUNSUP
    assert p(4096, 64, v(P), BF16, v(P), v(P + 4), None) == EALIGN


def append_w8(L, **kw):
    a = dict(nb=64, E=4096, nh=32, r=32, L_cap=8192, xq=P, sx=P, AK=P, AV=P, sK=P, sV=P, pos=P, C_K=P, C_V=P,
             C_dt=BF16, s_K=None, s_V=None, ws=P, ws_bytes=WS)
    a.update(kw)
    v = ctypes.c_void_p
    return L.wsvd_append_latent_w8a8(a["nb"], a["E"], a["nh"], a["r"], a["L_cap"], v(a["xq"]), v(a["sx"]),
                                     v(a["AK"]), v(a["AV"]), v(a["sK"]), v(a["sV"]), v(a["pos"]), v(a["C_K"]),
                                     v(a["C_V"]), a["C_dt"], v(a["s_K"]), v(a["s_V"]), v(a["ws"]), a["ws_bytes"],
                                     None)


@pytest.mark.parametrize("kw,want", [
    (dict(nb=0), ESHAPE), (dict(xq=None), ENULL), (dict(sV=None), ENULL), (dict(pos=None), ENULL),
    (dict(C_dt=F16), EDTYPE), (dict(C_dt=I8), ENULL), (dict(C_dt=I8, s_K=P, s_V=P, r=48), EUNSUP),
    (dict(E=4096 + 256), EUNSUP), (dict(r=24), EUNSUP), (dict(AK=P + 8), EALIGN), (dict(sx=P + 4), EALIGN),
    ({}, EWS), (dict(ws=None), EWS), (dict(C_dt=I8, s_K=P, s_V=P), EWS),
])
def test_append_w8a8_rejects(L, kw, want):
    assert append_w8(L, **kw) == want


def rope(L, **kw):
    a = dict(nb=2, nh=4, H=128, r=32, L_cap=256, Lp=P, q=P, q_dt=BF16, C_K=P, C_V=P, C_dt=BF16, B_K=P, B_V=P,
             B_dt=BF16, cos=P, sin=P, S=0, ws=P, ws_bytes=WS, out=P, out_dt=BF16)
    a.update(kw)
    v = ctypes.c_void_p
    return L.wsvd_decode_attn_rope(a["nb"], a["nh"], a["H"], a["r"], a["L_cap"], v(a["Lp"]), v(a["q"]), a["q_dt"],
                                   v(a["C_K"]), v(a["C_V"]), a["C_dt"], v(a["B_K"]), v(a["B_V"]), a["B_dt"],
                                   v(a["cos"]), v(a["sin"]), 0.0, a["S"], v(a["ws"]), a["ws_bytes"], v(a["out"]),
                                   a["out_dt"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(nb=0), ESHAPE), (dict(r=256), ESHAPE), (dict(cos=None), ENULL), (dict(sin=None), ENULL),
    (dict(C_dt=I8), EDTYPE), (dict(B_dt=F32), EDTYPE), (dict(out_dt=I8), EDTYPE),
    (dict(r=16), EUNSUP), (dict(r=48), EUNSUP), (dict(H=96), EUNSUP),
    (dict(cos=P + 4), EALIGN), (dict(C_V=P + 2), EALIGN), ({}, EWS), (dict(ws=None), EWS),
])
def test_rope_rejects(L, kw, want):
    assert rope(L, **kw) == want


def test_rope_tables_rejects(L):
    v = ctypes.c_void_p
    f = L.wsvd_rope_tables
    assert f(0, 128, 10000.0, v(P), v(P), None) == ESHAPE
    assert f(16, 127, 10000.0, v(P), v(P), None) == ESHAPE
    assert f(16, 128, 1.0, v(P), v(P), None) == ESHAPE
    assert f(16, 128, 10000.0, None, v(P), None) == ENULL
    assert f(16, 128, 10000.0, v(P), v(P + 4), None) == EALIGN


def svd(L, E=512, nh=4, H=128, r=32, W=P, A=P, B=P, sigma=P, sweeps=None, ws=P, ws_bytes=16):
    v = ctypes.c_void_p
    return L.wsvd_factorize_svd(E, nh, H, r, v(W) if W else None, v(A) if A else None, v(B) if B else None,
                                v(sigma) if sigma else None, v(sweeps) if sweeps else None, v(ws) if ws else None,
                                ws_bytes, None)


def test_factorize_svd_workspace_size(L):
    f = wsvd.factorize_svd_workspace_bytes
    for E, nh, H in [(4096, 32, 128), (100, 1, 64), (4096, 1, 128), (33, 700, 64)]:
        n = f(E, nh, H)
        chunks = n // (nh * H * H * 8)
        assert n == chunks * nh * H * H * 8 and 1 <= chunks <= max(1, (E + 63) // 64)
    assert f(0, 4, 128) == 0 and f(16, 4, 96) == 0


@pytest.mark.parametrize("kw,want", [
    (dict(E=0), ESHAPE), (dict(nh=0), ESHAPE), (dict(r=0), ESHAPE), (dict(r=129), ESHAPE),
    (dict(nh=70000), ESHAPE), (dict(H=96, r=32), EUNSUP), (dict(W=None), ENULL), (dict(A=None), ENULL),
    (dict(B=None), ENULL), (dict(sigma=None), ENULL), (dict(W=P + 4), EALIGN), (dict(sigma=P + 8), EALIGN),
    ({}, EWS), (dict(ws=None, ws_bytes=1 << 40), EWS), (dict(ws=P + 4, ws_bytes=1 << 40), EWS),
])
def test_factorize_svd_rejects(L, kw, want):
    assert svd(L, **kw) == want


@pytest.mark.parametrize("fn", ["wsvd_weighted_update_A", "wsvd_weighted_update_B"])
@pytest.mark.parametrize("args,want", [
    ((0, 4, 128, 32, P, P, P, P), ESHAPE), ((64, 4, 128, 0, P, P, P, P), ESHAPE),
    ((64, 4, 64, 128, P, P, P, P), ESHAPE), ((64, 4, 96, 32, P, P, P, P), EUNSUP),
    ((64, 4, 128, 40, P, P, P, P), EUNSUP), ((64, 4, 128, 32, None, P, P, P), ENULL),
    ((64, 4, 128, 32, P, None, P, P), ENULL), ((64, 4, 128, 32, P, P, None, P), ENULL),
    ((64, 4, 128, 32, P, P, P, None), ENULL), ((64, 4, 128, 32, P, P + 4, P, P), EALIGN),
    ((64, 4, 128, 32, P, P, P, P + 12), EALIGN),
])
def test_weighted_update_rejects(L, fn, args, want):
    v = ctypes.c_void_p
    conv = [a if i < 4 else (v(a) if a else None) for i, a in enumerate(args)]
    assert getattr(L, fn)(*conv, None) == want


def shared(L, nb=2, nh=4, H=128, R=1024, Lc=256, Lp=P, q=P, CK=P, CV=P, BK=P, BV=P, S=0, ws=P, wsb=16, out=P,
           out_dt=BF16):
    v = ctypes.c_void_p
    pp = lambda x: v(x) if x else None
    return L.wsvd_shared_decode_attn(nb, nh, H, R, Lc, pp(Lp), pp(q), pp(CK), pp(CV), pp(BK), pp(BV), 0.0, S, pp(ws),
                                     wsb, pp(out), out_dt, None)


def test_shared_workspace_size(L):
    f = wsvd.shared_decode_workspace_bytes
    for nb, nh, R, Lc, S in [(1, 32, 1024, 1088, 0), (16, 32, 2048, 4096, 3), (3, 5, 512, 100, 7)]:
        s = wsvd.decode_num_splits(nb, nh, Lc, S)
        assert f(nb, nh, R, Lc, S) >= nb * nh * R * 4 + nb * nh * s * (R + 1) * 4
    assert f(0, 32, 1024, 100, 0) == 0


@pytest.mark.parametrize("kw,want", [
    (dict(nb=0), ESHAPE), (dict(R=0), ESHAPE), (dict(S=-1), ESHAPE), (dict(S=300, Lc=256), ESHAPE),
    (dict(Lp=None), ENULL), (dict(CV=None), ENULL), (dict(BV=None), ENULL), (dict(out=None), ENULL),
    (dict(out_dt=I8), EDTYPE), (dict(out_dt=F16), EDTYPE), (dict(H=96), EUNSUP), (dict(R=768), EUNSUP),
    (dict(R=256), EUNSUP), (dict(q=P + 2), EALIGN), (dict(BK=P + 8), EALIGN), ({}, EWS), (dict(ws=None), EWS),
    (dict(ws=P + 16, wsb=1 << 40), EWS),
])
def test_shared_rejects(L, kw, want):
    assert shared(L, **kw) == want


def noalloc(L, **kw):
    a = dict(nb=1, nh=32, H=128, r=32, L_cap=1088, Lp=P, q=P, q_dt=BF16, C_K=P, C_V=P, C_dt=BF16, s_K=None,
             s_V=None, B_K=P, B_V=P, B_dt=BF16, scale=0.0, S=0, out=P, out_dt=BF16)
    a.update(kw)
    v = ctypes.c_void_p
    return L.wsvd_decode_attn_noalloc(a["nb"], a["nh"], a["H"], a["r"], a["L_cap"], v(a["Lp"]), v(a["q"]),
                                      a["q_dt"], v(a["C_K"]), v(a["C_V"]), a["C_dt"], v(a["s_K"]), v(a["s_V"]),
                                      v(a["B_K"]), v(a["B_V"]), a["B_dt"], a["scale"], a["S"], v(a["out"]),
                                      a["out_dt"], None)


# Every case is refused by the host checks, all of which run before the
# scratch is looked up (the lookup is the first HIP call).
@pytest.mark.parametrize("kw,want", [
    (dict(out=None), ENULL), (dict(q=None), ENULL), (dict(nb=0), ESHAPE), (dict(r=160), ESHAPE),
    (dict(H=96, r=32), EUNSUP), (dict(C_dt=F16), EDTYPE), (dict(q=P + 4), EALIGN),
    (dict(nb=65537, nh=1, L_cap=16), EWS),                      # more (b, h) pairs than the counter region holds
    (dict(L_cap=1 << 20, S=1100), EWS),                         # 32 x 1100 x 128 fp32 partials > 16 MiB
])
def test_decode_noalloc_rejects(L, kw, want):
    assert noalloc(L, **kw) == want


@pytest.mark.parametrize("mode,blocks,src,nbytes,sink,want", [
    (2, 160, P, 2560, P, ESHAPE), (0, 0, None, 0, P, ESHAPE), (0, 160, None, 0, None, ENULL),
    (1, 160, None, 2560, P, ENULL), (1, 160, P + 8, 2560, P, EALIGN), (1, 160, P, 2570, P, ESHAPE),
    (1, 160, P, 160 * 16 * 4097, P, ESHAPE), (1, 160, P, 0, P, ESHAPE),
])
def test_floor_probe_rejects(L, mode, blocks, src, nbytes, sink, want):
    v = ctypes.c_void_p
    assert L.wsvd_floor_probe(mode, blocks, v(src), nbytes, v(sink), None) == want
