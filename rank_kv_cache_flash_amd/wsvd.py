"""Python binding of libwsvd.so: torch tensors in, the same C calls out.

Argument marshalling only -- every step of the decode runs in the HIP
kernels behind include/wsvd.h.  Tensors must already live on the GPU;
there is no CPU path and a missing library raises at first use.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libwsvd.so")

F32, BF16, F16, I8 = 0, 1, 2, 3
_DT = {torch.float32: F32, torch.bfloat16: BF16, torch.float16: F16, torch.int8: I8}
_TORCH = {F32: torch.float32, BF16: torch.bfloat16, F16: torch.float16, I8: torch.int8}

_lib = None


class WsvdError(RuntimeError):
    def __init__(self, status: int, call: str):
        self.status = status
        super().__init__(f"{call} failed: {status_string(status)} ({status})")


def lib() -> ctypes.CDLL:
    """Load libwsvd.so once (after torch, so both share one HIP runtime)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m rank_kv_cache_flash_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    L.wsvd_decode_attn.argtypes = [i32, i32, i32, i32, i32, vp, vp, i32, vp, vp, i32, vp, vp, vp, vp, i32,
                                   f32, i32, vp, sz, vp, i32, vp]
    L.wsvd_decode_attn.restype = i32
    L.wsvd_decode_attn_noalloc.argtypes = [i32, i32, i32, i32, i32, vp, vp, i32, vp, vp, i32, vp, vp, vp, vp, i32,
                                           f32, i32, vp, i32, vp]
    L.wsvd_decode_attn_noalloc.restype = i32
    L.wsvd_dense_decode_attn.argtypes = [i32, i32, i32, i32, vp, vp, i32, vp, vp, i32, f32, i32, vp, sz, vp, i32, vp]
    L.wsvd_dense_decode_attn.restype = i32
    L.wsvd_combine_splits.argtypes = [i32, i32, i32, i32, vp, vp, vp, i32, vp]
    L.wsvd_combine_splits.restype = i32
    L.wsvd_append_latent.argtypes = [i32, i32, i32, i32, i32, vp, i32, vp, vp, i32, vp, vp, vp, i32, vp, vp,
                                     vp, sz, vp]
    L.wsvd_append_latent.restype = i32
    L.wsvd_append_latent_w8a8.argtypes = [i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, vp, vp,
                                          vp, sz, vp]
    L.wsvd_append_latent_w8a8.restype = i32
    L.wsvd_w8a8_quantize_activations.argtypes = [i32, i32, vp, i32, vp, vp, vp]
    L.wsvd_w8a8_quantize_activations.restype = i32
    L.wsvd_w8a8_prepare_factor.argtypes = [i32, i32, vp, i32, vp, vp, vp]
    L.wsvd_w8a8_prepare_factor.restype = i32
    L.wsvd_decode_attn_rope.argtypes = [i32, i32, i32, i32, i32, vp, vp, i32, vp, vp, i32, vp, vp, i32, vp, vp,
                                        f32, i32, vp, sz, vp, i32, vp]
    L.wsvd_decode_attn_rope.restype = i32
    L.wsvd_rope_tables.argtypes = [i32, i32, f32, vp, vp, vp]
    L.wsvd_rope_tables.restype = i32
    L.wsvd_decode_num_splits.argtypes = [i32, i32, i32, i32]
    L.wsvd_decode_num_splits.restype = i32
    L.wsvd_decode_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
    L.wsvd_decode_workspace_bytes.restype = sz
    L.wsvd_decode_lse_offset.argtypes = [i32, i32, i32, i32, i32]
    L.wsvd_decode_lse_offset.restype = sz
    L.wsvd_decode_opart_offset.argtypes = [i32, i32, i32, i32, i32]
    L.wsvd_decode_opart_offset.restype = sz
    L.wsvd_decode_counter_bytes.argtypes = [i32, i32]
    L.wsvd_decode_counter_bytes.restype = sz
    L.wsvd_append_counter_bytes.argtypes = [i32, i32, i32]
    L.wsvd_append_counter_bytes.restype = sz
    L.wsvd_append_workspace_bytes.argtypes = [i32, i32, i32, i32]
    L.wsvd_append_workspace_bytes.restype = sz
    L.wsvd_factorize_svd_workspace_bytes.argtypes = [i32, i32, i32]
    L.wsvd_factorize_svd_workspace_bytes.restype = sz
    L.wsvd_factorize_svd.argtypes = [i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, sz, vp]
    L.wsvd_factorize_svd.restype = i32
    L.wsvd_weighted_update_A.argtypes = [i32, i32, i32, i32, vp, vp, vp, vp, vp]
    L.wsvd_weighted_update_A.restype = i32
    L.wsvd_weighted_update_B.argtypes = [i32, i32, i32, i32, vp, vp, vp, vp, vp]
    L.wsvd_weighted_update_B.restype = i32
    L.wsvd_shared_decode_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
    L.wsvd_shared_decode_workspace_bytes.restype = sz
    L.wsvd_shared_decode_attn.argtypes = [i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, f32, i32, vp, sz, vp, i32,
                                          vp]
    L.wsvd_shared_decode_attn.restype = i32
    L.wsvd_floor_probe.argtypes = [i32, i32, vp, sz, vp, vp]
    L.wsvd_floor_probe.restype = i32
    L.wsvd_status_string.argtypes = [i32]
    L.wsvd_status_string.restype = ctypes.c_char_p
    L.wsvd_version.argtypes = []
    L.wsvd_version.restype = ctypes.c_char_p
    _lib = L
    return L


def status_string(status: int) -> str:
    return lib().wsvd_status_string(int(status)).decode()


def version() -> str:
    return lib().wsvd_version().decode()


def decode_num_splits(nb, nh, L_cap, n_splits=0) -> int:
    return int(lib().wsvd_decode_num_splits(nb, nh, L_cap, n_splits or 0))


def decode_workspace_bytes(nb, nh, H, L_cap, n_splits=0) -> int:
    return int(lib().wsvd_decode_workspace_bytes(nb, nh, H, L_cap, n_splits or 0))


def decode_lse_offset(nb, nh, H, L_cap, n_splits=0) -> int:
    return int(lib().wsvd_decode_lse_offset(nb, nh, H, L_cap, n_splits or 0))


def decode_opart_offset(nb, nh, H, L_cap, n_splits=0) -> int:
    return int(lib().wsvd_decode_opart_offset(nb, nh, H, L_cap, n_splits or 0))


def decode_counter_bytes(nb, nh) -> int:
    """Bytes of the merge-counter area at the start of a decode workspace."""
    return int(lib().wsvd_decode_counter_bytes(nb, nh))


def _zero_filled(t):
    """Mark a freshly zero-filled workspace: all of it is known to be zero."""
    t._wsvd_zero_bytes = t.numel() * t.element_size()
    return t


def _claim_counters(ws, counter_bytes, what, needs_zero=True):
    """The zero-counter rule, checked for workspaces this module zero-filled:
    a call that merges (needs_zero) needs its counter bytes still known to
    be zero.  Every call keeps its counter bytes as they were and may write
    anything past them, so afterwards only min(known, counter_bytes) bytes
    are known to be zero.  Workspaces from elsewhere carry no mark and are
    the caller's responsibility."""
    known = getattr(ws, "_wsvd_zero_bytes", None)
    if known is None:
        return
    if needs_zero and known < counter_bytes:
        raise ValueError(f"{what}: the workspace's first {counter_bytes} bytes (merge counters) must be zero, "
                         f"but an earlier call may have written partials past byte {known}; zero-fill it "
                         f"again or use a separate workspace")
    ws._wsvd_zero_bytes = min(known, counter_bytes)


def decode_workspace(nb, nh, H, L_cap, n_splits=0, device="cuda"):
    """A decode workspace, zero-filled once (its merge counters must start at zero)."""
    return _zero_filled(torch.zeros(decode_workspace_bytes(nb, nh, H, L_cap, n_splits), dtype=torch.uint8,
                                    device=device))


def append_workspace_bytes(nb, E, nh, r) -> int:
    return int(lib().wsvd_append_workspace_bytes(nb, E, nh, r))


def append_counter_bytes(nb, nh, r) -> int:
    return int(lib().wsvd_append_counter_bytes(nb, nh, r))


def _append_counter_claim(nb, E, nh, r):
    """Counter bytes an append call relies on (none when E is not split)."""
    return append_counter_bytes(nb, nh, r) if append_workspace_bytes(nb, E, nh, r) > 0 else 0


def append_workspace(nb, E, nh, r, device="cuda"):
    """Zero-filled append workspace (its tile counters must start at zero;
    every call leaves them zero again, so calls issued one after another
    on a stream can share one buffer)."""
    return _zero_filled(torch.zeros(max(append_workspace_bytes(nb, E, nh, r), 256), dtype=torch.uint8,
                                    device=device))


# ---------------------------------------------------------------------------
# argument checks: shapes and dtypes first (metadata only, so they also run
# without a GPU), then that every tensor is a contiguous GPU tensor
# ---------------------------------------------------------------------------
_ACT = (torch.float32, torch.bfloat16, torch.float16)
_CACHE = (torch.float32, torch.bfloat16, torch.int8)
_SCALE = (torch.float16, torch.int16)


def _need(t, name, shape, dtypes):
    if t is None:
        raise ValueError(f"{name} is required")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype not in dtypes:
        raise ValueError(f"{name} must be one of {[str(d) for d in dtypes]}, got {t.dtype}")


def _ndim(t, name, n):
    if t is None or t.dim() != n:
        raise ValueError(f"{name} must be a {n}-d tensor")


def _check_decode_args(q, C_K, C_V, B_K, B_V, L, s_K, s_V, out, *, cache_dtypes=_CACHE, factor_dtypes=_ACT):
    """Shapes and dtypes of a wsvd_decode_attn-style call; returns (nb, nh, H, L_cap, r)."""
    _ndim(q, "q", 3)
    _ndim(C_K, "C_K", 4)
    nb, nh, H = q.shape
    L_cap, r = C_K.shape[2], C_K.shape[3]
    _need(q, "q", (nb, nh, H), _ACT)
    _need(C_K, "C_K", (nb, nh, L_cap, r), cache_dtypes)
    _need(C_V, "C_V", (nb, nh, L_cap, r), (C_K.dtype,))
    _need(B_K, "B_K", (nh, r, H), factor_dtypes)
    _need(B_V, "B_V", (nh, r, H), (B_K.dtype,))
    _need(L, "L", (nb,), (torch.int32,))
    if C_K.dtype == torch.int8:
        _need(s_K, "s_K", (nb, nh, L_cap), _SCALE)
        _need(s_V, "s_V", (nb, nh, L_cap), _SCALE)
    elif s_K is not None or s_V is not None:
        raise ValueError("s_K / s_V are per-row scales of int8 caches only")
    if out is not None:
        _need(out, "out", (nb, nh, H), _ACT)
    return nb, nh, H, L_cap, r


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(t, name):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (there is no CPU path)")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check(st, call):
    if st != 0:
        raise WsvdError(st, call)


def decode_attn(q, C_K, C_V, B_K, B_V, L, *, s_K=None, s_V=None, softmax_scale=None, n_splits=None,
                out=None, out_dtype=None, workspace=None, partials_only=False, stream=None):
    """wsvd_decode_attn on torch tensors.

    q [nb, nh, H]; C_K / C_V [nb, nh, L_cap, r]; B_K / B_V [nh, r, H];
    L int32 [nb] (device); s_K / s_V fp16 [nb, nh, L_cap] for int8 caches.
    Returns out [nb, nh, H] (or None with partials_only) and the partial
    views (o_part [nb, nh, S, H], lse_part [nb, nh, S]) inside workspace;
    with an output and one split the kernel writes out directly and leaves
    those views unwritten.
    """
    nb, nh, H, L_cap, r = _check_decode_args(q, C_K, C_V, B_K, B_V, L, s_K, s_V, None if partials_only else out)
    for t, n in ((q, "q"), (C_K, "C_K"), (C_V, "C_V"), (B_K, "B_K"), (B_V, "B_V"), (L, "L"),
                 (s_K, "s_K"), (s_V, "s_V"), (out, "out"), (workspace, "workspace")):
        _dev(t, n)
    S = decode_num_splits(nb, nh, L_cap, n_splits or 0)
    if S <= 0:
        raise WsvdError(S, "wsvd_decode_num_splits")
    if workspace is None:
        workspace = decode_workspace(nb, nh, H, L_cap, n_splits or 0, device=q.device)
    if not partials_only and out is None:
        out = torch.empty((nb, nh, H), dtype=out_dtype or q.dtype, device=q.device)
    if partials_only:
        out = None
    _claim_counters(workspace, decode_counter_bytes(nb, nh), "wsvd_decode_attn", out is not None)
    if s_K is not None and s_K.dtype == torch.float16:
        s_K = s_K.view(torch.int16)
    if s_V is not None and s_V.dtype == torch.float16:
        s_V = s_V.view(torch.int16)
    st = lib().wsvd_decode_attn(
        nb, nh, H, r, L_cap, _ptr(L), _ptr(q), _DT[q.dtype], _ptr(C_K), _ptr(C_V), _DT[C_K.dtype],
        _ptr(s_K), _ptr(s_V), _ptr(B_K), _ptr(B_V), _DT[B_K.dtype],
        float(softmax_scale or 0.0), int(n_splits or 0), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _ptr(out), _DT[out.dtype] if out is not None else 0, _stream(stream))
    _check(st, "wsvd_decode_attn")
    return (out, *_partial_views(workspace, nb, nh, H, L_cap, n_splits, S))


def decode_attn_noalloc(q, C_K, C_V, B_K, B_V, L, *, s_K=None, s_V=None, softmax_scale=None, n_splits=None,
                        out=None, out_dtype=None, stream=None):
    """wsvd_decode_attn_noalloc: decode_attn with no workspace (the library's
    per-GPU static scratch holds the partials); returns out.  Calls that
    overlap on one GPU race on that scratch."""
    nb, nh, H, L_cap, r = _check_decode_args(q, C_K, C_V, B_K, B_V, L, s_K, s_V, out)
    for t, n in ((q, "q"), (C_K, "C_K"), (C_V, "C_V"), (B_K, "B_K"), (B_V, "B_V"), (L, "L"),
                 (s_K, "s_K"), (s_V, "s_V"), (out, "out")):
        _dev(t, n)
    if out is None:
        out = torch.empty((nb, nh, H), dtype=out_dtype or q.dtype, device=q.device)
    if s_K is not None and s_K.dtype == torch.float16:
        s_K = s_K.view(torch.int16)
    if s_V is not None and s_V.dtype == torch.float16:
        s_V = s_V.view(torch.int16)
    st = lib().wsvd_decode_attn_noalloc(
        nb, nh, H, r, L_cap, _ptr(L), _ptr(q), _DT[q.dtype], _ptr(C_K), _ptr(C_V), _DT[C_K.dtype],
        _ptr(s_K), _ptr(s_V), _ptr(B_K), _ptr(B_V), _DT[B_K.dtype], float(softmax_scale or 0.0), int(n_splits or 0),
        _ptr(out), _DT[out.dtype], _stream(stream))
    _check(st, "wsvd_decode_attn_noalloc")
    return out


def _partial_views(workspace, nb, nh, H, L_cap, n_splits, S):
    """(o_part [nb, nh, S, H], lse_part [nb, nh, S]) views inside a decode workspace."""
    o0 = decode_opart_offset(nb, nh, H, L_cap, n_splits or 0)
    off = decode_lse_offset(nb, nh, H, L_cap, n_splits or 0)
    wsb = workspace.view(torch.uint8).reshape(-1)
    o_part = wsb[o0: o0 + nb * nh * S * H * 4].view(torch.float32).view(nb, nh, S, H)
    lse_part = wsb[off: off + nb * nh * S * 4].view(torch.float32).view(nb, nh, S)
    return o_part, lse_part


def rope_tables(L_cap, H, base=10000.0, *, device="cuda", stream=None):
    """wsvd_rope_tables: (cos, sin) fp32 [L_cap, H/2] of angle t * base^(-2 i / H)."""
    c = torch.empty((L_cap, H // 2), dtype=torch.float32, device=device)
    s_ = torch.empty_like(c)
    _check(lib().wsvd_rope_tables(L_cap, H, float(base), _ptr(c), _ptr(s_), _stream(stream)), "wsvd_rope_tables")
    return c, s_


def _check_rope_args(q, C_K, C_V, B_K, B_V, L, rope_cos, rope_sin, out):
    nb, nh, H, L_cap, r = _check_decode_args(q, C_K, C_V, B_K, B_V, L, None, None, out,
                                             cache_dtypes=(torch.bfloat16,), factor_dtypes=(torch.bfloat16,))
    _need(rope_cos, "rope_cos", (L_cap, H // 2), (torch.float32,))
    _need(rope_sin, "rope_sin", (L_cap, H // 2), (torch.float32,))
    return nb, nh, H, L_cap, r


def _rope_args(q, C_K, C_V, B_K, B_V, L, rope_cos, rope_sin, softmax_scale, n_splits, workspace, out):
    nb, nh, H = q.shape
    L_cap, r = C_K.shape[2], C_K.shape[3]
    return (nb, nh, H, r, L_cap, _ptr(L), _ptr(q), _DT[q.dtype], _ptr(C_K), _ptr(C_V), _DT[C_K.dtype], _ptr(B_K),
            _ptr(B_V), _DT[B_K.dtype], _ptr(rope_cos), _ptr(rope_sin), float(softmax_scale or 0.0), int(n_splits or 0),
            _ptr(workspace), workspace.numel() * workspace.element_size(), _ptr(out),
            _DT[out.dtype] if out is not None else 0)


def decode_attn_rope(q, C_K, C_V, B_K, B_V, L, rope_cos, rope_sin, *, softmax_scale=None, n_splits=None, out=None,
                     out_dtype=None, workspace=None, partials_only=False, stream=None):
    """wsvd_decode_attn_rope: as decode_attn, with keys rotated to their positions
    (rope_cos / rope_sin fp32 [L_cap, H/2]); q is already rotated.  Returns
    (out, o_part, lse_part) like decode_attn."""
    nb, nh, H, L_cap, _ = _check_rope_args(q, C_K, C_V, B_K, B_V, L, rope_cos, rope_sin,
                                           None if partials_only else out)
    for t, n in ((q, "q"), (C_K, "C_K"), (C_V, "C_V"), (B_K, "B_K"), (B_V, "B_V"), (L, "L"),
                 (rope_cos, "rope_cos"), (rope_sin, "rope_sin"), (out, "out"), (workspace, "workspace")):
        _dev(t, n)
    S = decode_num_splits(nb, nh, L_cap, n_splits or 0)
    if S <= 0:
        raise WsvdError(S, "wsvd_decode_num_splits")
    if workspace is None:
        workspace = decode_workspace(nb, nh, H, L_cap, n_splits or 0, device=q.device)
    if not partials_only and out is None:
        out = torch.empty((nb, nh, H), dtype=out_dtype or q.dtype, device=q.device)
    if partials_only:
        out = None
    _claim_counters(workspace, decode_counter_bytes(nb, nh), "wsvd_decode_attn_rope", out is not None)
    st = lib().wsvd_decode_attn_rope(*_rope_args(q, C_K, C_V, B_K, B_V, L, rope_cos, rope_sin, softmax_scale,
                                                 n_splits, workspace, out), _stream(stream))
    _check(st, "wsvd_decode_attn_rope")
    return (out, *_partial_views(workspace, nb, nh, H, L_cap, n_splits, S))


class PreparedDecodeRope:
    """wsvd_decode_attn_rope with fixed buffers; __call__(stream) enqueues it."""

    def __init__(self, q, C_K, C_V, B_K, B_V, L, rope_cos, rope_sin, *, workspace, out=None, n_splits=None):
        nb, nh, _, _, _ = _check_rope_args(q, C_K, C_V, B_K, B_V, L, rope_cos, rope_sin, out)
        for t, n in ((q, "q"), (C_K, "C_K"), (C_V, "C_V"), (B_K, "B_K"), (B_V, "B_V"), (L, "L"),
                     (rope_cos, "rope_cos"), (rope_sin, "rope_sin"), (out, "out"), (workspace, "workspace")):
            _dev(t, n)
        _claim_counters(workspace, decode_counter_bytes(nb, nh), "wsvd_decode_attn_rope", out is not None)
        self._keep = (q, C_K, C_V, B_K, B_V, L, rope_cos, rope_sin, workspace, out)
        self._args = _rope_args(q, C_K, C_V, B_K, B_V, L, rope_cos, rope_sin, None, n_splits, workspace, out)
        self._fn = lib().wsvd_decode_attn_rope

    def __call__(self, stream=None):
        _check(self._fn(*self._args, _stream(stream)), "wsvd_decode_attn_rope")


def _check_dense_args(q, K, V, L, out):
    _ndim(q, "q", 3)
    _ndim(K, "K", 4)
    nb, nh, H = q.shape
    L_cap = K.shape[2]
    _need(q, "q", (nb, nh, H), _ACT)
    _need(K, "K", (nb, nh, L_cap, H), (torch.bfloat16,))
    _need(V, "V", (nb, nh, L_cap, H), (torch.bfloat16,))
    _need(L, "L", (nb,), (torch.int32,))
    if out is not None:
        _need(out, "out", (nb, nh, H), _ACT)
    return nb, nh, H, L_cap


def dense_decode_attn(q, K, V, L, *, softmax_scale=None, n_splits=None, out=None, out_dtype=None, workspace=None,
                      stream=None):
    """wsvd_dense_decode_attn (Flash-Decoding baseline): q [nb, nh, H]; K / V [nb, nh, L_cap, H] bf16."""
    nb, nh, H, L_cap = _check_dense_args(q, K, V, L, out)
    for t, n in ((q, "q"), (K, "K"), (V, "V"), (L, "L"), (out, "out"), (workspace, "workspace")):
        _dev(t, n)
    if workspace is None:
        workspace = decode_workspace(nb, nh, H, L_cap, n_splits or 0, device=q.device)
    if out is None:
        out = torch.empty((nb, nh, H), dtype=out_dtype or q.dtype, device=q.device)
    _claim_counters(workspace, decode_counter_bytes(nb, nh), "wsvd_dense_decode_attn")
    st = lib().wsvd_dense_decode_attn(nb, nh, H, L_cap, _ptr(L), _ptr(q), _DT[q.dtype], _ptr(K), _ptr(V),
                                      _DT[K.dtype], float(softmax_scale or 0.0), int(n_splits or 0), _ptr(workspace),
                                      workspace.numel() * workspace.element_size(), _ptr(out), _DT[out.dtype],
                                      _stream(stream))
    _check(st, "wsvd_dense_decode_attn")
    return out


class PreparedDense:
    """wsvd_dense_decode_attn with fixed buffers; __call__(stream) enqueues it."""

    def __init__(self, q, K, V, L, *, workspace, out, n_splits=None):
        nb, nh, H, _ = _check_dense_args(q, K, V, L, out)
        for t, n in ((q, "q"), (K, "K"), (V, "V"), (L, "L"), (out, "out"), (workspace, "workspace")):
            _dev(t, n)
        _claim_counters(workspace, decode_counter_bytes(nb, nh), "wsvd_dense_decode_attn")
        self._keep = (q, K, V, L, workspace, out)
        self._args = (nb, nh, H, K.shape[2], _ptr(L), _ptr(q), _DT[q.dtype], _ptr(K), _ptr(V), _DT[K.dtype], 0.0,
                      int(n_splits or 0), _ptr(workspace), workspace.numel() * workspace.element_size(), _ptr(out),
                      _DT[out.dtype])
        self._fn = lib().wsvd_dense_decode_attn

    def __call__(self, stream=None):
        _check(self._fn(*self._args, _stream(stream)), "wsvd_dense_decode_attn")


def combine_splits(o_part, lse_part, *, out=None, out_dtype=torch.float32, stream=None):
    """wsvd_combine_splits: o_part [nb, nh, S, H] fp32, lse_part [nb, nh, S] fp32."""
    _ndim(o_part, "o_part", 4)
    nb, nh, S, H = o_part.shape
    _need(o_part, "o_part", (nb, nh, S, H), (torch.float32,))
    _need(lse_part, "lse_part", (nb, nh, S), (torch.float32,))
    if out is not None:
        _need(out, "out", (nb, nh, H), _ACT)
    _dev(o_part, "o_part"); _dev(lse_part, "lse_part"); _dev(out, "out")
    if out is None:
        out = torch.empty((nb, nh, H), dtype=out_dtype, device=o_part.device)
    st = lib().wsvd_combine_splits(nb, nh, H, S, _ptr(o_part), _ptr(lse_part), _ptr(out), _DT[out.dtype],
                                   _stream(stream))
    _check(st, "wsvd_combine_splits")
    return out


def _check_caches(nb, C_K, C_V, s_K, s_V):
    _ndim(C_K, "C_K", 4)
    if C_K.shape[0] != nb:
        raise ValueError(f"C_K must hold {nb} sequences, got {C_K.shape[0]}")
    _, nh, L_cap, r = C_K.shape
    _need(C_K, "C_K", (nb, nh, L_cap, r), _CACHE)
    _need(C_V, "C_V", (nb, nh, L_cap, r), (C_K.dtype,))
    if C_K.dtype == torch.int8:
        _need(s_K, "s_K", (nb, nh, L_cap), _SCALE)
        _need(s_V, "s_V", (nb, nh, L_cap), _SCALE)
    elif s_K is not None or s_V is not None:
        raise ValueError("s_K / s_V are per-row scales of int8 caches only")
    return nh, L_cap, r


def _check_append_args(x, A_K, A_V, pos, C_K, C_V, s_K, s_V):
    _ndim(x, "x", 2)
    nb, E = x.shape
    nh, L_cap, r = _check_caches(nb, C_K, C_V, s_K, s_V)
    _need(x, "x", (nb, E), (torch.bfloat16,))
    _need(A_K, "A_K", (E, nh * r), (torch.bfloat16,))
    _need(A_V, "A_V", (E, nh * r), (torch.bfloat16,))
    _need(pos, "pos", (nb,), (torch.int32,))
    return nb, E, nh, L_cap, r


def append_latent(x, A_K, A_V, pos, C_K, C_V, *, s_K=None, s_V=None, workspace=None, stream=None):
    """wsvd_append_latent: x [nb, E] bf16, A_K / A_V [E, nh*r] bf16, pos int32 [nb],
    caches [nb, nh, L_cap, r] (bf16 / f32, or int8 with fp16 row scales
    s_K / s_V [nb, nh, L_cap]) written in place at row pos[b]."""
    nb, E, nh, L_cap, r = _check_append_args(x, A_K, A_V, pos, C_K, C_V, s_K, s_V)
    for t, n in ((x, "x"), (A_K, "A_K"), (A_V, "A_V"), (pos, "pos"), (C_K, "C_K"), (C_V, "C_V"),
                 (s_K, "s_K"), (s_V, "s_V"), (workspace, "workspace")):
        _dev(t, n)
    if workspace is None:
        workspace = append_workspace(nb, E, nh, r, device=x.device)
    _claim_counters(workspace, _append_counter_claim(nb, E, nh, r), "wsvd_append_latent")
    st = lib().wsvd_append_latent(nb, E, nh, r, L_cap, _ptr(x), _DT[x.dtype], _ptr(A_K), _ptr(A_V), _DT[A_K.dtype],
                                  _ptr(pos), _ptr(C_K), _ptr(C_V), _DT[C_K.dtype], _ptr(s_K), _ptr(s_V),
                                  _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "wsvd_append_latent")
    return C_K, C_V


def w8a8_prepare_factor(A, *, stream=None):
    """wsvd_w8a8_prepare_factor: A [E, N] -> (AqT int8 [N, E], sA float32 [N])."""
    _ndim(A, "A", 2)
    E, N = A.shape
    _need(A, "A", (E, N), _ACT)
    _dev(A, "A")
    AqT = torch.empty((N, E), dtype=torch.int8, device=A.device)
    sA = torch.empty((N,), dtype=torch.float32, device=A.device)
    _check(lib().wsvd_w8a8_prepare_factor(E, N, _ptr(A), _DT[A.dtype], _ptr(AqT), _ptr(sA), _stream(stream)),
           "wsvd_w8a8_prepare_factor")
    return AqT, sA


def w8a8_quantize_activations(x, *, xq=None, sx=None, stream=None):
    """wsvd_w8a8_quantize_activations: x [nb, E] -> (xq int8 [nb, E], sx float32 [nb])."""
    _ndim(x, "x", 2)
    nb, E = x.shape
    _need(x, "x", (nb, E), _ACT)
    if xq is not None:
        _need(xq, "xq", (nb, E), (torch.int8,))
    if sx is not None:
        _need(sx, "sx", (nb,), (torch.float32,))
    _dev(x, "x")
    xq = torch.empty((nb, E), dtype=torch.int8, device=x.device) if xq is None else xq
    sx = torch.empty((nb,), dtype=torch.float32, device=x.device) if sx is None else sx
    _dev(xq, "xq")
    _dev(sx, "sx")
    _check(lib().wsvd_w8a8_quantize_activations(nb, E, _ptr(x), _DT[x.dtype], _ptr(xq), _ptr(sx), _stream(stream)),
           "wsvd_w8a8_quantize_activations")
    return xq, sx


def append_latent_w8a8(xq, sx, AqT_K, sA_K, AqT_V, sA_V, pos, C_K, C_V, *, s_K=None, s_V=None, workspace=None,
                       stream=None):
    """wsvd_append_latent_w8a8: int8 token codes + scales and int8 transposed factor codes + scales;
    caches [nb, nh, L_cap, r] written in place at row pos[b]."""
    _ndim(xq, "xq", 2)
    nb, E = xq.shape
    nh, L_cap, r = _check_caches(nb, C_K, C_V, s_K, s_V)
    _need(xq, "xq", (nb, E), (torch.int8,))
    _need(sx, "sx", (nb,), (torch.float32,))
    for t, n in ((AqT_K, "AqT_K"), (AqT_V, "AqT_V")):
        _need(t, n, (nh * r, E), (torch.int8,))
    for t, n in ((sA_K, "sA_K"), (sA_V, "sA_V")):
        _need(t, n, (nh * r,), (torch.float32,))
    _need(pos, "pos", (nb,), (torch.int32,))
    for t, n in ((xq, "xq"), (sx, "sx"), (AqT_K, "AqT_K"), (sA_K, "sA_K"), (AqT_V, "AqT_V"), (sA_V, "sA_V"),
                 (pos, "pos"), (C_K, "C_K"), (C_V, "C_V"), (s_K, "s_K"), (s_V, "s_V"), (workspace, "workspace")):
        _dev(t, n)
    if workspace is None:
        workspace = append_workspace(nb, E, nh, r, device=xq.device)
    _claim_counters(workspace, _append_counter_claim(nb, E, nh, r), "wsvd_append_latent_w8a8")
    st = lib().wsvd_append_latent_w8a8(nb, E, nh, r, L_cap, _ptr(xq), _ptr(sx), _ptr(AqT_K), _ptr(AqT_V),
                                       _ptr(sA_K), _ptr(sA_V), _ptr(pos), _ptr(C_K), _ptr(C_V), _DT[C_K.dtype],
                                       _ptr(s_K), _ptr(s_V), _ptr(workspace),
                                       workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "wsvd_append_latent_w8a8")
    return C_K, C_V


# ---------------------------------------------------------------------------
# host arrays (storage dtypes from rank_kv_cache_flash_amd.inputs) -> device
# ---------------------------------------------------------------------------
def _f32(t, name):
    _dev(t, name)
    if t.dtype != torch.float32:
        raise ValueError(f"{name} must be float32")


def factorize_svd_workspace_bytes(E, nh, H) -> int:
    return int(lib().wsvd_factorize_svd_workspace_bytes(E, nh, H))


def factorize_svd(W, nh, r, *, workspace=None, stream=None):
    """wsvd_factorize_svd: W fp32 [E, nh*H] -> (A [E, nh*r], B [nh, r, H],
    sigma [nh, H], sweeps int32 [nh]), the per-head rank-r truncated SVD."""
    _ndim(W, "W", 2)
    E, NH = W.shape
    H = NH // nh
    if NH != nh * H:
        raise ValueError(f"W [{E}, {NH}] must hold {nh} column blocks")
    _f32(W, "W")
    dev = W.device
    A = torch.empty((E, nh * r), dtype=torch.float32, device=dev)
    B = torch.empty((nh, r, H), dtype=torch.float32, device=dev)
    sigma = torch.empty((nh, H), dtype=torch.float32, device=dev)
    sweeps = torch.empty((nh,), dtype=torch.int32, device=dev)
    if workspace is None:
        workspace = torch.empty(max(factorize_svd_workspace_bytes(E, nh, H), 256), dtype=torch.uint8, device=dev)
    _check(lib().wsvd_factorize_svd(E, nh, H, r, _ptr(W), _ptr(A), _ptr(B), _ptr(sigma), _ptr(sweeps),
                                    _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)),
           "wsvd_factorize_svd")
    return A, B, sigma, sweeps


def weighted_update_A(W, F, B, *, out=None, stream=None):
    """wsvd_weighted_update_A: rows of A [E, nh*r] minimising the F-weighted
    error against W for the given B [nh, r, H]."""
    _ndim(W, "W", 2)
    _ndim(B, "B", 3)
    nh, r, H = B.shape
    E = W.shape[0]
    _need(W, "W", (E, nh * H), (torch.float32,))
    _need(F, "F", (E, nh * H), (torch.float32,))
    if out is not None:
        _need(out, "out", (E, nh * r), (torch.float32,))
    for t, n in ((W, "W"), (F, "F"), (B, "B")):
        _f32(t, n)
    A = torch.empty((E, nh * r), dtype=torch.float32, device=W.device) if out is None else out
    _f32(A, "out")
    _check(lib().wsvd_weighted_update_A(E, nh, H, r, _ptr(W), _ptr(F), _ptr(B), _ptr(A), _stream(stream)),
           "wsvd_weighted_update_A")
    return A


def weighted_update_B(W, F, A, nh, *, out=None, stream=None):
    """wsvd_weighted_update_B: columns of B [nh, r, H] minimising the
    F-weighted error against W for the given A [E, nh*r]."""
    _ndim(W, "W", 2)
    _ndim(A, "A", 2)
    E, NH = W.shape
    H = NH // nh
    r = A.shape[1] // nh
    if NH != nh * H or A.shape[1] != nh * r:
        raise ValueError(f"W [{E}, {NH}] and A {tuple(A.shape)} must both hold {nh} column blocks")
    _need(F, "F", (E, NH), (torch.float32,))
    _need(A, "A", (E, nh * r), (torch.float32,))
    if out is not None:
        _need(out, "out", (nh, r, H), (torch.float32,))
    for t, n in ((W, "W"), (F, "F"), (A, "A")):
        _f32(t, n)
    B = torch.empty((nh, r, H), dtype=torch.float32, device=W.device) if out is None else out
    _f32(B, "out")
    _check(lib().wsvd_weighted_update_B(E, nh, H, r, _ptr(W), _ptr(F), _ptr(A), _ptr(B), _stream(stream)),
           "wsvd_weighted_update_B")
    return B


def shared_decode_workspace_bytes(nb, nh, R, L_cap, n_splits=0) -> int:
    return int(lib().wsvd_shared_decode_workspace_bytes(nb, nh, R, L_cap, n_splits))


def shared_decode_attn(q, C_K, C_V, B_K, B_V, L, *, softmax_scale=None, n_splits=None, out=None, out_dtype=None,
                       workspace=None, stream=None):
    """wsvd_shared_decode_attn: q [nb, nh, H]; C_K / C_V [nb, L_cap, R] and
    B_K / B_V [R, nh*H], all bfloat16; L int32 [nb]."""
    _ndim(q, "q", 3)
    _ndim(C_K, "C_K", 3)
    nb, nh, H = q.shape
    L_cap, R = C_K.shape[1], C_K.shape[2]
    bf = (torch.bfloat16,)
    _need(q, "q", (nb, nh, H), bf)
    _need(C_K, "C_K", (nb, L_cap, R), bf)
    _need(C_V, "C_V", (nb, L_cap, R), bf)
    _need(B_K, "B_K", (R, nh * H), bf)
    _need(B_V, "B_V", (R, nh * H), bf)
    _need(L, "L", (nb,), (torch.int32,))
    if out is not None:
        _need(out, "out", (nb, nh, H), (torch.float32, torch.bfloat16))
    for t, n in ((q, "q"), (C_K, "C_K"), (C_V, "C_V"), (B_K, "B_K"), (B_V, "B_V"), (L, "L"), (out, "out"),
                 (workspace, "workspace")):
        _dev(t, n)
    if workspace is None:
        workspace = torch.empty(max(shared_decode_workspace_bytes(nb, nh, R, L_cap, n_splits or 0), 256),
                                dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty((nb, nh, H), dtype=out_dtype or q.dtype, device=q.device)
    st = lib().wsvd_shared_decode_attn(nb, nh, H, R, L_cap, _ptr(L), _ptr(q), _ptr(C_K), _ptr(C_V), _ptr(B_K),
                                       _ptr(B_V), float(softmax_scale or 0.0), int(n_splits or 0), _ptr(workspace),
                                       workspace.numel() * workspace.element_size(), _ptr(out), _DT[out.dtype],
                                       _stream(stream))
    _check(st, "wsvd_shared_decode_attn")
    return out


def floor_probe(mode, blocks, sink, src=None, stream=None):
    """wsvd_floor_probe: mode 0 an empty launch of `blocks` x 256 threads,
    mode 1 a stream of all of src (uint8, contiguous) over the same grid;
    sink float32 [blocks]."""
    if sink is None or sink.dtype != torch.float32 or sink.numel() < blocks:
        raise ValueError(f"sink must be float32 with at least {blocks} elements")
    if src is not None and src.dim() != 1:
        raise ValueError("src must be a 1-d byte tensor")
    _dev(sink, "sink")
    _dev(src, "src")
    nbytes = 0 if src is None else src.numel() * src.element_size()
    _check(lib().wsvd_floor_probe(int(mode), int(blocks), _ptr(src), nbytes, _ptr(sink), _stream(stream)),
           "wsvd_floor_probe")


def shared_device_inputs(inp, device="cuda"):
    """SharedInputs (numpy, bf16 bit patterns) -> dict of GPU tensors."""
    return {"q": to_device(inp.q, inp.dt, device), "C_K": to_device(inp.C_K, inp.dt, device),
            "C_V": to_device(inp.C_V, inp.dt, device), "B_K": to_device(inp.B_K, inp.dt, device),
            "B_V": to_device(inp.B_V, inp.dt, device),
            "L": to_device(inp.L, "i32", device)}


def to_device(arr, dt: str, device="cuda"):
    """NumPy array in a storage dtype ('f32', 'bf16' bits, 'f16', 'i8', int32) -> GPU tensor."""
    import numpy as np
    if dt == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    elif dt == "f16":
        t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float16))
    elif dt == "f32":
        t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32))
    elif dt == "i8":
        t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.int8))
    elif dt == "i32":
        t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.int32))
    else:
        raise ValueError(dt)
    return t.to(device)


def device_inputs(inp, device="cuda"):
    """All tensors of a DecodeInputs on the GPU, keyed like the binding's arguments."""
    d = dict(
        q=to_device(inp.q, inp.q_dt, device),
        C_K=to_device(inp.C_K, inp.C_dt, device),
        C_V=to_device(inp.C_V, inp.C_dt, device),
        B_K=to_device(inp.B_K, inp.B_dt, device),
        B_V=to_device(inp.B_V, inp.B_dt, device),
        L=to_device(inp.L, "i32", device),
    )
    if inp.s_K is not None:
        d["s_K"] = to_device(inp.s_K, "f16", device)
        d["s_V"] = to_device(inp.s_V, "f16", device)
    if inp.x is not None:
        d["x"] = to_device(inp.x, inp.x_dt, device)
        d["A_K"] = to_device(inp.A_K, inp.A_dt, device)
        d["A_V"] = to_device(inp.A_V, inp.A_dt, device)
        d["pos"] = to_device(inp.pos, "i32", device)
    return d


# ---------------------------------------------------------------------------
# prepared calls: the ctypes argument tuple is built once, so issuing a step
# costs one foreign call (used for launch-rate-sensitive timing and graphs)
# ---------------------------------------------------------------------------
class PreparedDecode:
    """wsvd_decode_attn with fixed buffers; __call__(stream) enqueues it."""

    def __init__(self, q, C_K, C_V, B_K, B_V, L, *, s_K=None, s_V=None, workspace, out=None,
                 softmax_scale=None, n_splits=None):
        nb, nh, H, L_cap, r = _check_decode_args(q, C_K, C_V, B_K, B_V, L, s_K, s_V, out)
        for t, n in ((q, "q"), (C_K, "C_K"), (C_V, "C_V"), (B_K, "B_K"), (B_V, "B_V"), (L, "L"),
                     (s_K, "s_K"), (s_V, "s_V"), (out, "out"), (workspace, "workspace")):
            _dev(t, n)
        _claim_counters(workspace, decode_counter_bytes(nb, nh), "wsvd_decode_attn", out is not None)
        self.S = decode_num_splits(nb, nh, L_cap, n_splits or 0)
        self._keep = (q, C_K, C_V, B_K, B_V, L, s_K, s_V, workspace, out)
        if s_K is not None and s_K.dtype == torch.float16:
            s_K = s_K.view(torch.int16)
        if s_V is not None and s_V.dtype == torch.float16:
            s_V = s_V.view(torch.int16)
        self._args = (nb, nh, H, r, L_cap, _ptr(L), _ptr(q), _DT[q.dtype], _ptr(C_K), _ptr(C_V), _DT[C_K.dtype],
                      _ptr(s_K), _ptr(s_V), _ptr(B_K), _ptr(B_V), _DT[B_K.dtype], float(softmax_scale or 0.0),
                      int(n_splits or 0), _ptr(workspace), workspace.numel() * workspace.element_size(),
                      _ptr(out), _DT[out.dtype] if out is not None else 0)
        self._fn = lib().wsvd_decode_attn

    def __call__(self, stream=None):
        _check(self._fn(*self._args, _stream(stream)), "wsvd_decode_attn")


class PreparedAppend:
    """wsvd_append_latent with fixed buffers; __call__(stream) enqueues it."""

    def __init__(self, x, A_K, A_V, pos, C_K, C_V, *, workspace, s_K=None, s_V=None):
        nb, E, nh, L_cap, r = _check_append_args(x, A_K, A_V, pos, C_K, C_V, s_K, s_V)
        for t, n in ((x, "x"), (A_K, "A_K"), (A_V, "A_V"), (pos, "pos"), (C_K, "C_K"), (C_V, "C_V"),
                     (s_K, "s_K"), (s_V, "s_V"), (workspace, "workspace")):
            _dev(t, n)
        _claim_counters(workspace, _append_counter_claim(nb, E, nh, r), "wsvd_append_latent")
        self._keep = (x, A_K, A_V, pos, C_K, C_V, s_K, s_V, workspace)
        self._args = (nb, E, nh, r, L_cap, _ptr(x), _DT[x.dtype], _ptr(A_K), _ptr(A_V), _DT[A_K.dtype], _ptr(pos),
                      _ptr(C_K), _ptr(C_V), _DT[C_K.dtype], _ptr(s_K), _ptr(s_V), _ptr(workspace),
                      workspace.numel() * workspace.element_size())
        self._fn = lib().wsvd_append_latent

    def __call__(self, stream=None):
        _check(self._fn(*self._args, _stream(stream)), "wsvd_append_latent")
