#!/usr/bin/env python3
"""Benchmark of the WSVD low-rank decode step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 5] [--also 2,3,4]

A step is one pass of the whole hot path over one batch: the append of the
new token's latents (x . A_Kh, x . A_Vh into row L[b] - 1 of every head's
caches) when the workload has one, then the split decode and the split
merge.  The headline workload is the full step (workload 5, the largest).
Inputs are resident in HBM before timing starts.

Timing: the steps are captured once into a HIP graph holding K steps (at
least one per input copy, and enough copies that one replay reads >= 1 GiB
of distinct inputs, so every step reads cold HBM rather than the 256 MB
Infinity Cache).  After W eager warm-up steps, the graph is replayed untimed
for >= 200 ms (the GPU's clocks ramp up under sustained load); then each
timed region is one or more back-to-back replays (>= 1 ms) between events on
the replay stream, bracketed by device synchronisation; the median over five
regions is reported with every region's figure.

Prints ONE JSON line.  `value` is achieved GB/s = algorithmic bytes per step
/ time per step (higher is better); `ms_per_step` gives the time.  The
`roofline` object covers the dominant kernel (the split decode), timed the
same way in its own graph of back-to-back launches; `cpu_baseline` is the
fp64 oracle timed on the host on a bounded sample; `per_config` repeats the
whole measurement (with its own roofline and oracle baseline) on the other
workloads.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "fused low-rank decode attn: µs/step and achieved HBM GB/s (% of peak), 1 GPU"
COLD_BYTES = 1 << 30      # rotate input copies until >= 1 GiB is touched
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_traffic.json")
KERNEL_SOURCES = ("decode.hip", "decode_bf16_r32.hip", "wsvd_common.hpp", "split_merge.hpp", "abi.hip")


def kernel_src_hash() -> str:
    """Hash of the split kernel's code and of the host code that picks its
    launch shape (the split rule in abi.hip): the sources with comments and
    blank space removed, so that the counter summary stays valid across
    edits of comments only."""
    import re
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "rank_kv_cache_flash_amd", "csrc", f), encoding="utf-8") as fh:
            src = fh.read()
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
        src = re.sub(r"//[^\n]*", " ", src)
        h.update(" ".join(src.split()).encode())
    from rank_kv_cache_flash_amd.build import SOURCE_FLAGS      # per-file compiler options change the code too
    for f in KERNEL_SOURCES:
        h.update(" ".join(SOURCE_FLAGS.get(f, [])).encode())
    return h.hexdigest()[:16]


# ---------------------------------------------------------------------------
# workload on the device
# ---------------------------------------------------------------------------
class Workload:
    def __init__(self, cfg, copies=None, n_splits=None):
        import torch
        from rank_kv_cache_flash_amd import wsvd

        self.cfg = cfg
        t0 = time.time()
        self.inp = cfg.make()
        self.gen_s = time.time() - t0
        self.L = self.inp.L.copy()
        self.step_bytes = cfg.step_bytes(self.L)
        self.decode_bytes = cfg.decode_bytes(self.L)
        # bytes the split-decode kernel itself must read (out is written by the merge)
        sa = {"f32": 4, "bf16": 2, "f16": 2}[cfg.act_dt]
        self.decode_kernel_bytes = self.decode_bytes - cfg.nb * cfg.nh * cfg.H * sa
        if copies is None:
            copies = 1 if cfg.has_append else max(1, min(256, math.ceil(COLD_BYTES / self.decode_bytes)))
        self.copies = copies
        base = wsvd.device_inputs(self.inp)
        nb, nh, H = self.inp.q.shape
        self.sets = [base] + [{k: v.clone() for k, v in base.items()} for _ in range(copies - 1)]
        need = wsvd.decode_workspace_bytes(nb, nh, H, cfg.L_cap, n_splits or 0)
        self.ws = wsvd.decode_workspace(nb, nh, H, cfg.L_cap, n_splits or 0)       # counters start at zero
        self.ws_dec = wsvd.decode_workspace(nb, nh, H, cfg.L_cap, n_splits or 0)
        self.out = torch.empty((nb, nh, H), dtype=self.sets[0]["q"].dtype, device="cuda")
        self.S = wsvd.decode_num_splits(nb, nh, cfg.L_cap, n_splits or 0)
        self.full = []
        self.dec_only = []
        for d in self.sets:
            kw = dict(s_K=d.get("s_K"), s_V=d.get("s_V"), n_splits=n_splits)
            steps = []
            if cfg.has_append:
                aw = wsvd.append_workspace(nb, cfg.E, nh, cfg.r)
                d["_aws"] = aw
                steps.append(wsvd.PreparedAppend(d["x"], d["A_K"], d["A_V"], d["pos"], d["C_K"], d["C_V"],
                                                 workspace=aw))
            steps.append(wsvd.PreparedDecode(d["q"], d["C_K"], d["C_V"], d["B_K"], d["B_V"], d["L"],
                                             workspace=self.ws, out=self.out, **kw))
            self.full.append(steps)
            self.dec_only.append(wsvd.PreparedDecode(d["q"], d["C_K"], d["C_V"], d["B_K"], d["B_V"], d["L"],
                                                     workspace=self.ws_dec, out=None, **kw))
        torch.cuda.synchronize()

    def step(self, i):
        for call in self.full[i % self.copies]:
            call()

    def decode_only(self, i):
        self.dec_only[i % self.copies]()


MIN_REGION_S = 1e-3      # every timed region lasts at least this long
REGIONS = 5              # timed regions per measurement; the median is reported
WARM_S = 0.2             # untimed replays first, until the graph has run this long


def graph_timing(fn, steps, warmup, copies=1, min_region_s=MIN_REGION_S, regions=REGIONS):
    """Seconds per call of fn(i), from a HIP graph replayed on the current stream.

    The graph holds n calls, n = `steps` rounded up to a multiple of
    `copies`, so one replay touches every input copy (callers size `copies`
    so that is >= 1 GiB) whatever `steps` is.  After `warmup` eager calls and
    untimed replays for at least WARM_S of GPU time (the clocks of a
    compute-heavier kernel ramp up over tens of ms of sustained load: the
    rotary-key decode's first replays run 20 % slower than its steady state,
    while the memory-bound split kernel is flat), each timed region is k
    back-to-back replays between two events on the replay stream (k chosen so
    a region lasts >= min_region_s), bracketed by device synchronisation;
    the median over `regions` regions is returned with every region's
    figure."""
    import torch
    n = max(1, -(-max(steps, copies) // copies) * copies)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for i in range(warmup):
            fn(i)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(n):
            fn(i)
    g.replay()
    torch.cuda.synchronize()
    t_warm = time.time() + WARM_S
    while time.time() < t_warm:
        g.replay()
        torch.cuda.synchronize()

    def region(k):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(k):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3

    k = max(1, math.ceil(min_region_s / max(region(1), 1e-9)))
    per = [region(k) / (k * n) for _ in range(regions)]
    del g
    return {"s_per_call": statistics.median(per), "regions_s_per_call": per, "graph_calls": n,
            "replays_per_region": k, "regions": regions}


def graph_time(fn, steps, warmup, copies=1):
    """Median seconds per call (graph_timing)."""
    return graph_timing(fn, steps, warmup, copies)["s_per_call"]


def eager_time(fn, n, warmup):
    import torch
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(n):
        fn(i)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e-3 / n


def load_traffic(workload_name, launches_bytes):
    """HBM bytes per decode launch from the committed counter summary, if it
    was taken on the current kernel source; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    rec = t.get(workload_name)
    if not rec or rec.get("kernel_src_sha256_16") != kernel_src_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


# ---------------------------------------------------------------------------
# append alone: bf16 operands vs the W8A8 path (rotate + quantise x, int8 product)
# ---------------------------------------------------------------------------
def append_variants(cfg, steps, warmup=10, seed=0):
    """Time the append of one step alone at cfg's shapes (bf16 caches), with
    bf16 x and A and with the W8A8 path (wsvd_w8a8_quantize_activations +
    wsvd_append_latent_w8a8 on offline-prepared int8 factors).  Random GPU
    inputs (timing only; parity is in the tests), rotating over copies of the
    factors so A is read from HBM, graph replay."""
    import torch
    from rank_kv_cache_flash_amd import wsvd

    nb, E, nh, r, L_cap = cfg.nb, cfg.E, cfg.nh, cfg.r, cfg.L_cap
    N = nh * r
    g = torch.Generator(device="cuda").manual_seed(seed)
    bf = torch.bfloat16
    x = (torch.randn(nb, E, generator=g, device="cuda") * E ** -0.5).to(bf)
    pos = torch.randint(0, L_cap, (nb,), generator=g, device="cuda", dtype=torch.int32)
    C_K = torch.zeros(nb, nh, L_cap, r, dtype=bf, device="cuda")
    C_V = torch.zeros_like(C_K)
    ws = wsvd.append_workspace(nb, E, nh, r)
    ncopy = 8
    bf_calls, w8_facs = [], []
    for _ in range(ncopy):
        AK = (torch.randn(E, N, generator=g, device="cuda") * r ** -0.5).to(bf)
        AV = (torch.randn(E, N, generator=g, device="cuda") * r ** -0.5).to(bf)
        bf_calls.append(wsvd.PreparedAppend(x, AK, AV, pos, C_K, C_V, workspace=ws))
        w8_facs.append((*wsvd.w8a8_prepare_factor(AK), *wsvd.w8a8_prepare_factor(AV)))
    xq = torch.empty(nb, E, dtype=torch.int8, device="cuda")
    sx = torch.empty(nb, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    t_bf = graph_time(lambda i: bf_calls[i % ncopy](torch.cuda.current_stream()), steps, warmup, ncopy)

    def w8_step(i):
        AKq, sAK, AVq, sAV = w8_facs[i % ncopy]
        wsvd.w8a8_quantize_activations(x, xq=xq, sx=sx)
        wsvd.append_latent_w8a8(xq, sx, AKq, sAK, AVq, sAV, pos, C_K, C_V, workspace=ws)

    t_w8 = graph_time(w8_step, steps, warmup, ncopy)
    t_q = graph_time(lambda i: wsvd.w8a8_quantize_activations(x, xq=xq, sx=sx), steps, warmup)
    b_bf = 2 * E * N * 2 + nb * E * 2 + nb * 2 * N * 2
    b_w8 = 2 * E * N + 2 * N * 4 + nb * E * (2 + 1) + nb * 4 + nb * 2 * N * 2
    del bf_calls, w8_facs
    torch.cuda.empty_cache()
    return {"shape": f"x[{nb},{E}] -> {nh} heads x r {r}, bf16 caches",
            "bf16_us": round(t_bf * 1e6, 3), "w8a8_us": round(t_w8 * 1e6, 3),
            "w8a8_quantize_x_us": round(t_q * 1e6, 3),
            "bf16_bytes": b_bf, "w8a8_bytes": b_w8,
            "bf16_GB_per_s": round(b_bf / t_bf / 1e9, 1), "w8a8_GB_per_s": round(b_w8 / t_w8 / 1e9, 1)}


# ---------------------------------------------------------------------------
# rotary keys: rebuilt-key decode vs the folded decode on the same caches
# ---------------------------------------------------------------------------
def rope_vs_folded(w, steps, warmup=10):
    """Time wsvd_decode_attn_rope on the workload's own buffers (with its
    rotary tables) next to the folded wsvd_decode_attn already timed there.
    Returns the per-step time and GB/s (same latent/factor/q/out bytes plus
    the cos/sin tables once)."""
    import torch
    from rank_kv_cache_flash_amd import wsvd

    cfg = w.cfg
    if cfg.C_dt != "bf16" or cfg.r not in (32, 64) or cfg.H not in (64, 128):
        return None
    c, s_ = wsvd.rope_tables(cfg.L_cap, cfg.H)
    calls = []
    for d in w.sets:
        out = torch.empty(cfg.nb, cfg.nh, cfg.H, dtype=d["q"].dtype, device="cuda")
        ws = wsvd.decode_workspace(cfg.nb, cfg.nh, cfg.H, cfg.L_cap, 0)
        calls.append(wsvd.PreparedDecodeRope(d["q"], d["C_K"], d["C_V"], d["B_K"], d["B_V"], d["L"], c, s_,
                                             workspace=ws, out=out))
    t = graph_time(lambda i: calls[i % len(calls)](), steps, warmup, len(calls))
    nbytes = w.step_bytes + cfg.L_cap * cfg.H * 4
    del calls
    return {"us_per_step": round(t * 1e6, 3), "GB_per_s": round(nbytes / t / 1e9, 1),
            "pct_of_hbm_peak": round(100.0 * nbytes / t / 1e9 / HBM_PEAK_GBS, 1)}


# ---------------------------------------------------------------------------
# offline per-head factorisation (run once per layer, not part of a step)
# ---------------------------------------------------------------------------
FP64_PEAK_TFLOPS = 78.6   # MI355X fp64 vector (and matrix) peak


def factorize_offline(E=4096, nh=32, H=128, ranks=(32, 64), iters=5, cpu=True, seed=2900):
    """Time wsvd_factorize_svd and the two weighted half-steps on one LLaVA-7B
    projection (E 4096, 32 heads of 128) with eager launches, and the oracle
    on a bounded sample of the same work.  fp64 flop counts: the Gram matrix
    2 E H^2 per head (full square); each weighted solve 2 n r^2 to build its
    normal matrix over n terms plus 2 r^3 for Gauss-Jordan."""
    import numpy as np
    import torch
    from rank_kv_cache_flash_amd import inputs as I
    from rank_kv_cache_flash_amd import wsvd

    W = I.make_projection_weights(E, nh, H, seed=seed, spectrum="powerlaw")
    F = I.make_fisher_weights(E, nh, H, seed=seed)
    Wd = torch.from_numpy(W).cuda()
    Fd = torch.from_numpy(F).cuda()
    ws = torch.empty(wsvd.factorize_svd_workspace_bytes(E, nh, H), dtype=torch.uint8, device="cuda")
    rec = {"shape": f"E={E} nh={nh} H={H}", "launch": "eager, inputs resident", "fp64_peak_TFLOPs": FP64_PEAK_TFLOPS}
    for r in ranks:
        A, B, sig, sw = wsvd.factorize_svd(Wd, nh, r, workspace=ws)
        t_svd = eager_time(lambda i: wsvd.factorize_svd(Wd, nh, r, workspace=ws), iters, 2)
        t_a = eager_time(lambda i: wsvd.weighted_update_A(Wd, Fd, B, out=A), iters, 2)
        Bn = torch.empty_like(B)
        t_b = eager_time(lambda i: wsvd.weighted_update_B(Wd, Fd, A, nh, out=Bn), iters, 2)
        gram_flops = 2.0 * E * H * H * nh
        fa = E * nh * (2.0 * H * r * r + 2.0 * r ** 3)
        fb = nh * H * (2.0 * E * r * r + 2.0 * r ** 3)
        row = {"svd_ms": round(t_svd * 1e3, 3), "svd_sweeps_max": int(sw.max().item()),
               "svd_gram_TFLOPs_lower_bound": round(gram_flops / t_svd / 1e12, 2),
               "weighted_A_ms": round(t_a * 1e3, 3), "weighted_A_TFLOPs": round(fa / t_a / 1e12, 2),
               "weighted_B_ms": round(t_b * 1e3, 3), "weighted_B_TFLOPs": round(fb / t_b / 1e12, 2)}
        if cpu:
            import time
            import oracle as O
            hs = 1                                   # heads of the SVD sample
            t0 = time.perf_counter()
            O.svd_factors(W[:, :hs * H], hs, r)
            t_osvd = (time.perf_counter() - t0) * nh / hs
            rows = 16                                # rows of the A-step sample
            t0 = time.perf_counter()
            O.als_step_A(W[:rows], F[:rows], B.cpu().numpy().astype(np.float64), nh)
            t_oa = (time.perf_counter() - t0) * E / rows
            t0 = time.perf_counter()                 # one head of the B step
            O.als_step_B(W[:, :H], F[:, :H], A[:, :r].cpu().numpy().astype(np.float64), 1)
            t_ob = (time.perf_counter() - t0) * nh
            row["oracle_cpu"] = {"svd_ms": round(t_osvd * 1e3, 1), "weighted_A_ms": round(t_oa * 1e3, 1),
                                 "weighted_B_ms": round(t_ob * 1e3, 1), "cores": torch.get_num_threads(),
                                 "sample": f"SVD of {hs} heads x{nh // hs}; A step on {rows} rows x{E // rows}; "
                                           f"B step on 1 head x{nh}"}
        rec[f"r={r}"] = row
    return rec


# ---------------------------------------------------------------------------
# dense Flash-Decoding baseline at the same shape (the pages' comparison)
# ---------------------------------------------------------------------------
def dense_vs_wsvd(nb, nh, H, r, L, steps, warmup=10, seed=0, L_cap=None):
    """Time the WSVD decode step and dense Flash-Decoding on equal shapes.

    Random GPU-side bf16 inputs (timing only; parity is covered by the
    tests), cold-HBM rotation for both, graph replay of `steps` steps.
    L is an int or an int array [nb]; the cache capacity is L_cap (default
    max(L)).
    """
    import numpy as np
    import torch
    from rank_kv_cache_flash_amd import wsvd

    Ls = np.broadcast_to(np.asarray(L, dtype=np.int64), (nb,))
    L_cap = int(Ls.max()) if L_cap is None else int(L_cap)
    g = torch.Generator(device="cuda").manual_seed(seed)
    bf = torch.bfloat16

    def rnd(*shape, scale=1.0):
        return (torch.randn(*shape, generator=g, device="cuda") * scale).to(bf)

    def copies_for(nbytes):
        return max(1, min(256, math.ceil(COLD_BYTES / nbytes)))

    wb = int(Ls.sum()) * nh * 2 * r * 2 + nh * 2 * r * H * 2 + nb * nh * H * 4
    db = int(Ls.sum()) * nh * 2 * H * 2 + nb * nh * H * 4
    Lt = torch.tensor(Ls.astype(np.int32), device="cuda")
    ws = wsvd.decode_workspace(nb, nh, H, L_cap, 0)
    ws2 = wsvd.decode_workspace(nb, nh, H, L_cap, 0)
    out = torch.empty(nb, nh, H, dtype=bf, device="cuda")
    w_calls, d_calls = [], []
    for _ in range(copies_for(wb)):
        q = rnd(nb, nh, H, scale=H ** -0.5)
        CK, CV = rnd(nb, nh, L_cap, r, scale=r ** -0.5), rnd(nb, nh, L_cap, r, scale=r ** -0.5)
        BK, BV = rnd(nh, r, H, scale=H ** -0.5), rnd(nh, r, H, scale=H ** -0.5)
        w_calls.append(wsvd.PreparedDecode(q, CK, CV, BK, BV, Lt, workspace=ws, out=out))
    t_w = graph_time(lambda i: w_calls[i % len(w_calls)](), steps, warmup, len(w_calls))
    del w_calls
    torch.cuda.empty_cache()
    for _ in range(copies_for(db)):
        q = rnd(nb, nh, H, scale=H ** -0.5)
        K, V = rnd(nb, nh, L_cap, H, scale=H ** -0.5), rnd(nb, nh, L_cap, H, scale=H ** -0.5)
        d_calls.append(wsvd.PreparedDense(q, K, V, Lt, workspace=ws2, out=out))
    t_d = graph_time(lambda i: d_calls[i % len(d_calls)](), steps, warmup, len(d_calls))
    del d_calls
    torch.cuda.empty_cache()
    return {"nb": nb, "nh": nh, "H": H, "r": r, "L_sum": int(Ls.sum()), "L_cap": L_cap,
            "wsvd_us": round(t_w * 1e6, 3), "dense_us": round(t_d * 1e6, 3),
            "speedup": round(t_d / t_w, 3), "byte_ratio": round(db / wb, 3),
            "wsvd_GB_per_s": round(wb / t_w / 1e9, 1), "dense_GB_per_s": round(db / t_d / 1e9, 1)}


# ---------------------------------------------------------------------------
# ablation: conventional shared-latent decode at the same cache size
# ---------------------------------------------------------------------------
SHARED_SHAPES = {2: (1, 32, 128, 32, 1088), 3: (16, 32, 128, 64, 4096)}


def _shared_calls(nb, nh, H, R, L_cap, Lt, g, copies, out):
    import torch
    from rank_kv_cache_flash_amd import wsvd
    bf = torch.bfloat16
    ws = torch.empty(wsvd.shared_decode_workspace_bytes(nb, nh, R, L_cap, 0), dtype=torch.uint8, device="cuda")
    calls = []
    for _ in range(copies):
        q = (torch.randn(nb, nh, H, generator=g, device="cuda") * H ** -0.5).to(bf)
        CK = (torch.randn(nb, L_cap, R, generator=g, device="cuda") * R ** -0.5).to(bf)
        CV = (torch.randn(nb, L_cap, R, generator=g, device="cuda") * R ** -0.5).to(bf)
        BK = (torch.randn(R, nh * H, generator=g, device="cuda") * H ** -0.5).to(bf)
        BV = (torch.randn(R, nh * H, generator=g, device="cuda") * H ** -0.5).to(bf)
        calls.append(lambda q=q, CK=CK, CV=CV, BK=BK, BV=BV: wsvd.shared_decode_attn(q, CK, CV, BK, BV, Lt,
                                                                                     workspace=ws, out=out))
    return calls


def shared_vs_wsvd(nb, nh, H, r, L, steps, warmup=10, seed=0):
    """Per-head decode (rank r per head) against the conventional shared
    latent of the same cache size (R = nh r), on equal shapes: random GPU
    bf16 inputs (parity is covered by the tests), cold-HBM rotation for
    both, graph replay.  Reports both step times, the bytes each must read
    and the rebuild-cost ratio."""
    import numpy as np
    import torch
    from rank_kv_cache_flash_amd import wsvd

    R = nh * r
    L_cap = int(L)
    g = torch.Generator(device="cuda").manual_seed(seed)
    bf = torch.bfloat16
    Lt = torch.full((nb,), L_cap, dtype=torch.int32, device="cuda")
    out = torch.empty(nb, nh, H, dtype=bf, device="cuda")
    latent = nb * L_cap * 2 * R * 2                       # the same for both schemes
    w_fact = nh * 2 * r * H * 2
    s_fact = 2 * R * nh * H * 2                           # B_K once, B_V once per 8 sequences (lower bound)
    wb = latent + w_fact + 2 * nb * nh * H * 2
    sb_unique = latent + s_fact + 2 * nb * nh * H * 2
    sb_streamed = nh * latent + s_fact + 2 * nb * nh * H * 2

    def copies_for(nbytes):
        return max(1, min(256, math.ceil(COLD_BYTES / nbytes)))

    ws = wsvd.decode_workspace(nb, nh, H, L_cap, 0)
    w_calls = []
    for _ in range(copies_for(wb)):
        q = (torch.randn(nb, nh, H, generator=g, device="cuda") * H ** -0.5).to(bf)
        CK = (torch.randn(nb, nh, L_cap, r, generator=g, device="cuda") * r ** -0.5).to(bf)
        CV = (torch.randn(nb, nh, L_cap, r, generator=g, device="cuda") * r ** -0.5).to(bf)
        BK = (torch.randn(nh, r, H, generator=g, device="cuda") * H ** -0.5).to(bf)
        BV = (torch.randn(nh, r, H, generator=g, device="cuda") * H ** -0.5).to(bf)
        w_calls.append(wsvd.PreparedDecode(q, CK, CV, BK, BV, Lt, workspace=ws, out=out))
    t_w = graph_time(lambda i: w_calls[i % len(w_calls)](), steps, warmup, len(w_calls))
    del w_calls
    torch.cuda.empty_cache()
    s_calls = _shared_calls(nb, nh, H, R, L_cap, Lt, g, copies_for(sb_unique), out)
    t_s = graph_time(lambda i: s_calls[i % len(s_calls)](), steps, warmup, len(s_calls))
    del s_calls
    torch.cuda.empty_cache()
    return {"nb": nb, "nh": nh, "H": H, "r": r, "R": R, "L": L_cap, "r_over_R": round(r / R, 5),
            "latent_bytes_each": latent, "factor_bytes_per_head": w_fact, "factor_bytes_shared": s_fact,
            "per_head_us": round(t_w * 1e6, 3), "shared_us": round(t_s * 1e6, 3),
            "shared_over_per_head": round(t_s / t_w, 2),
            "rebuild_macs_per_token_head": {"per_head": 2 * r, "shared": 2 * R},
            "shared_bytes_if_every_head_streams_from_hbm": sb_streamed,
            "shared_effective_GB_per_s_unique": round(sb_unique / t_s / 1e9, 1),
            "per_head_GB_per_s": round(wb / t_w / 1e9, 1)}


# ---------------------------------------------------------------------------
# CPU baseline: the fp64 oracle on the host (bounded sample)
# ---------------------------------------------------------------------------
def cpu_baseline(w, gpu_out, budget_s=12.0):
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits

    import oracle as O

    cfg = w.cfg
    try:
        ncpu = len(os.sched_getaffinity(0))
    except AttributeError:
        ncpu = os.cpu_count() or 1
    with threadpool_limits(limits=ncpu):
        blas_threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
        inp = w.inp
        C_K, C_V = inp.C_K, inp.C_V
        if cfg.has_append:
            t0 = time.perf_counter()
            C_K, C_V, _, _ = O.apply_append(inp)
            t_append = time.perf_counter() - t0
        else:
            t_append = 0.0
        # (b, h) pairs in a fixed order; run until the budget is spent
        pairs = [(b, h) for b in range(cfg.nb) for h in range(cfg.nh)]
        done = []
        ref = {}
        t0 = time.perf_counter()
        k = 0
        while True:
            b, h = pairs[k % len(pairs)]
            ref[(b, h)] = O.decode_attn_one(inp, b, h, C_K=C_K, C_V=C_V)
            done.append((b, h))
            k += 1
            el = time.perf_counter() - t0
            if el >= budget_s and k >= min(len(pairs), 64):
                break
    # bytes the oracle consumed: the latents of the heads it did, factors once per head visited
    sc = {"f32": 4, "bf16": 2, "i8": 1}[cfg.C_dt]
    s_scale = 2 if cfg.C_dt == "i8" else 0
    sa = {"f32": 4, "bf16": 2, "f16": 2}[cfg.act_dt]
    lat = sum(int(w.L[b]) for b, _ in done) * 2 * (cfg.r * sc + s_scale)
    per_head = 2 * cfg.r * cfg.H * sa + cfg.H * 2 * sa
    nbytes = lat + per_head * len(done)
    frac_of_step = len(done) / float(cfg.nb * cfg.nh)
    step_s_equiv = (el + t_append) / frac_of_step if frac_of_step > 0 else float("nan")
    # parity of this benchmark run against the oracle rows it computed
    g = gpu_out.float().cpu().numpy().astype(np.float64)
    got = np.stack([g[b, h] for b, h in ref])
    want = np.stack([ref[p] for p in ref])
    err = float(np.max(np.abs(got - want)) / np.max(np.abs(want)))
    return {
        "value": round(nbytes / el / 1e9, 4),
        "unit": "GB/s",
        "cores": int(blas_threads),
        "kind": "oracle",
        "sample": (f"{len(done)} (sequence, head) rows of the {cfg.name} step in fp64, cycling over "
                   f"the step's rows ({len(done) / (cfg.nb * cfg.nh):.3g} steps' worth; {el:.1f} s)"),
        "us_per_step_equiv": round(step_s_equiv * 1e6, 1),
        "host_cpus": ncpu,
    }, err


# ---------------------------------------------------------------------------
def launch_floors(blocks, nbytes, steps, warmup, decode_grid):
    """What a launch of this size cannot beat on this device, timed like the
    step: an empty kernel, and a stream of the same bytes with every request
    issued at once (wsvd_floor_probe), rotating copies over >= 1 GiB."""
    import torch
    from rank_kv_cache_flash_amd import wsvd
    sink = torch.zeros(blocks, dtype=torch.float32, device="cuda")
    copies = max(1, min(256, math.ceil(COLD_BYTES / nbytes)))
    srcs = [torch.randint(0, 255, (nbytes,), dtype=torch.uint8, device="cuda") for _ in range(copies)]
    t_empty = graph_time(lambda i: wsvd.floor_probe(0, blocks, sink), steps, warmup)
    t_stream = graph_time(lambda i: wsvd.floor_probe(1, blocks, sink, srcs[i % copies]), steps, warmup, copies)
    del srcs
    return {"grid_blocks": blocks, "decode_grid_blocks": decode_grid, "bytes": int(nbytes),
            "empty_launch_us": round(t_empty * 1e6, 3),
            "stream_us": round(t_stream * 1e6, 3), "stream_GB_per_s": round(nbytes / t_stream / 1e9, 1),
            "stream_pct_of_hbm_peak": round(100.0 * nbytes / t_stream / 1e9 / HBM_PEAK_GBS, 1),
            "note": "wsvd_floor_probe: an empty kernel, and the decode kernel's bytes streamed with every request "
                    "issued at once (<= 64 KB per block: the decode's grid, or the smallest multiple of it that "
                    "fits); graph replay, cold HBM"}


def measure(cfg, steps, warmup, n_splits=None, cpu_budget=None, extras=True):
    """One workload: the whole step (append when the workload has one, split
    decode, merge), the dominant kernel alone for the roofline, a labelled
    warm-cache figure, the oracle on the host, and (extras) the dense
    Flash-Decoding and rotary-key comparisons on the same shapes."""
    import torch
    w = Workload(cfg, n_splits=n_splits)
    t_step = graph_timing(w.step, steps, warmup, w.copies)
    t_dec = graph_timing(w.decode_only, steps, warmup, w.copies)
    # Warm: every step on input copy 0, so whatever fits stays in L2 / the
    # Infinity Cache (256 MB).  Reported beside the cold figure, labelled.
    t_warm = graph_timing(lambda i: w.step(0), steps, warmup)
    ts, td, tw = t_step["s_per_call"], t_dec["s_per_call"], t_warm["s_per_call"]
    achieved = w.decode_kernel_bytes / td / 1e9
    rec = {
        "workload": cfg.name,
        "shape": cfg.describe(),
        "us_per_step": round(ts * 1e6, 3),
        "GB_per_s": round(w.step_bytes / ts / 1e9, 1),
        "pct_of_hbm_peak": round(100.0 * w.step_bytes / ts / 1e9 / HBM_PEAK_GBS, 1),
        "step_bytes": int(w.step_bytes),
        "splits": w.S,
        "input_copies": w.copies,
        "timing": {"graph_calls": t_step["graph_calls"], "replays_per_region": t_step["replays_per_region"],
                   "regions": t_step["regions"], "statistic": "median over regions",
                   "regions_us_per_step": [round(t * 1e6, 3) for t in t_step["regions_s_per_call"]],
                   "distinct_bytes_per_replay": int(w.step_bytes * min(t_step["graph_calls"], w.copies))},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": load_traffic(cfg.name, w.decode_kernel_bytes),
                     "kernel": "decode_split_kernel", "alg_bytes_per_launch": int(w.decode_kernel_bytes),
                     "avg_launch_us": round(td * 1e6, 3),
                     "launch_regions_us": [round(t * 1e6, 3) for t in t_dec["regions_s_per_call"]]},
        "warm_cache": {"us_per_step": round(tw * 1e6, 3), "GB_per_s": round(w.step_bytes / tw / 1e9, 1),
                       "note": "every step on one input copy (cache-resident where it fits); not an HBM figure"},
    }
    # The probe streams at most 4096 16-byte chunks per block: larger steps
    # use the smallest multiple of the decode's grid that fits.
    grid = cfg.nb * cfg.nh * w.S
    blocks = grid * max(1, math.ceil(w.decode_kernel_bytes / (16 * grid) / 4096))
    fb = w.decode_kernel_bytes // (16 * blocks) * 16 * blocks
    if fb > 0 and blocks <= (1 << 20):
        rec["floors"] = launch_floors(blocks, fb, steps, warmup, grid)
    if cpu_budget:
        torch.cuda.synchronize()
        rec["cpu_baseline"], rec["parity_max_rel_err_vs_oracle"] = cpu_baseline(w, w.out, budget_s=cpu_budget)
    if extras:
        rope = rope_vs_folded(w, steps, min(warmup, 10))
        if rope is not None:
            rec["rotary_keys"] = rope
    L = w.L.copy()
    del w
    torch.cuda.empty_cache()
    if extras and cfg.C_dt == "bf16":
        Lx = L if cfg.has_append else cfg.L
        rec["vs_dense_flash_decoding"] = dense_vs_wsvd(cfg.nb, cfg.nh, cfg.H, cfg.r, Lx, steps, min(warmup, 10),
                                                       L_cap=cfg.L_cap)
        if cfg.has_append:
            rec["vs_dense_flash_decoding"]["note"] = "decode only (no append) at the workload's ragged lengths"
    if extras and cfg.has_append:
        rec["append_alone"] = append_variants(cfg, max(steps, 100), min(warmup, 10))
    return rec


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=5)
    ap.add_argument("--also", default="2,3,4", help="other workloads measured into per_config ('' for none)")
    ap.add_argument("--splits", type=int, default=0, help="0 = the library's automatic choice")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-extras", dest="extras", action="store_false",
                    help="skip the dense, rotary and append-alone comparisons")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="oracle seconds for the headline workload")
    ap.add_argument("--cpu-budget-other", type=float, default=4.0, help="oracle seconds for each other workload")
    ap.add_argument("--mode", choices=["bench", "decode-loop", "step-loop", "copy-calib", "counters", "dense-sweep",
                                       "factorize-loop", "shared-loop", "rope-loop", "append-loop"],
                    default="bench",
                    help="decode-loop / step-loop / copy-calib / counters: plain launch loops for traces and counters")
    ap.add_argument("--configs", default="2,3,4,5", help="workloads for --mode counters")
    ap.add_argument("--calib-bytes", type=int, default=1 << 30)
    ap.add_argument("--graph", action="store_true",
                    help="decode-loop / step-loop / rope-loop: replay the calls as the benchmark does (a HIP graph)")
    ap.add_argument("--no-shared", dest="shared", action="store_false",
                    help="skip the shared-latent (conventional factorisation) ablation")
    ap.add_argument("--no-factorize", dest="factorize", action="store_false",
                    help="skip timing the offline per-head factorisation")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "the benchmark measures one GPU; the multi-GPU split is not implemented (run with --gpus 1)",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(3)
    torch.cuda.set_device(0)
    from rank_kv_cache_flash_amd import wsvd
    from rank_kv_cache_flash_amd.configs import CONFIGS
    wsvd.lib()

    if args.mode == "copy-calib":
        n = args.calib_bytes // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"mode": "copy-calib", "bytes_read": n * 4, "bytes_written": n * 4, "launches": 5}))
        return
    if args.mode == "dense-sweep":
        # WSVD decode vs dense Flash-Decoding over sequence length and batch
        # (32 heads, H = 128, r = 32 and 64); one JSON line per point.
        for r in (32, 64):
            for nb in (1, 8, 32):
                for L in (1024, 4096, 16384, 32768):
                    steps = max(10, min(400, int(2e-2 / max(nb * 32 * L * 2 * 128 * 2 / 6e12, 1e-7))))
                    rec = dense_vs_wsvd(nb, 32, 128, r, L, steps)
                    rec["steps"] = steps
                    print(json.dumps(rec), flush=True)
        return
    if args.mode == "counters":
        # 1) a plain device copy of known size (calibrates FETCH_SIZE / WRITE_SIZE),
        # 2) for each workload, the split kernel alone on the benchmark's buffers.
        n = args.calib_bytes // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        rec = {"copy_bytes": n * 4, "workloads": {}}
        for cid in [int(x) for x in args.configs.split(",") if x.strip()]:
            cfg = CONFIGS[cid]
            w = Workload(cfg)
            torch.cuda.synchronize()
            for i in range(args.steps):
                w.decode_only(i)
            if cfg.has_append:  # the append kernel alone, same count
                for i in range(args.steps):
                    w.full[i % w.copies][0]()
            torch.cuda.synchronize()
            rec["workloads"][cfg.name] = {"grid_blocks": w.cfg.nb * w.cfg.nh * w.S, "launches": args.steps,
                                          "alg_bytes_per_launch": int(w.decode_kernel_bytes), "splits": w.S}
            del w
            torch.cuda.empty_cache()
        print(json.dumps(rec))
        return
    if args.mode == "rope-loop":
        # Plain launch loop of the rotary-key decode (with output) on workload
        # --config's buffers, for kernel traces.
        cfg = CONFIGS[args.config]
        w = Workload(cfg)
        c, s_ = wsvd.rope_tables(cfg.L_cap, cfg.H)
        calls = []
        for d in w.sets:
            out = torch.empty(cfg.nb, cfg.nh, cfg.H, dtype=d["q"].dtype, device="cuda")
            ws = wsvd.decode_workspace(cfg.nb, cfg.nh, cfg.H, cfg.L_cap, 0)
            calls.append(wsvd.PreparedDecodeRope(d["q"], d["C_K"], d["C_V"], d["B_K"], d["B_V"], d["L"], c, s_,
                                                 workspace=ws, out=out))
        if args.graph:
            graph_timing(lambda i: calls[i % len(calls)](), args.steps, 5, len(calls), regions=1)
        else:
            for i in range(args.steps):
                calls[i % len(calls)]()
        torch.cuda.synchronize()
        print(json.dumps({"mode": args.mode, "workload": cfg.name, "launches": args.steps}))
        return
    if args.mode == "append-loop":
        # Plain launch loops of the append at workload 5's shape: bf16 operands,
        # then the W8A8 path (quantise x + integer append), --steps each.
        cfg = CONFIGS[5]
        nb, E, nh, r, L_cap = cfg.nb, cfg.E, cfg.nh, cfg.r, cfg.L_cap
        N = nh * r
        g = torch.Generator(device="cuda").manual_seed(0)
        bf = torch.bfloat16
        x = (torch.randn(nb, E, generator=g, device="cuda") * E ** -0.5).to(bf)
        pos = torch.randint(0, L_cap, (nb,), generator=g, device="cuda", dtype=torch.int32)
        C_K = torch.zeros(nb, nh, L_cap, r, dtype=bf, device="cuda")
        C_V = torch.zeros_like(C_K)
        ws = wsvd.append_workspace(nb, E, nh, r)
        facs = []
        for _ in range(8):
            AK = (torch.randn(E, N, generator=g, device="cuda") * r ** -0.5).to(bf)
            AV = (torch.randn(E, N, generator=g, device="cuda") * r ** -0.5).to(bf)
            facs.append((wsvd.PreparedAppend(x, AK, AV, pos, C_K, C_V, workspace=ws),
                         *wsvd.w8a8_prepare_factor(AK), *wsvd.w8a8_prepare_factor(AV)))
        xq = torch.empty(nb, E, dtype=torch.int8, device="cuda")
        sx = torch.empty(nb, dtype=torch.float32, device="cuda")
        torch.cuda.synchronize()
        for i in range(args.steps):
            facs[i % 8][0]()
        for i in range(args.steps):
            _, AKq, sAK, AVq, sAV = facs[i % 8]
            wsvd.w8a8_quantize_activations(x, xq=xq, sx=sx)
            wsvd.append_latent_w8a8(xq, sx, AKq, sAK, AVq, sAV, pos, C_K, C_V, workspace=ws)
        torch.cuda.synchronize()
        print(json.dumps({"mode": args.mode, "shape": f"x[{nb},{E}] -> {nh} heads x r {r}", "launches": args.steps}))
        return
    if args.mode == "shared-loop":
        # Plain launch loop of the shared-latent decode at the cache size of
        # workload --config (2 or 3), for kernel traces and counters.
        nb_, nh_, H_, r_, L_ = SHARED_SHAPES[args.config]
        R_ = nh_ * r_
        g = torch.Generator(device="cuda").manual_seed(0)
        Lt = torch.full((nb_,), L_, dtype=torch.int32, device="cuda")
        out = torch.empty(nb_, nh_, H_, dtype=torch.bfloat16, device="cuda")
        lat = nb_ * L_ * 2 * R_ * 2
        calls = _shared_calls(nb_, nh_, H_, R_, L_, Lt, g, max(1, min(64, math.ceil(COLD_BYTES / lat))), out)
        for i in range(args.steps):
            calls[i % len(calls)]()
        torch.cuda.synchronize()
        print(json.dumps({"mode": args.mode, "shape": f"nb={nb_} nh={nh_} H={H_} R={R_} L={L_}",
                          "launches": args.steps, "latent_bytes": lat}))
        return
    if args.mode == "factorize-loop":
        # Plain launch loop for kernel traces: per-head SVD at rank 32, then
        # one weighted A and B half-step, repeated.
        from rank_kv_cache_flash_amd import inputs as I
        E, nh, H, r = 4096, 32, 128, 32
        Wd = torch.from_numpy(I.make_projection_weights(E, nh, H, seed=2900, spectrum="powerlaw")).cuda()
        Fd = torch.from_numpy(I.make_fisher_weights(E, nh, H, seed=2900)).cuda()
        for _ in range(args.steps):
            A, B, _, _ = wsvd.factorize_svd(Wd, nh, r)
            wsvd.weighted_update_A(Wd, Fd, B, out=A)
            wsvd.weighted_update_B(Wd, Fd, A, nh, out=B)
        torch.cuda.synchronize()
        print(json.dumps({"mode": args.mode, "shape": f"E={E} nh={nh} H={H} r={r}", "launches": args.steps}))
        return
    if args.mode in ("decode-loop", "step-loop"):
        # Launch loops for kernel traces: the split kernel alone (partials
        # only, as timed for the roofline) or whole steps.  Plain launches, or
        # with --graph the benchmark's own graph replay of the same calls.
        cfg = CONFIGS[args.config]
        w = Workload(cfg, n_splits=args.splits or None)
        fn = w.decode_only if args.mode == "decode-loop" else w.step
        if args.graph:
            graph_timing(fn, args.steps, 5, w.copies, regions=1)
        else:
            for i in range(args.steps):
                fn(i)
        torch.cuda.synchronize()
        print(json.dumps({"mode": args.mode, "workload": cfg.name, "launches": args.steps,
                          "decode_kernel_bytes": w.decode_kernel_bytes, "splits": w.S}))
        return

    cfg = CONFIGS[args.config]
    main_rec = measure(cfg, args.steps, args.warmup, n_splits=args.splits or None,
                       cpu_budget=None if args.no_cpu else args.cpu_budget, extras=args.extras)

    per = {}
    also = [int(x) for x in args.also.split(",") if x.strip()] if args.also else []
    for cid in also:
        if cid == args.config:
            continue
        c = CONFIGS[cid]
        per[c.name] = measure(c, args.steps, min(args.warmup, 10),
                              cpu_budget=None if args.no_cpu else args.cpu_budget_other, extras=args.extras)
        per[c.name]["steps"] = args.steps
        torch.cuda.empty_cache()

    ablation = None
    if args.shared:
        ablation = {}
        for cid, (nb_, nh_, H_, r_, L_) in SHARED_SHAPES.items():
            ablation[CONFIGS[cid].name] = shared_vs_wsvd(nb_, nh_, H_, r_, L_, args.steps, min(args.warmup, 5))
            torch.cuda.empty_cache()

    offline = None
    if args.factorize:
        offline = factorize_offline(cpu=not args.no_cpu)
        torch.cuda.empty_cache()

    ts_us = main_rec["us_per_step"]
    line = {
        "metric": METRIC,
        "value": main_rec["GB_per_s"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ts_us * 1e-3, 6),
        "us_per_step": ts_us,
        "pct_of_hbm_peak": main_rec["pct_of_hbm_peak"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.act_dt == "bf16" else cfg.act_dt,
        "data": "synthetic (seeded N(0,1)/sqrt(dim) latents and factors; LLaVA-7B layer shapes)",
        "config": {"workload": cfg.name, "shape": cfg.describe(), "splits": main_rec["splits"],
                   "input_copies": main_rec["input_copies"],
                   "timing": "hip-graph replay of whole steps on one stream, cold HBM (>= 1 GiB touched per "
                             "replay), median of timed regions of >= 1 ms",
                   "step": ("append x.A_Kh / x.A_Vh of the new token, split decode, merge" if cfg.has_append
                            else "split decode and merge")},
        "timing": main_rec["timing"],
        "roofline": main_rec["roofline"],
        "warm_cache": main_rec["warm_cache"],
        "floors": main_rec.get("floors"),
        "cpu_baseline": main_rec.get("cpu_baseline"),
        "parity_max_rel_err_vs_oracle": main_rec.get("parity_max_rel_err_vs_oracle"),
        "vs_dense_flash_decoding": main_rec.get("vs_dense_flash_decoding"),
        "rotary_keys": main_rec.get("rotary_keys"),
        "append_alone": main_rec.get("append_alone"),
        "per_config": per,
        "shared_latent_ablation": ablation,
        "offline_factorize": offline,
        "kernel_src": kernel_src_hash(),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
