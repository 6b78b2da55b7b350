"""The five synthetic decode workloads and their algorithmic byte model.

Shapes borrow a LLaVA-7B attention layer (E = 4096, 32 heads, head dim
H = 128); 1088 = 576 image tokens + 512 text tokens.  Per-head rank r and
cache dtypes vary per workload.  Bytes are what the method must move per
step -- latent K/V rows (plus int8 scales) of the attended tokens, the
factors B_K / B_V once, q and out, and for the full step the projection
factors A_K / A_V, x and the appended latent rows.  Split partials are an
implementation overhead and are not credited.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from . import inputs as _inp

DT_SIZE = {"f32": 4, "bf16": 2, "f16": 2, "i8": 1}


@dataclass(frozen=True)
class Config:
    id: int
    name: str
    nb: int
    nh: int
    H: int
    r: int
    L: int | None           # uniform attended length (None for the ragged step)
    L_cap: int
    act_dt: str             # q, B_K, B_V, out (and x, A for the full step)
    C_dt: str
    E: int = 0
    L_lo: int = 0
    L_hi: int = 0
    outlier_p: float = 0.0
    outlier_mul: float = 1.0

    @property
    def seed(self) -> int:
        return 1000 + self.id

    @property
    def has_append(self) -> bool:
        return self.E > 0

    def make(self, q_gain: float = 1.0) -> _inp.DecodeInputs:
        if self.has_append:
            return _inp.make_ragged_step_inputs(self.nb, self.nh, self.H, self.r, self.E,
                                                self.L_lo, self.L_hi, self.L_cap,
                                                seed=self.seed, q_gain=q_gain, dt=self.act_dt)
        return _inp.make_decode_inputs(self.nb, self.nh, self.H, self.r, self.L, self.L_cap,
                                       seed=self.seed, act_dt=self.act_dt, C_dt=self.C_dt,
                                       outlier_p=self.outlier_p, outlier_mul=self.outlier_mul,
                                       q_gain=q_gain)

    def draw_L(self) -> np.ndarray:
        """Attended lengths of this workload without drawing the tensors."""
        if self.has_append:
            g = _inp._rng(self.seed, _inp.T_L)
            return g.integers(self.L_lo, self.L_hi, size=self.nb, endpoint=True).astype(np.int32)
        return np.full(self.nb, self.L, dtype=np.int32)

    # ---- algorithmic bytes -------------------------------------------------
    def decode_bytes(self, L=None) -> int:
        L = self.draw_L() if L is None else np.asarray(L)
        sc = DT_SIZE[self.C_dt]
        s_scale = 2 if self.C_dt == "i8" else 0
        sa = DT_SIZE[self.act_dt]
        lat = int(np.sum(L.astype(np.int64))) * self.nh * 2 * (self.r * sc + s_scale)
        fac = self.nh * 2 * self.r * self.H * sa
        qo = self.nb * self.nh * self.H * (sa + sa)
        return lat + fac + qo

    def append_bytes(self) -> int:
        if not self.has_append:
            return 0
        sa = DT_SIZE[self.act_dt]
        sc = DT_SIZE[self.C_dt]
        return (self.E * 2 * self.nh * self.r * sa + self.nb * self.E * sa
                + self.nb * self.nh * 2 * self.r * sc)

    def step_bytes(self, L=None) -> int:
        return self.decode_bytes(L) + self.append_bytes()

    def append_flops(self) -> int:
        return 2 * self.nb * self.E * 2 * self.nh * self.r if self.has_append else 0

    def describe(self) -> str:
        if self.has_append:
            return (f"full step nb={self.nb} E={self.E} nh={self.nh} H={self.H} r={self.r} "
                    f"L~U[{self.L_lo},{self.L_hi}] L_cap={self.L_cap} {self.act_dt}")
        return (f"nb={self.nb} nh={self.nh} H={self.H} r={self.r} L={self.L} "
                f"C={self.C_dt} act={self.act_dt}")


CONFIGS = {
    1: Config(1, "tiny-fp32", nb=1, nh=4, H=64, r=16, L=256, L_cap=256,
              act_dt="f32", C_dt="f32"),
    2: Config(2, "llava7b-layer-bf16", nb=1, nh=32, H=128, r=32, L=1088, L_cap=1088,
              act_dt="bf16", C_dt="bf16"),
    3: Config(3, "batched-bf16", nb=16, nh=32, H=128, r=64, L=4096, L_cap=4096,
              act_dt="bf16", C_dt="bf16"),
    4: Config(4, "w8a8-cache-int8", nb=32, nh=32, H=128, r=32, L=2048, L_cap=2048,
              act_dt="bf16", C_dt="i8", outlier_p=0.01, outlier_mul=20.0),
    5: Config(5, "full-step-ragged-bf16", nb=64, nh=32, H=128, r=48, L=None, L_cap=8192,
              act_dt="bf16", C_dt="bf16", E=4096, L_lo=1024, L_hi=8192),
}
