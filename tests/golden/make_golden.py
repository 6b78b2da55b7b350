"""Write the stored oracle outputs under tests/golden/.

Calls only the seeded generators and oracle/ (never the GPU library).
Run from the repository root:  python tests/golden/make_golden.py
Each fixture is the fp64 oracle on the tiny fp32 workload (batch 1, 4
heads, H = 64, r = 16, L = 256, seed 1001), printed with 17 significant
digits; the GPU tests compare against these, and a CPU test re-derives
them from the oracle so any drift in the oracle shows up.
"""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle as O  # noqa: E402
from rank_kv_cache_flash_amd.configs import CONFIGS  # noqa: E402

HERE = os.path.dirname(os.path.abspath(__file__))


def fixtures():
    c = CONFIGS[1]
    base = c.make()
    peaked = c.make(q_gain=4.0 * c.H)
    out = {
        "config1_out": O.decode_attn(base).reshape(-1),
        "config1_peaked_out": O.decode_attn(peaked).reshape(-1),
    }
    o3 = []
    l3 = []
    for h in range(c.nh):
        o, lse = O.decode_partials_one(base, 0, h, 3)
        o3.append(o)
        l3.append(lse)
    out["config1_split3_o"] = np.array(o3).reshape(-1)
    out["config1_split3_lse"] = np.array(l3).reshape(-1)
    return out


def write():
    for name, arr in fixtures().items():
        with open(os.path.join(HERE, name + ".txt"), "w") as f:
            f.write(f"# {name}: fp64 oracle, tiny fp32 workload (seed 1001); "
                    f"written by tests/golden/make_golden.py\n")
            for v in arr:
                f.write(f"{v:.17g}\n")


def read(name):
    with open(os.path.join(HERE, name + ".txt")) as f:
        return np.array([float(x) for x in f if not x.startswith("#")])


if __name__ == "__main__":
    write()
