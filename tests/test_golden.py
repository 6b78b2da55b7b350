"""The stored oracle fixtures still match the oracle (CPU)."""
import numpy as np

from tests.golden import make_golden as G


def test_golden_fixtures_reproduce():
    for name, arr in G.fixtures().items():
        np.testing.assert_allclose(G.read(name), arr, rtol=1e-15, atol=1e-300)


def test_golden_split_partials_merge_to_output():
    import oracle as O
    o = G.read("config1_split3_o").reshape(4, 3, 64)
    lse = G.read("config1_split3_lse").reshape(4, 3)
    out = G.read("config1_out").reshape(4, 64)
    for h in range(4):
        np.testing.assert_allclose(O.combine(o[h], lse[h]), out[h], atol=1e-14)
