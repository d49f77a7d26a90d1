"""CPU check of the division-free level shortcut of the QSGD quantizer.

x' = RN(|g| * RN(RN(1/norm) * s)) is within 40 * 2^-24 < 2^-18 of the exact
x = RN(RN(|g| / norm) * s) for |g| <= norm (norm in [2^-120, 2^120]); the
kernel trusts x' only where no integer and no uniform lies within 2^-18 of
it, and otherwise takes the IEEE division."""
import numpy as np


def test_reciprocal_level_error_bound():
    rs = np.random.default_rng(3)
    F = np.float32
    bound = np.float64(40.0 * 2.0 ** -24)
    assert bound < 2.0 ** -18
    for s in range(1, 8):
        sf = F(s)
        for norm_exp in (-120, -60, -20, 0, 20, 60, 119):
            norm = (rs.uniform(1, 2, 20_000) * 2.0 ** norm_exp).astype(np.float32)
            a = rs.uniform(0, 1, 20_000) ** rs.choice([1, 4, 16], 20_000)
            a[:200] = 1.0                                 # |g| == norm
            g = (a * norm.astype(np.float64)).astype(np.float32)
            g = np.minimum(g, norm)
            x = (g / norm).astype(np.float32) * sf        # float32 division, then * s
            rsv = ((F(1) / norm).astype(np.float32) * sf).astype(np.float32)
            xp = (g * rsv).astype(np.float32)
            assert np.all(np.abs(x.astype(np.float64) - xp.astype(np.float64)) < bound), (s, norm_exp)
