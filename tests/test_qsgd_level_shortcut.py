"""CPU check of the division-free level shortcut of the QSGD quantizer.

x' = RN(|g| * RN(RN(1/norm) * s)) is within 40 * 2^-24 < 2^-18 of the exact
x = RN(RN(|g| / norm) * s) for |g| <= norm (norm in [2^-120, 2^120]).  The
level l + [u < x - l] (l = floor(x)) equals ceil(x - u); the kernel takes
ceil(d) for d = RN(x' - u) wherever d lies more than 2^-18 from every
integer, and otherwise the IEEE division.  These tests check the bound, the
identity, and the decisions against the level's definition on random and
near-tie inputs."""
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


def _exact_levels(g, norm, s, u):
    """The level as the QSGD quantizer defines it (float32 arithmetic):
    x = RN(RN(|g|/norm) * s), l = floor(x), level l + [u < x - l], x >= s -> s."""
    F = np.float32
    x = ((np.abs(g) / norm).astype(F) * F(s)).astype(F)
    l = np.floor(x)
    p = (x - l).astype(F)
    lev = l.astype(np.int64) + (u < p)
    return np.where(x >= F(s), s, lev)


def _shortcut(g, norm, s, U):
    """The division-free decision: d = RN(RN(|g| rs) - U 2^-24), level
    ceil(d), trusted when |(ceil(d) - d) - 0.5| < 0.5 - 2^-18 (float32)."""
    F = np.float32
    rs = ((F(1) / norm).astype(F) * F(s)).astype(F)
    xp = (np.abs(g) * rs).astype(F)
    u = (U * 2.0 ** -24).astype(F)
    d = (xp.astype(np.float64) - u.astype(np.float64)).astype(F)   # one rounding, as the fma
    c = np.ceil(d)
    dist = np.abs(((c - d).astype(F) - F(0.5)).astype(F))
    safe = dist < F(0.5) - F(2.0 ** -18)
    return c.astype(np.int64), safe


def test_ceil_identity_matches_definition():
    # l + [u < p] == ceil(x - u) in exact arithmetic, checked on float inputs
    rs = np.random.default_rng(11)
    x = np.concatenate([rs.uniform(0, 7, 100_000), np.arange(8.0)]).astype(np.float32)
    U = rs.integers(0, 1 << 24, x.size)
    U[:8] = 0
    u = U * 2.0 ** -24
    l = np.floor(x.astype(np.float64))
    p = x - l
    lhs = l + (u < p)
    rhs = np.ceil(x.astype(np.float64) - u)
    assert np.array_equal(lhs, rhs)


def test_shortcut_decides_like_the_definition():
    rs = np.random.default_rng(12)
    F = np.float32
    total_unsafe = 0
    total = 0
    for s in range(1, 8):
        for norm_exp in (-120, -40, 0, 40, 119):
            m = 40_000
            norm = (rs.uniform(1, 2, m) * 2.0 ** norm_exp).astype(F)
            a = rs.uniform(0, 1, m)
            # adversarial: x near an integer, u near the fraction, x near s
            k = rs.integers(0, s + 1, m)
            near = (k + rs.uniform(-3e-6, 3e-6, m)) / s
            a = np.where(rs.uniform(size=m) < 0.3, np.clip(near, 0, 1), a)
            a[:300] = 1.0
            a[300:600] = 0.0
            g = (a * norm.astype(np.float64)).astype(F)
            g = np.minimum(g, norm)
            g[600:900] *= F(-1)
            U = rs.integers(0, 1 << 24, m)
            x = ((np.abs(g) / norm).astype(F) * F(s)).astype(F)
            frac = x - np.floor(x)
            # u right at, just below and just above the fraction
            pick = rs.uniform(size=m) < 0.2
            U = np.where(pick, np.clip(np.round(frac * 2 ** 24) + rs.integers(-40, 41, m), 0,
                                       (1 << 24) - 1), U).astype(np.int64)
            U[900:1000] = 0
            u = (U * 2.0 ** -24).astype(F)
            exact = _exact_levels(g, norm, s, u)
            lev, safe = _shortcut(g, norm, s, U)
            assert np.array_equal(lev[safe], exact[safe]), (s, norm_exp)
            total_unsafe += int((~safe).sum())
            total += m
    # the fallback is for near-ties only (here heavily over-sampled)
    assert total_unsafe < 0.5 * total


def test_shortcut_fallback_is_rare_on_plain_inputs():
    rs = np.random.default_rng(13)
    F = np.float32
    g = rs.standard_normal(512 * 400).astype(F).reshape(400, 512)
    norm = np.sqrt((g.astype(np.float64) ** 2).sum(axis=1)).astype(F)[:, None]
    U = rs.integers(0, 1 << 24, g.shape)
    lev, safe = _shortcut(g, np.broadcast_to(norm, g.shape), 7, U)
    exact = _exact_levels(g, np.broadcast_to(norm, g.shape), 7, (U * 2.0 ** -24).astype(F))
    assert np.array_equal(lev[safe], exact[safe])
    assert (~safe).mean() < 1e-4
