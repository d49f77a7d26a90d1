"""CPU check of the division-free level shortcut of the QSGD quantizer.

The level (QSGD summary, Knowl 1) is l + [u < x - l] with x = RN(RN(|g| /
norm) * s), l = floor(x), clamped to s, and u = (c >> 8) 2^-24 for the raw
32-bit generator word c.  With T = x + 1 - u that level is trunc(T) whenever
T is not an integer (|g| <= norm, so x <= s).  The kernel computes
d = RN(RN(|g| rs + 1 + 2^-18) - RN(c) 2^-32), rs = RN(r * s) (two fmas) for
a reciprocal r of the norm within one ulp (hardware estimate and a Newton
step), which stays within 53 * 2^-24 < 2^-18 of T + 2^-18 for a norm in
[2^-120, 2^120], and takes trunc(d) wherever fract(d) >= 2^-17; otherwise
the IEEE division.  These tests check the bound (with r rounded either way
from 1/norm, the worst the kernel can hold), the identity, and the
decisions against the level's definition on random and near-tie inputs.

The model below evaluates each fma as an exact float64 value rounded once
to float32.  RN(|g| rs + 1 + 2^-18) goes through a float64 sum, which is
exact for |g| rs >= 2^-5 and otherwise rounds twice; a double rounding
that lands on a different float32 needs the float64 sum to fall exactly on
a float32 midpoint, which random inputs do not reach."""
import numpy as np

F = np.float32
GUARD = 2.0 ** -18


def _recip(norm, way=0):
    """1/norm rounded to nearest (way 0), down (-1) or up (+1) in float32."""
    r = (F(1) / norm).astype(F)
    if way == 0:
        return r
    exact = 1.0 / norm.astype(np.float64)
    below = np.where(r.astype(np.float64) > exact, np.nextafter(r, F(0)), r)
    above = np.where(r.astype(np.float64) < exact, np.nextafter(r, F(np.inf)), r)
    return (below if way < 0 else above).astype(F)


def _rs(norm, s, way=0):
    return (_recip(norm, way) * F(s)).astype(F)


def _x_exact(g, norm, s):
    return ((np.abs(g) / norm).astype(F) * F(s)).astype(F)


def _d(g, norm, s, c, way=0):
    """The kernel's d = RN(RN(|g| rs + 1 + 2^-18) - RN(c) 2^-32)."""
    P = np.abs(g).astype(np.float64) * _rs(norm, s, way).astype(np.float64)   # exact product
    t = (P + (1.0 + GUARD)).astype(F)
    up = np.asarray(c, dtype=np.uint64).astype(F).astype(np.float64) * 2.0 ** -32
    return (t.astype(np.float64) - up).astype(F)    # exact difference, one rounding


def _exact_levels(g, norm, s, c):
    """The level as the QSGD quantizer defines it (float32 arithmetic)."""
    x = _x_exact(g, norm, s)
    u = ((np.asarray(c, dtype=np.uint64) >> 8).astype(np.float64) * 2.0 ** -24).astype(F)
    l = np.floor(x)
    p = (x - l).astype(F)
    lev = l.astype(np.int64) + (u < p)
    return np.where(x >= F(s), s, lev)


def _shortcut(g, norm, s, c, way=0):
    d = _d(g, norm, s, c, way)
    f = (d - np.floor(d)).astype(F)                    # v_fract: exact on [0, 10)
    safe = f >= F(2 * GUARD)
    return np.trunc(d).astype(np.int64), safe


def _words(rs, U):
    """32-bit generator words whose top 24 bits are U (random low byte)."""
    return (np.asarray(U, dtype=np.uint64) << np.uint64(8)) | rs.integers(0, 256, np.size(U)).astype(np.uint64)


def test_level_error_bound():
    rs = np.random.default_rng(3)
    bound = 53.0 * 2.0 ** -24
    assert bound < GUARD
    for s in range(1, 8):
        for norm_exp in (-120, -60, -20, 0, 20, 60, 119):
            m = 20_000
            norm = (rs.uniform(1, 2, m) * 2.0 ** norm_exp).astype(F)
            a = rs.uniform(0, 1, m) ** rs.choice([1, 4, 16], m)
            a[:200] = 1.0                                 # |g| == norm
            g = (a * norm.astype(np.float64)).astype(F)
            g = np.minimum(g, norm)
            c = rs.integers(0, 1 << 32, m, dtype=np.uint64)
            c[:50] = 0
            c[50:100] = (1 << 32) - 1                      # converts to 2^32: u' = 1
            x = _x_exact(g, norm, s).astype(np.float64)
            assert np.all(x <= s)
            u = (c >> np.uint64(8)).astype(np.float64) * 2.0 ** -24
            T = x + 1.0 - u                               # exact in float64
            for way in (-1, 0, 1):
                d = _d(g, norm, s, c, way).astype(np.float64)
                assert np.all(np.abs(d - (T + GUARD)) < bound), (s, norm_exp, way)
                assert np.all(d > 0)


def test_trunc_identity_matches_definition():
    # l + [u < p] (clamped to s) == trunc(x + 1 - u) when x + 1 - u is not an
    # integer, checked on float inputs with x in [0, s]
    rs = np.random.default_rng(11)
    for s in (1, 3, 7):
        x = np.concatenate([rs.uniform(0, s, 100_000), np.arange(s + 1.0)]).astype(F)
        U = rs.integers(0, 1 << 24, x.size)
        U[-(s + 1):] = 0
        u = U * 2.0 ** -24
        l = np.floor(x.astype(np.float64))
        p = x - l
        lhs = np.where(x >= s, s, l + (u < p))
        T = x.astype(np.float64) + 1.0 - u
        frac = T != np.floor(T)
        assert np.array_equal(lhs[frac], np.trunc(T)[frac])
        assert frac.sum() > 0.99 * x.size


def test_shortcut_decides_like_the_definition():
    rs = np.random.default_rng(12)
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
            x = _x_exact(g, norm, s)
            frac = x - np.floor(x)
            # u right at, just below and just above the fraction
            pick = rs.uniform(size=m) < 0.2
            U = np.where(pick, np.clip(np.round(frac * 2 ** 24) + rs.integers(-40, 41, m), 0,
                                       (1 << 24) - 1), U).astype(np.int64)
            U[900:1000] = 0
            c = _words(rs, U)
            c[1000:1100] = U[1000:1100].astype(np.uint64) << np.uint64(8)   # low byte 0
            c[1100:1200] = (U[1100:1200].astype(np.uint64) << np.uint64(8)) | np.uint64(255)
            exact = _exact_levels(g, norm, s, c)
            for way in (-1, 0, 1):
                lev, safe = _shortcut(g, norm, s, c, way)
                assert np.array_equal(lev[safe], exact[safe]), (s, norm_exp, way)
                assert np.all(lev[safe] <= s) and np.all(lev[safe] >= 0)
            total_unsafe += int((~safe).sum())
            total += m
    # the fallback is for near-ties only (here heavily over-sampled)
    assert total_unsafe < 0.5 * total


def test_shortcut_fallback_is_rare_on_plain_inputs():
    rs = np.random.default_rng(13)
    g = rs.standard_normal(512 * 400).astype(F).reshape(400, 512)
    norm = np.sqrt((g.astype(np.float64) ** 2).sum(axis=1)).astype(F)[:, None]
    nb = np.broadcast_to(norm, g.shape)
    c = rs.integers(0, 1 << 32, g.shape, dtype=np.uint64)
    lev, safe = _shortcut(g, nb, 7, c)
    exact = _exact_levels(g, nb, 7, c)
    assert np.array_equal(lev[safe], exact[safe])
    assert (~safe).mean() < 1e-4


def test_planted_mistakes_fail():
    # the exact comparison above tells a wrong level rule apart: trunc(x - u)
    # (the +1 forgotten) disagrees with the definition
    rs = np.random.default_rng(14)
    g = rs.standard_normal(200_000).astype(F)
    norm = np.full(g.shape, np.sqrt((g.astype(np.float64) ** 2).sum()), dtype=F) * F(0.01)
    g = np.minimum(np.abs(g), norm) * np.sign(g)
    c = rs.integers(0, 1 << 32, g.size, dtype=np.uint64)
    exact = _exact_levels(g, norm, 7, c)
    d = _d(g, norm, 7, c)
    wrong = np.trunc(d - F(1)).astype(np.int64)        # no +1: trunc(x - u)
    assert not np.array_equal(wrong, exact)
