"""Pins of the CPU oracle's QSGD widenings against what the pages fix.

QSGD summary (chapterpal): Knowl 8, max-norm scaling (a bucket is scaled by
its largest coordinate magnitude instead of its L2 norm); Knowl 3, each
processor decodes all K peers' messages and averages them; Knowl 1, the
level distribution that makes Q_s unbiased."""
from fractions import Fraction

import numpy as np

import oracle

F = np.float32


def _decode_levels(nib, n):
    i = np.arange(n)
    v = (nib[i // 8] >> (28 - 4 * (i % 8)).astype(np.uint32)) & 15
    return (v & 7).astype(np.int64), (v >> 3).astype(np.int64)


# ---------------------------------------------------------------- max-norm
def test_maxnorm_scale_is_the_largest_magnitude():
    rs = np.random.default_rng(31)
    for d in (1, 7, 64, 512, 1000):
        n = 5 * d + 3
        g = (rs.standard_normal(n) * 10.0 ** rs.uniform(-5, 2, n)).astype(F)
        g[rs.random(n) < 0.05] = F(-0.0)
        sc = oracle.qsgd_maxnorms(g, d)
        for b in range(sc.size):
            assert sc[b] == np.max(np.abs(g[b * d:(b + 1) * d])), (d, b)


def test_maxnorm_nan_ignored_inf_kept_zero_bucket():
    g = np.array([0.5, np.nan, -2.0, 1.0,   np.nan, np.nan, 0.0, -0.0,   1.0, np.inf, 3.0, 0.0],
                 dtype=F)
    sc = oracle.qsgd_maxnorms(g, 4)
    assert sc[0] == 2.0                                # NaN never becomes the scale
    assert sc[1] == 0.0 and not np.signbit(sc[1])      # NaNs and zeros: scale +0
    assert sc[2] == np.inf
    scales, nib = oracle.qsgd_quantize_maxnorm(g, 4, 7, 5)
    lev, sgn = _decode_levels(nib, g.size)
    assert lev[1] == 0 and sgn[1] == 0                 # NaN -> level 0, not negative
    assert lev[2] == 7 and sgn[2] == 1                 # the max element: level s
    assert np.all(lev[4:8] == 0)                       # zero-scale bucket


def test_maxnorm_max_element_is_level_s_and_decodes_to_itself():
    rs = np.random.default_rng(32)
    for s in range(1, 8):
        d, nb = 64, 200
        g = (rs.standard_normal(d * nb) * 0.01).astype(F)
        scales, nib = oracle.qsgd_quantize_maxnorm(g, d, s, 100 + s)
        lev, sgn = _decode_levels(nib, g.size)
        out = oracle.qsgd_dequant(scales, nib, g.size, d, s)
        for b in range(nb):
            blk = np.abs(g[b * d:(b + 1) * d])
            j = b * d + int(np.argmax(blk))
            assert lev[j] == s and sgn[j] == int(g[j] < 0)
            # (scale * s) / s is within one rounding of the scale
            assert abs(float(out[j]) - float(g[j])) <= float(np.spacing(np.abs(g[j])))
        assert np.all(lev <= s)


def test_maxnorm_levels_match_the_l2_quantizer_given_scales():
    # the levels step is shared: given the same scales, the same nibbles
    rs = np.random.default_rng(33)
    g = (rs.standard_normal(10_000) * 0.02).astype(F)
    scales, nib = oracle.qsgd_quantize_maxnorm(g, 512, 7, 9)
    assert np.array_equal(nib, oracle.qsgd_levels(g, 512, 7, 9, scales))


def test_maxnorm_unbiased_and_variance_bound():
    # Knowl 1's construction with scale m: E[Q] = v, and each coordinate's
    # variance is (m/s)^2 p(1 - p) <= m^2 / (4 s^2)
    rs = np.random.default_rng(34)
    n, d, s, M = 8, 4, 3, 1 << 14
    g = (rs.standard_normal(n) * 0.3).astype(F)
    acc = np.zeros(n)
    sq = np.zeros(n)
    for k in range(M):
        scales, nib = oracle.qsgd_quantize_maxnorm(g, d, s, 1000 + k)
        q = oracle.qsgd_dequant(scales, nib, n, d, s).astype(np.float64)
        acc += q
        sq += (q - g) ** 2
    scales = oracle.qsgd_maxnorms(g, d).astype(np.float64)
    m = np.repeat(scales, d)[:n]
    x = np.abs(g) / m * s
    p = x - np.floor(x)
    sd = (m / s) * np.sqrt(p * (1 - p))
    assert np.all(np.abs(acc / M - g) <= 5 * sd / np.sqrt(M) + 1e-7)
    assert np.all(sq / M <= m ** 2 / (4 * s * s) * 1.1 + 1e-9)


# ----------------------------------------------------- K-way decode-average
def _msgs(rs, K, n, d, s, seed0=0, maxnorm=False):
    scales, nibs = [], []
    for k in range(K):
        g = (rs.standard_normal(n) * 0.02).astype(F)
        sc, nb = (oracle.qsgd_quantize_maxnorm if maxnorm else oracle.qsgd_quantize)(
            g, d, s, seed0 + k)
        scales.append(sc)
        nibs.append(nb)
    return scales, nibs


def test_average_of_one_worker_is_its_decode():
    rs = np.random.default_rng(41)
    scales, nibs = _msgs(rs, 1, 4099, 512, 7)
    out = oracle.qsgd_dequant_average(scales, nibs, 4099, 512, 7)
    dq = oracle.qsgd_dequant(scales[0], nibs[0], 4099, 512, 7)
    assert np.array_equal(out.view(np.uint32), (dq + F(0)).view(np.uint32))   # -0 + sum from +0


def test_average_of_two_equal_messages_is_the_message():
    rs = np.random.default_rng(42)
    scales, nibs = _msgs(rs, 1, 3000, 256, 5)
    out = oracle.qsgd_dequant_average(scales * 2, nibs * 2, 3000, 256, 5)
    dq = oracle.qsgd_dequant(scales[0], nibs[0], 3000, 256, 5)
    assert np.array_equal(out, dq + F(0))


def test_average_is_exact_for_dyadic_values():
    # scales 2^e and s = 4: every decoded value and every partial sum is a
    # short dyadic number, so the float32 mean equals the exact mean
    rs = np.random.default_rng(43)
    K, n, d, s = 8, 1000, 100, 4
    scales = [(2.0 ** rs.integers(-6, 3, 10)).astype(F) for _ in range(K)]
    nibs = [rs.integers(0, 1 << 32, (n + 7) // 8, dtype=np.uint64).astype(np.uint32)
            for _ in range(K)]
    out = oracle.qsgd_dequant_average(scales, nibs, n, d, s)
    for i in range(0, n, 3):
        tot = Fraction(0)
        for k in range(K):
            nib = (int(nibs[k][i // 8]) >> (28 - 4 * (i % 8))) & 15
            v = Fraction(float(scales[k][i // d])) * (nib & 7) / s
            tot += -v if nib >> 3 else v
        assert Fraction(float(out[i])) == tot / K, i


def test_average_error_bound_and_worker_order():
    rs = np.random.default_rng(44)
    K, n, d, s = 5, 2000, 512, 7
    scales, nibs = _msgs(rs, K, n, d, s, seed0=50)
    out = oracle.qsgd_dequant_average(scales, nibs, n, d, s)
    dq = [oracle.qsgd_dequant(scales[k], nibs[k], n, d, s) for k in range(K)]
    for i in range(0, n, 5):
        vals = [Fraction(float(x[i])) for x in dq]
        exact = sum(vals, Fraction(0)) / K
        mag = sum(abs(v) for v in vals) / K
        assert abs(Fraction(float(out[i])) - exact) <= Fraction(K + 1, 1 << 24) * mag, i
    # the sum runs in worker order: reversing the workers changes some results
    rev = oracle.qsgd_dequant_average(scales[::-1], nibs[::-1], n, d, s)
    assert not np.array_equal(rev, out)


def test_average_is_unbiased_over_draws():
    # E[mean of K decodes] = mean of the K inputs (Knowl 1 unbiasedness, Knowl 3)
    rs = np.random.default_rng(45)
    K, n, d, s, M = 3, 6, 3, 2, 1 << 13
    gs = [(rs.standard_normal(n) * 0.1).astype(F) for _ in range(K)]
    acc = np.zeros(n)
    for m in range(M):
        scales, nibs = [], []
        for k in range(K):
            sc, nb = oracle.qsgd_quantize(gs[k], d, s, (m << 4) | k)
            scales.append(sc)
            nibs.append(nb)
        acc += oracle.qsgd_dequant_average(scales, nibs, n, d, s)
    want = np.mean(gs, axis=0)
    norms = [np.repeat(oracle.qsgd_norms(g, d), d)[:n].astype(np.float64) for g in gs]
    sd = np.sqrt(sum((nm / s) ** 2 / 4 for nm in norms)) / K
    assert np.all(np.abs(acc / M - want) <= 5 * sd / np.sqrt(M))


def test_average_divides_by_k_once():
    # three identical messages whose value v decodes exactly (s = 1, level
    # 1: v = scale); the sum is RN(RN(2v) + v) = RN(3v), and the mean must be
    # the correctly rounded RN(3v) / 3 -- for some v that differs from
    # RN(3v) * RN(1/3); brute force over many v at this tiny size
    rs = np.random.default_rng(46)
    vals = (rs.uniform(1, 2, 4000)).astype(F)
    nib = np.array([0x10000000], dtype=np.uint32)        # element 0: sign 0, level 1
    differs = 0
    for v in vals:
        sc = [np.array([v], F)] * 3
        out = oracle.qsgd_dequant_average(sc, [nib] * 3, 1, 1, 1)[0]
        three_v = F(F(v + v) + v)
        assert out == three_v / F(3), v
        differs += bool(three_v / F(3) != three_v * F(1.0 / 3.0))
    assert differs > 0


def test_average_sums_in_worker_order():
    # brute force on a few elements: float32 additions in order 0..K-1 of
    # the (pinned) single-worker decodes, from +0, then one division by K
    rs = np.random.default_rng(47)
    K, n, d, s = 6, 400, 64, 7
    scales, nibs = _msgs(rs, K, n, d, s, seed0=70)
    out = oracle.qsgd_dequant_average(scales, nibs, n, d, s)
    dq = [oracle.qsgd_dequant(scales[k], nibs[k], n, d, s) for k in range(K)]
    for i in range(n):
        acc = F(0)
        for k in range(K):
            acc = F(acc + dq[k][i])
        assert out[i] == F(acc / F(K)), i
