"""Pins of the CPU oracle's SAPS sparsification against what the pages fix.

"Communication-Efficient Decentralized Learning with Sparsification and
Adaptive Peer Selection": the model is masked by Bernoulli(1/c) entries drawn
from a seed every worker shares, so all workers keep the same components;
only the kept components are exchanged; each worker talks to one peer (two
non-zero entries per row of a doubly stochastic gossip matrix).

The uniform stream is the Philox-4x32-10 stream of the QSGD quantizer (the
pages name no generator: parity of the exact stream is unpinned by them); the
mask is checked here against an independent Python-integer Philox
(tests/brute.py), so the oracle's mask rule and indexing are pinned."""
from fractions import Fraction

import numpy as np

import oracle
from tests import brute

F = np.float32


def _brute_keep(seed, n, c):
    q = np.arange((n + 3) // 4, dtype=np.uint64)
    words = brute.philox4x32_10_np(q & np.uint64(0xFFFFFFFF), q >> np.uint64(32), 0, 0,
                                   seed & 0xFFFFFFFF, seed >> 32)
    w = np.stack(words, axis=1).reshape(-1)[:n]
    U = (w >> np.uint64(8)).astype(np.float64)
    return U * float(F(c)) < 2.0 ** 24            # u c < 1, exact in float64


def _kept_indices(n, c, seed):
    return oracle.saps_gather(np.arange(n, dtype=np.float32), c, seed).astype(np.int64)


def test_mask_matches_independent_generator():
    n = 20_000
    for seed in (1, 0xDEADBEEF12345678):
        for c in (1.0, 1.5, 3.5, 4.0, 100.0, 1e6):
            want = np.flatnonzero(_brute_keep(seed, n, c))
            assert np.array_equal(_kept_indices(n, c, seed), want), (seed, c)


def test_keep_range_at_any_start():
    # the per-range mask the whole-size GPU tests use: element start + j is
    # kept exactly when the independent generator's draw for that global
    # index says so, whatever the start (a multiple of 4 or not)
    seed, c, n = 0xDEADBEEF12345678, 3.5, 9_001
    for start in (0, 1, 12_345, (1 << 33) + 3):
        q = np.arange(start >> 2, ((start + n + 3) >> 2) + 1, dtype=np.uint64)
        words = brute.philox4x32_10_np(q & np.uint64(0xFFFFFFFF), q >> np.uint64(32), 0, 0,
                                       seed & 0xFFFFFFFF, seed >> 32)
        w = np.stack(words, axis=1).reshape(-1)
        U = (w >> np.uint64(8)).astype(np.float64)[start - 4 * (start >> 2):][:n]
        want = U * float(F(c)) < 2.0 ** 24
        assert np.array_equal(oracle.saps_keep(seed, n, c, start=start), want), start


def test_exact_threshold_at_powers_of_two():
    # c = 2^k: kept exactly when the 24-bit draw U < 2^(24-k); u c == 1 is dropped
    n = 40_000
    q = np.arange(n // 4, dtype=np.uint64)
    w = np.stack(brute.philox4x32_10_np(q, 0, 0, 0, 9, 0), axis=1).reshape(-1)
    U = (w >> np.uint64(8)).astype(np.int64)
    for k in (0, 1, 2, 5):
        want = np.flatnonzero(U < (1 << (24 - k)))
        assert np.array_equal(_kept_indices(n, 2.0 ** k, 9), want), k
    assert _kept_indices(1000, 1.0, 3).size == 1000       # c = 1 keeps everything


def test_density_and_seed_independence():
    n, c = 2_000_000, 100.0
    a = _kept_indices(n, c, 11)
    b = _kept_indices(n, c, 11)
    other = _kept_indices(n, c, 12)
    assert np.array_equal(a, b)                           # the shared seed: the same mask
    mu, sd = n / c, np.sqrt(n / c * (1 - 1 / c))
    assert abs(a.size - mu) < 5 * sd
    both = np.intersect1d(a, other).size                  # ~ n / c^2 for independent masks
    assert abs(both - n / c / c) < 5 * np.sqrt(n / c / c) + 5


def test_gather_is_masked_selection_in_order():
    rs = np.random.default_rng(5)
    n = 50_001
    x = rs.standard_normal(n).astype(F)
    x[::97] = F(-0.0)
    x[5::1001] = np.nan
    for c in (2.0, 7.25, 100.0):
        vals = oracle.saps_gather(x, c, 21)
        want = x[_brute_keep(21, n, c)]
        assert np.array_equal(vals.view(np.uint32), want.view(np.uint32)), c


def test_merge_rules():
    rs = np.random.default_rng(6)
    n, c, seed = 30_000, 10.0, 33
    keep = _brute_keep(seed, n, c)
    x = rs.standard_normal(n).astype(F)
    # merging one's own values changes nothing
    x1 = x.copy()
    cnt = oracle.saps_merge(x1, c, seed, oracle.saps_gather(x, c, seed))
    assert cnt == keep.sum()
    assert np.array_equal(x1.view(np.uint32), x.view(np.uint32))
    # dyadic values: the average is exact; unkept components untouched
    xa = (rs.integers(-512, 512, n) / 256.0).astype(F)
    xb = (rs.integers(-512, 512, n) / 64.0).astype(F)
    m = xa.copy()
    oracle.saps_merge(m, c, seed, oracle.saps_gather(xb, c, seed))
    for i in np.flatnonzero(keep)[:2000]:
        assert Fraction(float(m[i])) == (Fraction(float(xa[i])) + Fraction(float(xb[i]))) / 2
    assert np.array_equal(m[~keep].view(np.uint32), xa[~keep].view(np.uint32))


def test_pairwise_exchange_reaches_agreement():
    # two peers exchange their kept components and each merges the other's:
    # afterwards they agree exactly on every kept component (the gossip step)
    rs = np.random.default_rng(7)
    n, c, seed = 20_000, 4.0, 44
    a = rs.standard_normal(n).astype(F)
    b = rs.standard_normal(n).astype(F)
    va, vb = oracle.saps_gather(a, c, seed), oracle.saps_gather(b, c, seed)
    oracle.saps_merge(a, c, seed, vb)
    oracle.saps_merge(b, c, seed, va)
    keep = _brute_keep(seed, n, c)
    assert np.array_equal(a[keep], b[keep])
    # and each kept component is within half an ulp of the exact average
    for i in np.flatnonzero(keep)[:500]:
        exact = (Fraction(float(va[np.searchsorted(np.flatnonzero(keep), i)])) +
                 Fraction(float(vb[np.searchsorted(np.flatnonzero(keep), i)]))) / 2
        assert abs(Fraction(float(a[i])) - exact) <= Fraction(float(np.spacing(abs(a[i]))))


def test_boundary_u_times_c_equal_one_is_dropped():
    # find draws U = 2^j (searched in the independent Python Philox stream);
    # with c = 2^(24-j), u c == 1 exactly: dropped (the rule is u c < 1), and
    # kept for the next float below c
    seed = 77
    q = np.arange(1 << 20, dtype=np.uint64)
    w = np.stack(brute.philox4x32_10_np(q, 0, 0, 0, seed, 0), axis=1).reshape(-1)
    U = (w >> np.uint64(8)).astype(np.int64)
    pow2 = (U >= 256) & ((U & (U - 1)) == 0)
    hits = np.flatnonzero(pow2)[:4]
    assert hits.size >= 2
    lib = oracle._load()
    import ctypes
    for i in hits:
        c = F(2.0 ** 24 / U[i])
        assert not lib.oracle_saps_keep(seed, int(i), ctypes.c_float(c)), i
        assert lib.oracle_saps_keep(seed, int(i), ctypes.c_float(np.nextafter(c, F(0)))), i
