"""Pins of the CPU oracle's Elias-omega coding of QSGD buckets.

QSGD summary (chapterpal), Knowl 2: a quantized bucket is the tuple (norm,
signs, levels), the norm in 32 bits, the non-zero coordinates coded by the
omega code of the distance between them with their sign and level; the
expected message length for s >= 2 is bounded by
(3 + (3/2 + o(1)) log2(2(s^2 + n) / (s(s + sqrt n)))) s(s + sqrt n) + 32.
The omega code itself is P. Elias, "Universal codeword sets and
representations of the integers" (1975)."""
import os

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "elias_omega_codes.txt")


def _golden():
    codes, msg = {}, {}
    for line in open(GOLDEN):
        if line.startswith("code "):
            _, k, bits = line.split()
            codes[int(k)] = bits
        elif line.startswith("message_"):
            key, _, rest = line.partition(" ")
            msg[key] = rest.strip()
    return codes, msg


def _bits(words, lo, hi):
    s = "".join(format(int(w), "032b") for w in words)
    return s[lo:hi]


def _nibbles_for(n, entries):
    nib = np.zeros((n + 7) // 8, np.uint32)
    for i, (sign, level) in entries.items():
        nib[i // 8] |= np.uint32(((sign << 3) | level) << (28 - 4 * (i % 8)))
    return nib


def test_omega_codes_match_the_definition():
    codes, _ = _golden()
    assert len(codes) == 11
    for k, want in codes.items():
        assert oracle.omega_length(k) == len(want), k
        # a bucket whose only non-zero coordinate sits at distance k from -1
        d = 1024
        nib = _nibbles_for(d, {k - 1: (1, 1)})
        offs, words = oracle.qsgd_elias_encode(np.array([1.0], np.float32), nib, d, d)
        assert int(offs[1]) == 32 + len(want) + 2, k
        assert _bits(words, 32, int(offs[1])) == want + "1" + "0", k


def test_worked_message():
    _, msg = _golden()
    d = int(msg["message_d"])
    nib = np.array([int(msg["message_nibbles"], 16) >> 32, int(msg["message_nibbles"], 16) &
                    0xFFFFFFFF], np.uint32)
    norm = np.array([int(msg["message_norm"], 16)], np.uint32).view(np.float32)
    offs, words = oracle.qsgd_elias_encode(norm, nib, d, d)
    want = msg["message_bits"].replace(" ", "")
    assert int(offs[1]) == len(want) == 56
    assert _bits(words, 0, len(want)) == want
    assert _bits(words, len(want), 32 * words.size) == "0" * (32 * words.size - len(want))
    n2, nib2 = oracle.qsgd_elias_decode(words, offs, d, d)
    assert np.array_equal(n2.view(np.uint32), norm.view(np.uint32))
    assert np.array_equal(nib2, nib)


def _clear_zero_level_signs(nib, n):
    out = nib.copy()
    for i in range(n):
        v = (int(out[i // 8]) >> (28 - 4 * (i % 8))) & 15
        if v == 8:
            out[i // 8] &= np.uint32(~(0xF << (28 - 4 * (i % 8))) & 0xFFFFFFFF)
    return out


def test_round_trip_restores_norms_levels_and_signs():
    rs = np.random.default_rng(61)
    for n, d, s, spiky in ((4096, 512, 7, False), (5000, 512, 3, True), (777, 64, 7, True),
                           (2048, 256, 1, False), (1000, 8, 7, False)):
        g = (rs.standard_normal(n) * 0.01).astype(np.float32)
        if spiky:
            g[rs.integers(0, n, n // 50)] *= np.float32(200.0)
        g[rs.integers(0, n, 20)] = np.float32(-0.0)
        norms, nib = oracle.qsgd_quantize(g, d, s, 99)
        offs, words = oracle.qsgd_elias_encode(norms, nib, n, d)
        n2, nib2 = oracle.qsgd_elias_decode(words, offs, n, d)
        assert np.array_equal(n2.view(np.uint32), norms.view(np.uint32))
        # signs are coded only where the level is not 0 (the value is +-0 there)
        assert np.array_equal(nib2, _clear_zero_level_signs(nib, n)), (n, d, s)
        # offsets are non-decreasing, each bucket at least its 32 norm bits
        assert np.all(np.diff(offs.astype(np.int64)) >= 32)


def test_zero_buckets_are_32_bits():
    n, d = 3000, 500
    norms = np.zeros(6, np.float32)
    offs, words = oracle.qsgd_elias_encode(norms, np.zeros(375, np.uint32), n, d)
    assert np.array_equal(offs, np.arange(7, dtype=np.uint64) * 32)
    assert not np.any(words)


def test_bits_per_bucket_within_the_sparse_regime_bound():
    # Knowl 2, s >= 2: expected bits per bucket of dimension d below
    # (3 + (3/2 + o(1)) log2(2 (s^2 + d) / (s (s + sqrt d)))) s (s + sqrt d) + 32,
    # here checked with the o(1) term set to 0 on Gaussian buckets
    rs = np.random.default_rng(62)
    d, nb = 512, 400
    for s in (2, 3, 5, 7):
        g = rs.standard_normal(d * nb).astype(np.float32)
        norms, nib = oracle.qsgd_quantize(g, d, s, 500 + s)
        offs, _ = oracle.qsgd_elias_encode(norms, nib, d * nb, d)
        mean_bits = float(offs[-1]) / nb
        a = s * (s + np.sqrt(d))
        bound = (3 + 1.5 * np.log2(2 * (s * s + d) / a)) * a + 32
        assert mean_bits <= bound, (s, mean_bits, bound)
