"""GPU parity of the Elias-omega coding of QSGD buckets (qsgd_elias_encode,
qsgd_elias_decode) against the CPU oracle, bit-exact: bit offsets, coded
words, decoded norms and nibbles.

QSGD summary (chapterpal), Knowl 2; the omega code of P. Elias (1975)."""
import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.gpu


def say(*a):
    print("[gpu]", *a, flush=True)


def dev(a):
    import torch

    if a.dtype == np.uint32:
        a = a.view(np.int32)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    a = t.detach().cpu().numpy()
    return a.view(np.uint32) if a.dtype == np.int32 else a


def clear_zero_level_signs(nib):
    v = nib.copy()
    for k in range(8):
        sh = np.uint32(28 - 4 * k)
        f = (v >> sh) & np.uint32(15)
        v &= ~np.where(f == 8, np.uint32(15) << sh, np.uint32(0))
    return v


def check(gpu, norms_h, nib_h, n, d):
    import torch

    offs_d, out_d = gpu.qsgd_elias_encode(dev(norms_h), dev(nib_h), n, d)
    offs_h, words_h = oracle.qsgd_elias_encode(norms_h, nib_h, n, d)
    offs = host(offs_d).astype(np.uint64)
    assert np.array_equal(offs, offs_h), (n, d)
    nw = words_h.size
    assert np.array_equal(host(out_d)[:nw], words_h), (n, d)
    # decode on the GPU what the oracle coded, and compare with the oracle's decode
    norms2, nib2 = gpu.qsgd_elias_decode(dev(words_h) if nw else torch.zeros(1, dtype=torch.int32,
                                                                             device="cuda"),
                                         offs_d, n, d)
    n_h, nb_h = oracle.qsgd_elias_decode(words_h if nw else np.zeros(1, np.uint32), offs_h, n, d)
    assert np.array_equal(host(norms2).view(np.uint32), n_h.view(np.uint32)), (n, d)
    assert np.array_equal(host(nib2), nb_h), (n, d)
    # and the round trip restores the quantizer output up to level-0 signs
    assert np.array_equal(nb_h, clear_zero_level_signs(nib_h)), (n, d)
    return offs_d, out_d


@pytest.mark.parametrize("d", [8, 16, 64, 256, 512, 1000, 2048])
def test_bucket_sizes(gpu, d):
    say("elias d", d)
    rs = np.random.default_rng(100 + d)
    for n in (d, 3 * d + 5, 70_001, 8):
        for s, spiky in ((7, False), (3, True), (1, False), (7, True)):
            g = (rs.standard_normal(n) * 0.01).astype(np.float32)
            if spiky:
                g[rs.integers(0, n, max(n // 40, 1))] *= np.float32(300.0)
            g[rs.integers(0, n, 5)] = np.float32(-0.0)
            norms, nib = oracle.qsgd_quantize(g, d, s, 7 * n + s)
            check(gpu, norms, nib, n, d)


def test_dense_and_empty_buckets(gpu):
    # every coordinate non-zero (the longest codes), all-zero buckets (32 bits
    # each), and random nibbles with every sign/level
    say("elias dense / empty")
    rs = np.random.default_rng(110)
    for d in (8, 512, 2048):
        n = 5 * d
        nib = rs.integers(0, 1 << 32, (n + 7) // 8, dtype=np.uint64).astype(np.uint32)
        nib |= np.uint32(0x11111111)              # no level 0 anywhere
        norms = rs.uniform(0.1, 3, (n + d - 1) // d).astype(np.float32)
        check(gpu, norms, nib, n, d)
        check(gpu, norms, np.zeros((n + 7) // 8, np.uint32), n, d)
        nib2 = rs.integers(0, 1 << 32, (n + 7) // 8, dtype=np.uint64).astype(np.uint32)
        check(gpu, norms, nib2, n, d)


def test_capacity_and_guard_words(gpu):
    import torch

    say("elias capacity")
    rs = np.random.default_rng(111)
    n, d = 100_000, 512
    g = (rs.standard_normal(n) * 0.01).astype(np.float32)
    norms, nib = oracle.qsgd_quantize(g, d, 7, 3)
    offs_h, words_h = oracle.qsgd_elias_encode(norms, nib, n, d)
    for cap in (words_h.size, words_h.size // 2, 17):
        out = torch.full((words_h.size + 64,), 0x5A5A5A5A, dtype=torch.int32, device="cuda")
        offs = torch.empty(offs_h.size, dtype=torch.int64, device="cuda")
        gpu.qsgd_elias_encode(dev(norms), dev(nib), n, d, offsets=offs, out=out[:cap])
        o = host(out)
        assert np.array_equal(host(offs).astype(np.uint64), offs_h)
        # every word below the capacity is complete (each bucket writes its
        # words that fit), nothing past it is touched
        assert np.array_equal(o[:cap], words_h[:cap]), cap
        assert np.all(o[cap:] == 0x5A5A5A5A), cap


def test_wavefronts_past_the_stage(gpu):
    # a wavefront codes 64 consecutive buckets; when their words exceed its
    # LDS stage (1984 words) each lane stores its words itself: dense buckets
    # of 129+ words each, mixed with sparse ones, at several capacities
    import torch

    say("elias unstaged wavefronts")
    rs = np.random.default_rng(113)
    for d in (512, 256):
        nb = 3 * 64 + 7
        n = nb * d - 3
        nib = rs.integers(0, 1 << 32, (n + 7) // 8, dtype=np.uint64).astype(np.uint32)
        dense = rs.uniform(size=nb) < 0.7
        for bk in range(nb):
            w0, w1 = bk * d // 8, min((bk + 1) * d // 8, nib.size)
            if dense[bk]:
                nib[w0:w1] |= np.uint32(0x11111111)
            else:
                nib[w0:w1] &= np.uint32(0x88888888) | (nib[w0:w1] >> np.uint32(5)) & np.uint32(0x01000100)
        norms = rs.uniform(0.1, 3, nb).astype(np.float32)
        check(gpu, norms, nib, n, d)
        offs_h, words_h = oracle.qsgd_elias_encode(norms, nib, n, d)
        for cap in (words_h.size // 3, 4097):
            out = torch.full((words_h.size + 64,), 0x5A5A5A5A, dtype=torch.int32, device="cuda")
            offs = torch.empty(offs_h.size, dtype=torch.int64, device="cuda")
            gpu.qsgd_elias_encode(dev(norms), dev(nib), n, d, offsets=offs, out=out[:cap])
            o = host(out)
            assert np.array_equal(o[:cap], words_h[:cap]), (d, cap)
            assert np.all(o[cap:] == 0x5A5A5A5A), (d, cap)


def test_round_trip_on_gpu(gpu):
    say("elias gpu round trip")
    rs = np.random.default_rng(112)
    n, d = 1_000_003 - 3, 512
    g = (rs.standard_normal(n) * 0.02).astype(np.float32)
    norms_d, nib_d = gpu.qsgd_quantize(dev(g), d, 7, 11)
    offs, words = gpu.qsgd_elias_encode(norms_d, nib_d, n, d)
    norms2, nib2 = gpu.qsgd_elias_decode(words, offs, n, d)
    assert np.array_equal(host(norms2).view(np.uint32), host(norms_d).view(np.uint32))
    assert np.array_equal(host(nib2), clear_zero_level_signs(host(nib_d)))


def test_encode_from_unaligned_nibbles(gpu):
    # d a multiple of 32 with nibbles that are 4- but not 16-byte aligned: the
    # encoder reads word by word instead of 16-byte blocks
    import torch

    say("elias encode, unaligned nibbles")
    rs = np.random.default_rng(115)
    for d in (256, 512):
        n = 70 * d + 77
        g = (rs.standard_normal(n) * 0.01).astype(np.float32)
        norms, nib = oracle.qsgd_quantize(g, d, 7, 51 + d)
        offs_h, words_h = oracle.qsgd_elias_encode(norms, nib, n, d)
        buf = torch.zeros(nib.size + 4, dtype=torch.int32, device="cuda")
        buf[1:1 + nib.size] = dev(nib)
        offs, out = gpu.qsgd_elias_encode(dev(norms), buf[1:1 + nib.size], n, d)
        assert np.array_equal(host(offs).astype(np.uint64), offs_h), d
        assert np.array_equal(host(out)[:words_h.size], words_h), d


def _bits(words, lo, hi):
    w = np.ascontiguousarray(words).astype(">u4").view(np.uint8)
    return np.unpackbits(w)[lo:hi]


def test_decode_into_unaligned_output(gpu):
    # d a multiple of 32 with an output that is 4- but not 16-byte aligned:
    # the word-by-word store path, against the oracle's decode
    import torch

    say("elias decode, unaligned output")
    rs = np.random.default_rng(114)
    for d in (256, 512):
        n = 37 * d + 100
        g = (rs.standard_normal(n) * 0.01).astype(np.float32)
        norms, nib = oracle.qsgd_quantize(g, d, 7, 41 + d)
        offs_h, words_h = oracle.qsgd_elias_encode(norms, nib, n, d)
        nw = nib.size
        buf = torch.full((nw + 8,), 0x3C3C3C3C, dtype=torch.int32, device="cuda")
        out_n = torch.empty(norms.size, device="cuda")
        gpu.qsgd_elias_decode(dev(words_h), dev(offs_h.astype(np.int64)), n, d, norms=out_n,
                              nibbles=buf[1:1 + nw])
        _, nb_h = oracle.qsgd_elias_decode(words_h, offs_h, n, d)
        b = host(buf)
        assert np.array_equal(b[1:1 + nw], nb_h), d
        assert b[0] == 0x3C3C3C3C and np.all(b[1 + nw:] == 0x3C3C3C3C)
        assert np.array_equal(host(out_n).view(np.uint32), norms.view(np.uint32))


def _reference_truncated_decode(words, offs, n, d, in_count):
    """The decode contract on an input cut to in_count words, bit by bit in
    Python: no bit past the cut or past a bucket's end is read; a norm needs
    its 32 bits (else 0); a coordinate whose codes do not all fit, or whose
    index or level is out of range, stops the bucket; uncoded coordinates
    get nibble 0.  Omega codes: groups of a 1 and k more digits, ended by 0."""
    bits = np.unpackbits(np.ascontiguousarray(words[:in_count]).astype(">u4").view(np.uint8))
    limit = in_count * 32
    nb = (n + d - 1) // d
    norms = np.zeros(nb, np.uint32)
    nib = np.zeros((n + 7) // 8, np.uint32)
    for b in range(nb):
        blen = min(d, n - b * d)
        start, end = int(offs[b]), min(int(offs[b + 1]), limit)
        start = min(start, end)
        st = {"pos": start, "ok": True}

        def get(k):
            if not st["ok"] or st["pos"] + k > end:
                st["ok"] = False
                return 0
            v = 0
            for i in range(k):
                v = (v << 1) | int(bits[st["pos"] + i])
            st["pos"] += k
            return v

        def omega():
            k = 1
            while st["ok"] and get(1):
                if k >= 31:
                    st["ok"] = False
                    return 0
                k = (1 << k) | get(k)
            return k

        norms[b] = get(32)
        prev = -1
        while st["ok"] and st["pos"] < end:
            li = prev + omega()
            sign = get(1)
            level = omega()
            if not st["ok"] or li >= blen or level > 7:
                break
            i = b * d + li
            nib[i // 8] |= np.uint32(((sign << 3) | level) << (28 - 4 * (i % 8)))
            prev = li
    return norms, nib


@pytest.mark.parametrize("d", [64, 512, 1000])
def test_decode_of_a_truncated_input(gpu, d):
    # the input cut short at several word counts: buckets before the cut decode
    # as usual, the bucket across it keeps its whole coordinates, later ones
    # come out as zeros; nothing past the cut is read
    say("elias truncated input d", d)
    rs = np.random.default_rng(115 + d)
    n = 12 * d + 7
    g = (rs.standard_normal(n) * 0.01).astype(np.float32)
    g[rs.integers(0, n, n // 30)] *= np.float32(200.0)
    norms, nib = oracle.qsgd_quantize(g, d, 7, 51 + d)
    offs_h, words_h = oracle.qsgd_elias_encode(norms, nib, n, d)
    offs_d = dev(offs_h.astype(np.int64))
    total = words_h.size
    for cut in sorted({1, 2, total // 5, total // 2 + 3, total - 1, total}):
        want_n, want_nib = _reference_truncated_decode(words_h, offs_h, n, d, cut)
        got_n, got_nib = gpu.qsgd_elias_decode(dev(words_h[:cut]), offs_d, n, d)
        assert np.array_equal(host(got_n).view(np.uint32), want_n), (d, cut)
        assert np.array_equal(host(got_nib), want_nib), (d, cut)
