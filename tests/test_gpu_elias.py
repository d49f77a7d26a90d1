"""GPU parity of the Elias-omega coding of QSGD buckets (qsgd_elias_encode,
qsgd_elias_decode) against the CPU oracle, bit-exact: bit offsets, coded
words, decoded norms and nibbles.

QSGD summary (chapterpal), Knowl 2; the omega code of P. Elias (1975)."""
import numpy as np
import pytest

import oracle
from gradient_compression_distributed_amd import workloads as wl

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


def _bits(words, lo, hi):
    w = np.ascontiguousarray(words).astype(">u4").view(np.uint8)
    return np.unpackbits(w)[lo:hi]


def test_full_size_sampled(gpu):
    """2^30 elements, d = 512, s = 7 (the launches the benchmark times):
    sampled buckets' lengths and bits against the oracle coding them alone,
    and the decode of sampled buckets."""
    import torch

    n, d, s = 1 << 30, 512, 7
    say("elias full size", n)
    cfg = wl.CONFIGS[5]
    g = torch.empty(n, device="cuda")
    wl.fill_bucketed_normal_(g, cfg, 0)
    norms, nib = gpu.qsgd_quantize(g, d, s, wl.qsgd_seed(3))
    del g
    offs, words = gpu.qsgd_elias_encode(norms, nib, n, d)
    norms2, nib2 = gpu.qsgd_elias_decode(words, offs, n, d)
    torch.cuda.synchronize()
    o = host(offs).astype(np.int64)
    say("coded bits per element", o[-1] / n)
    rs = np.random.default_rng(113)
    nbk = n // d
    for b in sorted(set([0, nbk - 1] + [int(x) for x in rs.integers(0, nbk, 30)])):
        nm = host(norms[b:b + 1])
        nb = host(nib[b * d // 8:(b + 1) * d // 8])
        oh, wh = oracle.qsgd_elias_encode(nm, nb, d, d)
        assert o[b + 1] - o[b] == int(oh[-1]), b
        w0 = o[b] // 32
        got = _bits(host(words[w0:(o[b + 1] + 31) // 32 + 1]), o[b] - 32 * w0,
                    o[b + 1] - 32 * w0)
        assert np.array_equal(got, _bits(wh, 0, int(oh[-1]))), b
        assert host(norms2[b:b + 1]).view(np.uint32)[0] == nm.view(np.uint32)[0]
        assert np.array_equal(host(nib2[b * d // 8:(b + 1) * d // 8]), clear_zero_level_signs(nb))
