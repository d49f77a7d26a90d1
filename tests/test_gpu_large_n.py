"""Element counts past 2^32 (64-bit indexing) on the GPU, against the CPU
oracle on slices around the 2^32 boundary and the ragged tail.

n = 2^32 + 37: the 2-bit quantizer's packed word 2^28 starts at element
2^32 and the last word holds 5 codes; the reduce over two workers'
buffers; the fused CD-SGD update; QSGD with d = 512 (bucket 2^23 starts at
element 2^32, the last bucket holds 37 elements), its dequant, the
two-worker average (L2 and max-norm messages) and the Elias coding; the
SAPS mask, gather and merge (the last mask word holds 5 bits).  Each
test needs up to about 50 GiB of device memory and frees it before
returning.  n = 2^34 + 4099 takes the uniforms' Philox counter past a
change of its high word (QSGD and the SAPS mask, about 73 GiB)."""
import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.gpu

N = (1 << 32) + 37
EDGE = 1 << 32


def say(*a):
    print("[gpu]", *a, flush=True)


def host(t):
    a = t.detach().cpu().numpy()
    return a.view(np.uint32) if a.dtype == np.int32 else a


def bits(a):
    return np.ascontiguousarray(a).view(np.uint32)


def windows(n, align):
    """[lo, hi) slices with lo a multiple of `align`: the start, both sides
    of 2^32 and the ragged end."""
    out = []
    for lo in (0, EDGE - 4 * align, EDGE - align, n - (n % align) - align):
        lo -= lo % align
        out.append((lo, min(n, lo + 8 * align)))
    return out


def _free():
    import torch

    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def test_gc2_quantize_past_2_32(gpu):
    import torch

    say("gc2 n", N)
    t = 0.01
    g = torch.empty(N, device="cuda").normal_(0.0, 0.01, generator=torch.Generator("cuda").manual_seed(3))
    r = torch.empty(N, device="cuda").uniform_(-0.005, 0.005, generator=torch.Generator("cuda").manual_seed(4))
    win = windows(N, 16)
    g_h = [host(g[lo:hi]) for lo, hi in win]
    r_h = [host(r[lo:hi]).copy() for lo, hi in win]
    words = gpu.gc2_quantize(g, r, t)
    torch.cuda.synchronize()
    assert words.numel() == (N + 15) // 16
    for (lo, hi), gh, rh in zip(win, g_h, r_h):
        want = oracle.gc2_quantize(gh, rh, t)
        assert np.array_equal(host(words[lo // 16:(hi + 15) // 16]), want), lo
        assert np.array_equal(bits(host(r[lo:hi])), bits(rh)), lo
    del g, r, words
    _free()


def test_gc2_dequant_reduce_past_2_32(gpu):
    import torch

    say("dequant-reduce n", N)
    t = 0.01
    nw = (N + 15) // 16
    gen = torch.Generator("cuda").manual_seed(5)
    words = [torch.randint(-(1 << 31), 1 << 31, (nw,), dtype=torch.int64, device="cuda",
                           generator=gen).to(torch.int32) for _ in range(2)]
    # zero the tail word's unused fields, as the quantizer leaves them
    for w in words:
        w[-1] = w[-1] & ~((1 << 2 * (16 - N % 16)) - 1)
    acc = gpu.gc2_dequant_reduce(words, N, t)
    torch.cuda.synchronize()
    for lo, hi in windows(N, 16):
        wl_h = [host(w[lo // 16:(hi + 15) // 16]).copy() for w in words]
        want = oracle.gc2_dequant_reduce(wl_h, hi - lo, t)
        assert np.array_equal(bits(host(acc[lo:hi])), bits(want)), lo
    del words, acc
    _free()


def test_qsgd_past_2_32(gpu):
    import torch

    say("qsgd n", N)
    d, s, seed = 512, 7, 0x5EED
    g = torch.empty(N, device="cuda").normal_(0.0, 0.01, generator=torch.Generator("cuda").manual_seed(6))
    norms, nib = gpu.qsgd_quantize(g, d, s, seed)
    out = gpu.qsgd_dequant(norms, nib, N, d, s)
    torch.cuda.synchronize()
    assert norms.numel() == (N + d - 1) // d and nib.numel() == (N + 7) // 8
    for lo, hi in windows(N, d):
        gh = host(g[lo:hi])
        nb_lo, nb_hi = lo // d, (hi + d - 1) // d
        got_norms = host(norms[nb_lo:nb_hi])
        np.testing.assert_allclose(got_norms, oracle.qsgd_norms(gh, d), rtol=1e-6)
        want_nib = oracle.qsgd_levels(gh, d, s, seed, got_norms, index_base=lo)
        assert np.array_equal(host(nib[lo // 8:(hi + 7) // 8]), want_nib), lo
        want_out = oracle.qsgd_dequant(got_norms, want_nib, hi - lo, d, s)
        assert np.array_equal(bits(host(out[lo:hi])), bits(want_out)), lo
    del g, norms, nib, out
    _free()


def test_cdsgd_update_quantize_past_2_32(gpu):
    import torch

    say("cdsgd n", N)
    t, eta = 0.01, 0.1
    g = torch.empty(N, device="cuda").normal_(0.0, 0.01, generator=torch.Generator("cuda").manual_seed(7))
    r = torch.zeros(N, device="cuda")
    w = torch.empty(N, device="cuda").normal_(0.0, 0.05, generator=torch.Generator("cuda").manual_seed(8))
    win = windows(N, 16)
    snap = [(host(g[lo:hi]), host(r[lo:hi]).copy(), host(w[lo:hi]).copy()) for lo, hi in win]
    words = gpu.cdsgd_update_quantize(g, r, w, t, eta)
    torch.cuda.synchronize()
    for (lo, hi), (gh, rh, wh) in zip(win, snap):
        want = oracle.cdsgd_update_quantize(gh, rh, wh, t, eta)
        assert np.array_equal(host(words[lo // 16:(hi + 15) // 16]), want), lo
        assert np.array_equal(bits(host(r[lo:hi])), bits(rh)), lo
        assert np.array_equal(bits(host(w[lo:hi])), bits(wh)), lo
    del g, r, w, words
    _free()


def test_qsgd_average_past_2_32(gpu):
    import torch

    say("qsgd average n", N)
    d, s = 512, 7
    g = torch.empty(N, device="cuda").normal_(0.0, 0.01, generator=torch.Generator("cuda").manual_seed(9))
    msgs = [gpu.qsgd_quantize(g, d, s, 100 + k, maxnorm=(k == 1)) for k in range(2)]
    del g
    out = gpu.qsgd_dequant_average([m[0] for m in msgs], [m[1] for m in msgs], N, d, s)
    torch.cuda.synchronize()
    for lo, hi in windows(N, d):
        sc = [host(m[0][lo // d:(hi + d - 1) // d]) for m in msgs]
        nb = [host(m[1][lo // 8:(hi + 7) // 8]) for m in msgs]
        want = oracle.qsgd_dequant_average(sc, nb, hi - lo, d, s)
        assert np.array_equal(bits(host(out[lo:hi])), bits(want)), lo
    del msgs, out
    _free()


def _bits(words, lo, hi):
    w = np.ascontiguousarray(words).astype(">u4").view(np.uint8)
    return np.unpackbits(w)[lo:hi]


def test_elias_past_2_32(gpu):
    """Encode and decode of 2^32 + 37 elements (8,388,609 buckets, the last
    holding 37): the buckets around element 2^32 and the ragged last ones,
    each against the oracle coding it alone (bit length and bits at the
    GPU's offset), and their decode against the oracle's."""
    import torch

    say("elias n", N)
    d, s = 512, 7
    g = torch.empty(N, device="cuda").normal_(0.0, 0.01, generator=torch.Generator("cuda").manual_seed(10))
    norms, nib = gpu.qsgd_quantize(g, d, s, 0xE1)
    del g
    offs, words = gpu.qsgd_elias_encode(norms, nib, N, d)
    norms2, nib2 = gpu.qsgd_elias_decode(words, offs, N, d)
    torch.cuda.synchronize()
    o = host(offs).astype(np.int64)
    nbk = (N + d - 1) // d
    assert nbk - 1 == EDGE // d                    # the ragged last bucket starts at 2^32
    for b in [0, 1, EDGE // d - 3, EDGE // d - 2, EDGE // d - 1, nbk - 1]:
        blen = min(d, N - b * d)
        nm = host(norms[b:b + 1])
        nb = host(nib[b * d // 8:(b * d + blen + 7) // 8])
        oh, wh = oracle.qsgd_elias_encode(nm, nb, blen, d)
        assert o[b + 1] - o[b] == int(oh[-1]), b
        w0 = o[b] // 32
        got = _bits(host(words[w0:(o[b + 1] + 31) // 32 + 1]), o[b] - 32 * w0, o[b + 1] - 32 * w0)
        assert np.array_equal(got, _bits(wh, 0, int(oh[-1]))), b
        assert host(norms2[b:b + 1]).view(np.uint32)[0] == nm.view(np.uint32)[0], b
        _, want_nib = oracle.qsgd_elias_decode(wh, oh, blen, d)
        assert np.array_equal(host(nib2[b * d // 8:(b * d + blen + 7) // 8]), want_nib), b
    del norms, nib, offs, words, norms2, nib2
    _free()


_POP8 = np.array([bin(i).count("1") for i in range(256)], dtype=np.uint8)


def _popcount(words_u32):
    return int(_POP8[np.ascontiguousarray(words_u32).view(np.uint8)].sum(dtype=np.int64))


def test_saps_past_2_32(gpu):
    """Mask (bit j of word w = element 32 w + j), kept total, gather and
    merge for 2^32 + 37 elements: mask bits around element 2^32 and in the
    5-bit last word against the oracle's keep rule, the total against the
    mask's popcount, and the gathered and merged values of the kept
    elements there at their ranks."""
    import torch

    say("saps n", N)
    c, seed = 100.0, 0x5A95
    x = torch.empty(N, device="cuda").normal_(0.0, 1.0, generator=torch.Generator("cuda").manual_seed(11))
    mask, offs = gpu.saps_mask(N, c, seed)
    total = gpu.saps_count(offs)
    mask_h = host(mask)
    assert mask_h.size == (N + 31) // 32
    assert total == _popcount(mask_h)
    vals = gpu.saps_gather(x, mask, offs)
    peer = torch.remainder(torch.arange(total, device="cuda"), 1024).to(torch.float32)  # exact
    wins = [(EDGE - 4096, EDGE + 4096), (N - 37 - 2048, N)]
    x_old = [host(x[lo:hi]).copy() for lo, hi in wins]
    gpu.saps_merge(x, mask, offs, peer)
    torch.cuda.synchronize()
    for (lo, hi), xo in zip(wins, x_old):
        hi = min(hi, N)
        keep = oracle.saps_keep(seed, hi - lo, c, start=lo)
        bits_gpu = (mask_h[(np.arange(lo, hi) // 32)] >> (np.arange(lo, hi) % 32).astype(np.uint32)) & 1
        assert np.array_equal(bits_gpu.astype(bool), keep), lo
        rank0 = _popcount(mask_h[:lo // 32])        # lo is a multiple of 32
        k = int(keep.sum())
        assert np.array_equal(bits(host(vals[rank0:rank0 + k])), bits(xo[keep])), lo
        want = xo.copy()
        want[keep] = (xo[keep] + (np.arange(rank0, rank0 + k) % 1024).astype(np.float32)) * np.float32(0.5)
        assert np.array_equal(bits(host(x[lo:hi])), bits(want)), lo
    del x, mask, offs, vals, peer
    _free()


# Past 2^34 elements the Philox counter q = i / 4 of the QSGD uniforms and
# the SAPS mask has a non-zero high word: n = 2^34 + 4099 crosses that
# boundary (high word 1 from element 2^34 on) and ends ragged (the last QSGD
# bucket holds 3 elements, the last mask word 3 bits).
N34 = (1 << 34) + 4099
EDGE34 = 1 << 34


def windows34(n, align):
    out = []
    for lo in (0, EDGE34 - 4 * align, EDGE34 - align, n - (n % align) - align):
        lo -= lo % align
        out.append((lo, min(n, lo + 8 * align)))
    return out


def test_qsgd_past_2_34(gpu):
    """QSGD d = 512 (L2 and max-norm) for 2^34 + 4099 elements: norms,
    nibbles at their global indices on both sides of element 2^34 and in
    the ragged tail, against the oracle (about 73 GiB of device memory)."""
    import torch

    say("qsgd n", N34)
    d, s, seed = 512, 7, 0x5EED34
    g = torch.empty(N34, device="cuda").normal_(0.0, 0.01, generator=torch.Generator("cuda").manual_seed(16))
    for maxnorm in (False, True):
        norms, nib = gpu.qsgd_quantize(g, d, s, seed, maxnorm=maxnorm)
        torch.cuda.synchronize()
        for lo, hi in windows34(N34, d):
            gh = host(g[lo:hi])
            got = host(norms[lo // d:(hi + d - 1) // d])
            if maxnorm:
                assert np.array_equal(bits(got), bits(oracle.qsgd_maxnorms(gh, d))), lo
            else:
                np.testing.assert_allclose(got, oracle.qsgd_norms(gh, d), rtol=1e-6)
            want = oracle.qsgd_levels(gh, d, s, seed, got, index_base=lo)
            assert np.array_equal(host(nib[lo // 8:(hi + 7) // 8]), want), (maxnorm, lo)
        del norms, nib
        _free()
    del g
    _free()


def test_saps_mask_past_2_34(gpu):
    """The SAPS mask for 2^34 + 4099 elements: mask bits on both sides of
    element 2^34 and in the 3-bit last word against the oracle's keep rule,
    the tile offsets there, and the total against the mask's popcount."""
    import torch

    say("saps mask n", N34)
    c, seed = 100.0, 0x5A9534
    mask, offs = gpu.saps_mask(N34, c, seed)
    total = gpu.saps_count(offs)
    mask_h = host(mask)
    assert mask_h.size == (N34 + 31) // 32
    assert total == _popcount(mask_h)
    offs_h = host(offs).view(np.int64)
    for lo, hi in ((EDGE34 - 16384, N34 - 3), (N34 - 4099, N34)):
        keep = oracle.saps_keep(seed, hi - lo, c, start=lo)
        got = (mask_h[np.arange(lo, hi) // 32] >> (np.arange(lo, hi) % 32).astype(np.uint32)) & 1
        assert np.array_equal(got.astype(bool), keep), lo
        t0 = lo // 8192                 # lo is a multiple of 8192: offs[t0] = kept before lo
        assert offs_h[t0] == _popcount(mask_h[:lo // 32]), lo
    del mask, offs
    _free()
