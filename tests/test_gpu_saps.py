"""GPU parity of the SAPS sparsification (saps_mask, saps_gather, saps_merge)
against the CPU oracle, bit-exact: mask words, tile offsets and total count,
gathered values, merged vectors.

"Communication-Efficient Decentralized Learning with Sparsification and
Adaptive Peer Selection": the shared-seed Bernoulli(1/c) mask, only the kept
components exchanged, single-peer gossip."""
import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.gpu

TILE = 8192


def say(*a):
    print("[gpu]", *a, flush=True)


def dev(a):
    import torch

    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    a = t.detach().cpu().numpy()
    return a.view(np.uint32) if a.dtype == np.int32 else a


def fbits(a):
    a = np.ascontiguousarray(a)
    b = a.view(np.uint32).copy()
    b[np.isnan(a)] = 0x7FC00000
    return b


def oracle_mask(n, c, seed):
    """Mask words and tile offsets from the oracle's kept indices."""
    kept = oracle.saps_gather(np.arange(n, dtype=np.float32), c, seed).astype(np.int64)
    words = np.zeros((n + 31) // 32, dtype=np.uint64)
    np.add.at(words, kept // 32, np.left_shift(np.uint64(1), (kept % 32).astype(np.uint64)))
    ntiles = (n + TILE - 1) // TILE
    counts = np.bincount(kept // TILE, minlength=ntiles)[:ntiles]
    offs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    return words.astype(np.uint32), offs, kept


def check(gpu, x, c, seed):
    import torch

    n = x.size
    mask, offs = gpu.saps_mask(n, c, seed)
    w_h, o_h, kept = oracle_mask(n, c, seed)
    assert np.array_equal(host(mask), w_h), (n, c, seed)
    assert np.array_equal(host(offs), o_h), (n, c, seed)
    total = gpu.saps_count(offs)
    assert total == kept.size
    # gather, with sentinels past the used part of the buffer
    buf = torch.full((total + 5,), 3.25, device="cuda")
    gpu.saps_gather(dev(x), mask, offs, values=buf[:total])
    vals = oracle.saps_gather(x, c, seed)
    b = host(buf)
    assert np.array_equal(fbits(b[:total]), fbits(vals)), (n, c)
    assert np.all(b[total:] == 3.25)
    # merge a peer's values
    rs = np.random.default_rng(n % 1000 + 1)
    peer = rs.standard_normal(total).astype(np.float32)
    xd = dev(x)
    gpu.saps_merge(xd, mask, offs, dev(peer))
    xh = x.copy()
    oracle.saps_merge(xh, c, seed, peer)
    assert np.array_equal(fbits(host(xd)), fbits(xh)), (n, c)
    return mask, offs


@pytest.mark.parametrize("c", [1.0, 2.0, 3.5, 100.0, 1e6, 2.0 ** 24, 1e30])
def test_ratios(gpu, c):
    say("saps c", c)
    rs = np.random.default_rng(90)
    for n in (1, 31, 32, 33, 8191, 8192, 8193, 100_003, 1_000_000):
        x = rs.standard_normal(n).astype(np.float32)
        check(gpu, x, c, 1234 + n)


def test_ragged_sizes_and_specials(gpu):
    say("saps ragged sizes")
    rs = np.random.default_rng(91)
    sp = np.array([0.0, -0.0, np.nan, np.inf, -np.inf, 1e-45, 3e38], np.float32)
    for n in list(range(0, 70)) + [TILE * 3 + 17, TILE * 16]:
        x = rs.standard_normal(n).astype(np.float32)
        m = rs.random(n) < 0.1
        x[m] = sp[rs.integers(0, sp.size, m.sum())]
        if n == 0:
            mask, offs = gpu.saps_mask(0, 4.0, 1)
            assert gpu.saps_count(offs) == 0
            continue
        check(gpu, x, 4.0, 77 + n)


def test_short_capacity_writes_only_what_fits(gpu):
    import torch

    say("saps capacity")
    n, c, seed = 200_000, 10.0, 5
    x = np.random.default_rng(92).standard_normal(n).astype(np.float32)
    mask, offs = gpu.saps_mask(n, c, seed)
    total = gpu.saps_count(offs)
    cap = total // 3
    buf = torch.full((total,), 7.5, device="cuda")
    gpu.saps_gather(dev(x), mask, offs, values=buf[:cap])
    vals = oracle.saps_gather(x, c, seed)
    b = host(buf)
    assert np.array_equal(b[:cap], vals[:cap])
    assert np.all(b[cap:] == 7.5)
    # merge with a short peer buffer: only the first cap kept components move
    xd = dev(x)
    peer = np.full(total, 1.0, np.float32)
    gpu.saps_merge(xd, mask, offs, dev(peer[:cap]))
    xh = x.copy()
    kept = oracle_mask(n, c, seed)[2]
    xh[kept[:cap]] = (xh[kept[:cap]] + np.float32(1.0)) * np.float32(0.5)
    assert np.array_equal(host(xd), xh)


def test_two_peers_agree_after_exchange(gpu):
    say("saps exchange")
    rs = np.random.default_rng(93)
    n, c, seed = 500_000, 100.0, 2026
    a, b = rs.standard_normal(n).astype(np.float32), rs.standard_normal(n).astype(np.float32)
    ad, bd = dev(a), dev(b)
    mask, offs = gpu.saps_mask(n, c, seed)
    va, vb = gpu.saps_gather(ad, mask, offs), gpu.saps_gather(bd, mask, offs)
    gpu.saps_merge(ad, mask, offs, vb)
    gpu.saps_merge(bd, mask, offs, va)
    kept = oracle_mask(n, c, seed)[2]
    ah, bh = host(ad), host(bd)
    assert np.array_equal(ah[kept], bh[kept])
    oracle.saps_merge(a, c, seed, host(vb))
    assert np.array_equal(ah, a)


def test_offsets_across_scan_chunks(gpu):
    # 9000 tiles: the offsets scan runs over more than one 8192-entry chunk,
    # the second one partial
    n, c, seed = 9000 * TILE + 5, 100.0, 31337
    say("saps offsets over", (n + TILE - 1) // TILE, "tiles")
    mask, offs = gpu.saps_mask(n, c, seed)
    # gather each element's tile number (exact in float32, unlike an index
    # past 2^24): the tiles of the kept elements, in order
    tile_of = (np.arange(n, dtype=np.int64) // TILE).astype(np.float32)
    kept_tiles = oracle.saps_gather(tile_of, c, seed).astype(np.int64)
    ntiles = (n + TILE - 1) // TILE
    counts = np.bincount(kept_tiles, minlength=ntiles)[:ntiles]
    want = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    assert np.array_equal(host(offs), want)
