"""GPU parity of the QSGD widenings against the CPU oracle: max-norm bucket
scales (qsgd_quantize_maxnorm) and the K-worker decode-average
(qsgd_dequant_average).

QSGD summary (chapterpal): Knowl 8 (max-norm scaling), Knowl 3 (decode
every peer's message and average).  The max is exact, so scales, levels and
signs are compared bit for bit; the average is bit-exact too (the same
float32 operations in the same order), with NaNs compared by position
(IEEE 754 leaves the sign and payload of a generated NaN to the platform)."""
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


def fbits(a):
    a = np.ascontiguousarray(a)
    b = a.view(np.uint32).copy()
    b[np.isnan(a)] = 0x7FC00000
    return b


@pytest.fixture
def knobs(gpu):
    old = gpu.get_tuning()
    yield gpu
    gpu.set_tuning(**old)


def check_maxnorm(gpu, g, d, s, seed):
    sc_d, nib_d = gpu.qsgd_quantize_maxnorm(dev(g), d, s, seed)
    sc_h, nib_h = oracle.qsgd_quantize_maxnorm(g, d, s, seed)
    assert np.array_equal(fbits(host(sc_d)), fbits(sc_h)), (g.size, d, s)
    assert np.array_equal(host(nib_d), nib_h), (g.size, d, s)
    return sc_d, nib_d


# ---------------------------------------------------------------- max-norm
@pytest.mark.parametrize("rcp,bpc", [(1, 32), (0, 0), (1, 0)])
def test_maxnorm_alexnet_sized(knobs, rcp, bpc):
    gpu = knobs
    gpu.set_tuning(qsgd_rcp=rcp, qsgd_blocks_per_cu=bpc)
    cfg = wl.QSGD_ALEXNET
    say("qsgd max-norm AlexNet-sized", cfg.n, "rcp", rcp, "blocks/CU", bpc)
    check_maxnorm(gpu, wl.gradient(cfg, 0), cfg.d, cfg.s, wl.qsgd_seed(0))


@pytest.mark.parametrize("d", [1, 7, 64, 256, 512, 1000, 1024, 2048, 4096])
def test_maxnorm_bucket_sizes_and_levels(gpu, d):
    say("qsgd max-norm d", d)
    for n in (1, d - 1 if d > 1 else 1, d, 3 * d + 5, 70_001):
        g = wl.qsgd_spiky(n, d, 7 + n)
        for s in (1, 3, 7):
            check_maxnorm(gpu, g, d, s, 1000 * d + n + s)


@pytest.mark.parametrize("rcp", [1, 0])
def test_maxnorm_special_values(knobs, rcp):
    gpu = knobs
    gpu.set_tuning(qsgd_rcp=rcp)
    say("qsgd max-norm specials rcp", rcp)
    rs = np.random.default_rng(80)
    d = 512
    g = (rs.standard_normal(d * 40) * 0.01).astype(np.float32)
    g[0:d] = 0.0                                   # zero bucket
    g[d:2 * d] = -0.0
    g[2 * d + 5] = np.nan                          # a NaN does not become the scale
    g[3 * d + 7] = np.inf
    g[4 * d + 9] = -np.inf
    g[5 * d:6 * d] = np.float32(0.25)              # constant bucket: every level s
    g[6 * d + 1] = np.float32(1e-40)               # subnormal
    g[7 * d:8 * d] = (rs.standard_normal(d) * 1e-38).astype(np.float32)
    g[8 * d:9 * d] = (rs.standard_normal(d) * 1e37).astype(np.float32)
    g[9 * d + 3] = np.nan
    g[9 * d + 4] = np.float32(-np.nan)
    for s in (1, 7):
        check_maxnorm(gpu, g, d, s, 55 + s)


def test_maxnorm_dequant_round_trip(gpu):
    rs = np.random.default_rng(81)
    g = (rs.standard_normal(1 << 20) * 0.02).astype(np.float32)
    sc_d, nib_d = check_maxnorm(gpu, g, 512, 7, 3)
    out = host(gpu.qsgd_dequant(sc_d, nib_d, g.size, 512, 7))
    want = oracle.qsgd_dequant(host(sc_d), host(nib_d), g.size, 512, 7)
    assert np.array_equal(fbits(out), fbits(want))


# ----------------------------------------------------- K-way decode-average
def _messages(gpu, K, n, d, s, seed0, maxnorm=False, sigma=0.02):
    rs = np.random.default_rng(seed0)
    scales, nibs = [], []
    for k in range(K):
        g = (rs.standard_normal(n) * sigma).astype(np.float32)
        sc, nb = gpu.qsgd_quantize(dev(g), d, s, seed0 * 100 + k, maxnorm=maxnorm)
        scales.append(sc)
        nibs.append(nb)
    return scales, nibs


def check_average(gpu, scales, nibs, n, d, s):
    out = gpu.qsgd_dequant_average(scales, nibs, n, d, s)
    want = oracle.qsgd_dequant_average([host(x) for x in scales], [host(x) for x in nibs],
                                       n, d, s)
    assert np.array_equal(fbits(host(out)), fbits(want)), (len(scales), n, d, s)
    return out


@pytest.mark.parametrize("K", [1, 2, 3, 4, 5, 6, 7, 8, 9, 12, 16, 22, 24, 31, 64])
def test_average_workers(knobs, K):
    gpu = knobs
    say("qsgd average K", K)
    for dbpc, nt, cap in ((0, 1, 0), (3, 0, 2), (0, 1, 5)):
        gpu.set_tuning(qsgd_dequant_blocks_per_cu=dbpc, qsgd_dequant_nt=nt,
                       qsgd_avg_resident_per_cu=cap)
        for n, d in ((2048, 512), (2049, 512), (100_003, 512), (65_536 + 17, 256), (10_000, 1000),
                     (50_000, 4096), (9_000, 64), (777, 1), (20_000, 255), (30_000, 341),
                     (30_000, 340)):
            scales, nibs = _messages(gpu, K, n, d, 7, K * 31 + n % 97, maxnorm=(n % 2 == 1))
            check_average(gpu, scales, nibs, n, d, 7)


def test_average_ragged_and_tiny(gpu):
    say("qsgd average ragged sizes")
    for n in list(range(1, 40)) + [2047, 2048, 2049, 4095, 4097, 6144 + 3]:
        for d in (256, 512, 3):
            scales, nibs = _messages(gpu, 3, n, d, 5, n)
            check_average(gpu, scales, nibs, n, d, 5)


def test_average_specials(gpu):
    # random nibbles (every sign/level pattern) with zero, subnormal, huge and
    # infinite scales: decoded +-inf, inf*0 = NaN and overflowing sums
    import torch

    say("qsgd average specials")
    rs = np.random.default_rng(82)
    K, n, d, s = 4, 5 * 2048 + 11, 512, 7
    nb = oracle.num_buckets(n, d)
    scales, nibs = [], []
    for k in range(K):
        sc = (rs.uniform(0, 1, nb) * 10.0 ** rs.uniform(-3, 3, nb)).astype(np.float32)
        sc[k] = 0.0
        sc[4 + k] = np.float32(1e-41)
        sc[8 + k] = np.float32(3e38)
        if k < 2:
            sc[12] = np.inf
        scales.append(dev(sc))
        nibs.append(dev(rs.integers(0, 1 << 32, oracle.nibble_words(n), dtype=np.uint64)
                        .astype(np.uint32)))
    check_average(gpu, scales, nibs, n, d, s)
    torch.cuda.synchronize()
