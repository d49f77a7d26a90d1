"""GPU parity of gc2_dequant_reduce against the CPU oracle, bit-exact.

MXNet PR "2bit gradient compression", "Local kvstore": device 0
dequantizes the W devices' packed gradients and sums them; CD-SGD 3.4.1:
11 -> +t, 10 -> -t.  The sum is taken in worker order 0..W-1."""
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


def bits(a):
    return np.ascontiguousarray(a).view(np.uint32)


def test_w16_resnet50_sized(gpu):
    cfg = wl.REDUCE_W16_RESNET50
    say("dequant W = 16 ResNet-50-sized", cfg.n, cfg.workers)
    nw = oracle.packed_words(cfg.n)
    ws = [wl.worker_words(cfg, w, nw) for w in range(cfg.workers)]
    acc_d = gpu.gc2_dequant_reduce([dev(w) for w in ws], cfg.n, cfg.t)
    acc_h = oracle.gc2_dequant_reduce(ws, cfg.n, cfg.t)
    assert np.array_equal(bits(host(acc_d)), bits(acc_h))


DQ_VARIANTS = [dict(dq_nt_loads=l, dq_nt_stores=s, dq_lds_stores=d, dq_blocks_per_cu=b,
                    dq_fp4_decode=f, dq_words_per_thread=k, dq_resident_per_cu=c)
               for (l, s, d, b, f, k, c) in [(1, 1, 1, 0, 1, 1, 2), (1, 0, 0, 0, 1, 1, 0),
                                             (0, 1, 1, 4, 0, 1, 3), (0, 0, 0, 2, 1, 1, 2),
                                             (1, 1, 0, 0, 0, 1, 8), (0, 0, 1, 1, 1, 1, 0),
                                             (1, 1, 1, 8, 0, 1, 2), (0, 1, 0, 0, 1, 1, 4),
                                             (1, 1, 1, 0, 1, 2, 2), (0, 0, 1, 3, 0, 2, 0),
                                             (1, 0, 1, 0, 1, 2, 3), (0, 1, 1, 0, 0, 2, 8),
                                             (1, 1, 1, 0, 1, 2, 0), (1, 1, 1, 2, 1, 2, 2),
                                             (1, 1, 1, 0, 1, 0, 3)]]


@pytest.mark.parametrize("var", range(len(DQ_VARIANTS)))
def test_workers_sizes_thresholds(gpu, var):
    import torch

    old = gpu.set_tuning(**DQ_VARIANTS[var])
    try:
        rs = np.random.default_rng(21 + var)
        for W in (1, 2, 3, 7, 15, 16, 17, 31, 33, 64):
            for n in (1, 15, 16, 17, 63, 4095, 4096, 4097, 8192, 100_003):
                # t = 1e-37 exercises the path for thresholds below 2^-120
                t = float(rs.choice([0.01, 1e-3, 0.5, 0.1, 7.7, 1e-37]))
                say("dequant W", W, "n", n, "t", t)
                nw = oracle.packed_words(n)
                ws = [wl.iid_field_words(rs, nw, 0.3, 0.3) for _ in range(W)]
                # sprinkle the never-produced code 01 (read as zero)
                ws[0][: max(1, nw // 3)] |= np.uint32(0x11111111)
                ws[0][: max(1, nw // 3)] &= np.uint32(~0x22222222 & 0xFFFFFFFF)
                guard = torch.full((n + 64,), 1234.5, device="cuda")
                gpu.gc2_dequant_reduce([dev(w) for w in ws], n, t, acc=guard[:n])
                acc_h = oracle.gc2_dequant_reduce(ws, n, t)
                out = host(guard)
                assert np.array_equal(bits(out[:n]), bits(acc_h)), (W, n, t)
                assert np.all(out[n:] == np.float32(1234.5))
    finally:
        gpu.set_tuning(**old)


def test_aliased_workers(gpu):
    say("dequant aliased workers")
    n = 10_000
    w = wl.iid_field_words(np.random.default_rng(4), oracle.packed_words(n), 0.4, 0.4)
    d = dev(w)
    acc = gpu.gc2_dequant_reduce([d, d, d, d, d], n, 1e-3)
    assert np.array_equal(bits(host(acc)), bits(oracle.gc2_dequant_reduce([w] * 5, n, 1e-3)))


def test_roundtrip_with_gpu_quantizer(gpu):
    # W workers quantize their own gradients on the GPU, the reduce sums
    # them; compared with the oracle doing both steps
    import torch

    say("dequant roundtrip")
    n, W, t = 200_001, 8, 0.01
    rs = np.random.default_rng(12)
    gs = [(rs.standard_normal(n) * 0.01).astype(np.float32) for _ in range(W)]
    words_d, words_h = [], []
    for g in gs:
        r_d = torch.zeros(n, device="cuda")
        words_d.append(gpu.gc2_quantize(dev(g), r_d, t))
        words_h.append(oracle.gc2_quantize(g, np.zeros(n, np.float32), t))
    acc = gpu.gc2_dequant_reduce(words_d, n, t)
    assert np.array_equal(bits(host(acc)), bits(oracle.gc2_dequant_reduce(words_h, n, t)))


def test_probes_compute_what_they_state(gpu):
    # the measurement probes keep every load and store (their outputs are
    # defined): the reduce probe's acc[16 i] is the XOR of the workers'
    # word i and its other sums +0; the stream probe's c is a XOR b and its
    # word 16k + L the bits of c[256k + 4L]
    import torch

    say("probes")
    rs = np.random.default_rng(41)
    for n, W in ((16 * 4096 + 7, 16), (1 << 20, 5)):
        nw = oracle.packed_words(n)
        ws = [rs.integers(0, 1 << 32, nw, dtype=np.uint64).astype(np.uint32) for _ in range(W)]
        acc = torch.full((n,), 3.0, device="cuda")
        gpu.probe_reduce([dev(w) for w in ws], n, acc)
        got = host(acc).view(np.uint32)
        x = np.bitwise_xor.reduce(np.stack(ws), axis=0)
        want = np.zeros(nw * 16, np.uint32)
        want[::16] = x
        assert np.array_equal(got, want[:n]), (n, W)
    n = 1 << 20
    a = dev(rs.integers(0, 1 << 32, n, dtype=np.uint64).astype(np.uint32)).view(torch.float32)
    b = dev(rs.integers(0, 1 << 32, n, dtype=np.uint64).astype(np.uint32)).view(torch.float32)
    c = torch.empty(n, device="cuda")
    words = torch.empty(n // 16, dtype=torch.int32, device="cuda")
    gpu.probe_stream(a, c, b=b, words=words)
    ah, bh, ch = (host(t).view(np.uint32) for t in (a, b, c))
    assert np.array_equal(ch, ah ^ bh)
    k = np.arange(n // 16)
    assert np.array_equal(host(words), ch[(k // 16) * 256 + 4 * (k % 16)])
    gpu.probe_stream(a, c)
    assert np.array_equal(host(c).view(np.uint32), ah)
    gpu.probe_stream(a, b, b=b, words=words)          # in place, as the quantizer updates r
    assert np.array_equal(host(b).view(np.uint32), ah ^ bh)
