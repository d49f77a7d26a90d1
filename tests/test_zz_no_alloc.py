"""gc2_quantize_buckets_noalloc, the fused 2-bit quantizer for callers that
cannot allocate (its descriptor table is a fixed device array of the
library), called through the C ABI and compared bit for bit with
gc2_quantize_buckets on the same inputs, and with the oracle.

Two calls in a row on one stream, the second with fewer and smaller
buckets than the first, so the second runs on a table the first left
behind; then the first list again."""
import ctypes

import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.gpu


def say(*a):
    print("[gpu]", *a, flush=True)


def _dev(a):
    import torch

    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _host_u32(t):
    a = t.detach().cpu().numpy()
    return a.view(np.uint32) if a.dtype == np.int32 else a


def _bits(a):
    return np.ascontiguousarray(a).view(np.uint32)


GUARD = 0x5A5A5A5A


def _case(gpu, rs, sizes, t):
    """Inputs of one call, twice over: (g, r, out) for the existing entry
    point and for the no-alloc one, with guard words after every output."""
    import torch

    gs = [(rs.standard_normal(n) * 0.03).astype(np.float32) for n in sizes]
    r0 = [(rs.standard_normal(n) * 0.005).astype(np.float32) for n in sizes]
    g_d = [_dev(a) for a in gs]
    sides = []
    for _ in range(2):
        r_d = [_dev(a.copy()) for a in r0]
        o_d = [torch.full((oracle.packed_words(n) + 4,), GUARD, dtype=torch.int32, device="cuda")
               for n in sizes]
        bl = gpu.BucketList([(g_d[i], r_d[i], o_d[i][:oracle.packed_words(n)], t)
                             for i, n in enumerate(sizes)])
        sides.append((bl, r_d, o_d))
    return gs, [a.copy() for a in r0], g_d, sides


def _call(lib, name, bl):
    import torch

    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rc = getattr(lib, name)(bl.array, bl.count, stream)
    assert rc == 0, (name, rc)


def test_noalloc_matches_fused_entry_point_on_consecutive_calls(gpu):
    import torch

    lib = gpu.load()
    rs = np.random.default_rng(2024)
    t = 0.02
    big = [int(x) for x in rs.integers(1, 40_000, 300)]
    big[7] = big[150] = 0                        # empty buckets in the list
    big[20] = 4096 * 3                           # whole tiles only
    small = [int(x) for x in rs.integers(1, 3000, 5)]
    say("no-alloc fused quantizer:", len(big), "then", len(small), "then", len(big), "buckets")
    cases = [_case(gpu, rs, big, t), _case(gpu, rs, small, t)]
    # call 1 (300 buckets), call 2 (5 buckets), call 1's list again: all
    # queued on one stream with no synchronization in between
    order = [0, 1, 0]
    for k in order:
        _, _, _, sides = cases[k]
        _call(lib, "gc2_quantize_buckets", sides[0][0])
        _call(lib, "gc2_quantize_buckets_noalloc", sides[1][0])
    torch.cuda.synchronize()
    for k in (0, 1):
        gs, r_h, _, sides = cases[k]
        steps = order.count(k)
        for _ in range(steps):
            want = [oracle.gc2_quantize(gs[i], r_h[i], t) for i in range(len(gs))]
        (_, ra, oa), (_, rb, ob) = sides
        for i in range(len(gs)):
            a, b = _host_u32(oa[i]), _host_u32(ob[i])
            nw = want[i].size
            assert np.array_equal(b, a), (k, i)                  # no-alloc == existing entry point
            assert np.array_equal(b[:nw], want[i]), (k, i)       # and == the oracle
            assert np.all(b[nw:] == GUARD), (k, i)
            assert np.array_equal(_bits(_host_u32(rb[i])), _bits(_host_u32(ra[i]))), (k, i)
            assert np.array_equal(_bits(_host_u32(rb[i])), _bits(r_h[i])), (k, i)


def test_noalloc_rejects_more_buckets_than_its_table(gpu):
    lib = gpu.load()
    assert gpu.GC2_NOALLOC_MAX_BUCKETS == 4096
    n = gpu.GC2_NOALLOC_MAX_BUCKETS + 1
    arr = (gpu.Gc2Bucket * n)()
    for i in range(n):          # valid-looking, disjoint fake buckets: only the count is wrong
        arr[i] = gpu.Gc2Bucket(0x7F0000000000 + 3 * i * 4096, 0x7F0000000000 + (3 * i + 1) * 4096,
                               0x7F0000000000 + (3 * i + 2) * 4096, 16, 0.5)
    assert lib.gc2_quantize_buckets_noalloc(arr, n, ctypes.c_void_p(0)) == -3
