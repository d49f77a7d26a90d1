"""The C ABI on the host: libgcq.so loads, exports every function that
include/gcq.h declares, and rejects invalid arguments on the host before
anything is enqueued (no device call is made by these tests: every call
here fails validation or has no work).  Fake device addresses are never
dereferenced."""
import ctypes
import os
import re

import pytest

import gradient_compression_distributed_amd as gcq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gcq.h")

OK, E_NULL, E_THR, E_PARAM, E_ALIGN, E_OVERLAP = 0, -1, -2, -3, -4, -5
A = 0x7F0000000000          # a fake, 256-byte aligned "device" address
F = ctypes.c_float
NULL = ctypes.c_void_p(0)


def vp(x):
    return ctypes.c_void_p(x)


@pytest.fixture(scope="module")
def lib():
    return gcq.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert {"gc2_quantize", "gc2_quantize_buckets", "gc2_dequant_reduce", "qsgd_quantize",
            "qsgd_dequant", "gc2_packed_words", "qsgd_num_buckets", "qsgd_nibble_words",
            "gcq_status_string"} <= set(names)
    for name in names:
        assert hasattr(lib, name), name
    out = os.popen(f"nm -D --defined-only {gcq.lib_path()}").read()
    for name in names:
        assert re.search(rf"\bT {name}$", out, flags=re.M), name


def test_sizes(lib):
    for n, w in [(0, 0), (1, 1), (16, 1), (17, 2), (65_541, 4_097), (25_557_032, 1_597_315),
                 (1 << 30, 67_108_864)]:
        assert lib.gc2_packed_words(n) == w
    assert lib.qsgd_num_buckets(61_100_840, 512) == 119_338
    assert lib.qsgd_num_buckets(10, 0) == 0
    assert lib.qsgd_nibble_words(61_100_840) == 7_637_605
    assert lib.qsgd_nibble_words(9) == 2


def test_status_strings(lib):
    for s in range(-7, 1):
        assert lib.gcq_status_string(s)
    assert lib.gcq_status_string(-99) == b"unknown status"


def test_gc2_quantize_validation(lib):
    n = 1000
    g, r, o = A, A + (1 << 20), A + (2 << 20)
    q = lambda g_, r_, n_, t_, o_: lib.gc2_quantize(vp(g_), vp(r_), n_, F(t_), vp(o_), NULL)
    assert q(0, r, n, 0.5, o) == E_NULL
    assert q(g, 0, n, 0.5, o) == E_NULL
    assert q(g, r, n, 0.5, 0) == E_NULL
    for bad_t in (0.0, -1.0, float("inf"), float("nan")):
        assert q(g, r, n, bad_t, o) == E_THR
        assert q(g, r, 0, bad_t, o) == E_THR        # no default threshold, even for n == 0
    assert q(g + 4, r, n, 0.5, o) == E_ALIGN
    assert q(g, r + 8, n, 0.5, o) == E_ALIGN
    assert q(g, r, n, 0.5, o + 2) == E_ALIGN
    assert q(g, g, n, 0.5, o) == E_OVERLAP           # g and r alias
    assert q(g, g + 16 * 10, n, 0.5, o) == E_OVERLAP  # r starts inside g
    assert q(g, r, n, 0.5, r + 3996) == E_OVERLAP    # out over the end of r
    assert q(0, 0, 0, 0.5, 0) == OK                  # empty: no work, nothing touched


def test_gc2_buckets_validation(lib):
    def call(descs):
        arr = (gcq.Gc2Bucket * len(descs))(*[gcq.Gc2Bucket(*d) for d in descs])
        return lib.gc2_quantize_buckets(arr, len(descs), NULL)

    mb = 1 << 20
    good = lambda i, n=1000: (A + 3 * i * mb, A + (3 * i + 1) * mb, A + (3 * i + 2) * mb, n, 0.5)
    assert lib.gc2_quantize_buckets(None, 0, NULL) == OK
    assert lib.gc2_quantize_buckets(None, 3, NULL) == E_NULL
    assert call([good(0), (A + 3 * mb, A + 4 * mb, A + 5 * mb, 1000, 0.0)]) == E_THR
    assert call([good(0), (A + 3 * mb + 4, A + 4 * mb, A + 5 * mb, 1000, 0.5)]) == E_ALIGN
    # bucket 1 writes its residual over bucket 0's gradient
    assert call([good(0), (A + 3 * mb, A, A + 5 * mb, 1000, 0.5)]) == E_OVERLAP
    # bucket 1's packed output over bucket 0's packed output
    assert call([good(0), (A + 3 * mb, A + 4 * mb, A + 2 * mb + 64, 1000, 0.5)]) == E_OVERLAP
    # two buckets may read the same gradient (read-only ranges can overlap) ...
    assert call([(A, A + mb, A + 2 * mb, 0, 0.5)] * 3) == OK   # ... and empty buckets are no work
    assert call([(0, 0, 0, 0, 0.5), (0, 0, 0, 0, 0.5)]) == OK


def test_gc2_buckets_noalloc_validation(lib):
    # the entry point that allocates nothing checks exactly what
    # gc2_quantize_buckets checks, plus its table size, all before any
    # device call
    def call(descs):
        arr = (gcq.Gc2Bucket * len(descs))(*[gcq.Gc2Bucket(*d) for d in descs])
        return lib.gc2_quantize_buckets_noalloc(arr, len(descs), NULL)

    mb = 1 << 20
    good = lambda i, n=1000: (A + 3 * i * mb, A + (3 * i + 1) * mb, A + (3 * i + 2) * mb, n, 0.5)
    assert "#define GC2_NOALLOC_MAX_BUCKETS 4096" in open(HEADER).read()
    assert lib.gc2_quantize_buckets_noalloc(None, 0, NULL) == OK
    assert lib.gc2_quantize_buckets_noalloc(None, 3, NULL) == E_NULL
    assert call([good(0), (A + 3 * mb, A + 4 * mb, A + 5 * mb, 1000, 0.0)]) == E_THR
    assert call([good(0), (A + 3 * mb + 4, A + 4 * mb, A + 5 * mb, 1000, 0.5)]) == E_ALIGN
    assert call([good(0), (A + 3 * mb, A, A + 5 * mb, 1000, 0.5)]) == E_OVERLAP
    assert call([(A, A + mb, A + 2 * mb, 0, 0.5)] * 3) == OK
    assert call([good(i, 16) for i in range(4097)]) == E_PARAM
    half = (1 << 59) + 1
    assert call([(A, A + (1 << 20), A + (2 << 20), half, 0.5),
                 (A, A + (3 << 20), A + (4 << 20), half, 0.5)]) == E_PARAM


def test_probe_validation(lib):
    ps = lambda a, b, c, w, n: lib.gcq_probe_stream(vp(a), vp(b), vp(c), vp(w), n, NULL)
    mb = 1 << 20
    assert ps(A, 0, A + mb, 0, 0) == OK
    assert ps(A, 0, A + mb, 0, 1000) == E_PARAM          # not a multiple of 1024
    assert ps(0, 0, A + mb, 0, 1024) == E_NULL
    assert ps(A, 0, 0, 0, 1024) == E_NULL
    assert ps(A + 4, 0, A + mb, 0, 1024) == E_ALIGN
    assert ps(A, A + 8, A + mb, 0, 1024) == E_ALIGN
    assert ps(A, 0, A + mb, A + 2 * mb + 2, 1024) == E_ALIGN
    assert ps(A, 0, A + 64, 0, 1024) == E_OVERLAP
    assert ps(A, A + mb, A + 2 * mb, A + mb + 64, 1024) == E_OVERLAP
    # c may be b itself (in place), but not overlap it partly (the accepted
    # in-place form is exercised on a GPU, with real buffers)
    assert ps(A, A + mb, A + mb + 16, 0, 1024) == E_OVERLAP
    ws = (ctypes.c_void_p * 2)(A, A + mb)
    pr = lambda W, n, acc: lib.gcq_probe_reduce(ws, W, n, vp(acc), NULL)
    assert pr(2, 0, A + 2 * mb) == OK
    assert pr(0, 100, A + 2 * mb) == E_PARAM
    assert pr(65, 100, A + 2 * mb) == E_PARAM
    assert pr(2, 100, 0) == E_NULL
    assert pr(2, 100, A + 2 * mb + 4) == E_ALIGN
    assert pr(2, 100, A + mb) == E_OVERLAP


def test_cdsgd_validation(lib):
    n = 1000
    g, r, w, o = A, A + (1 << 20), A + (2 << 20), A + (3 << 20)
    q = lambda g_, r_, w_, n_, t_, e_, o_: lib.cdsgd_update_quantize(
        vp(g_), vp(r_), vp(w_), n_, F(t_), F(e_), vp(o_), NULL)
    assert q(g, r, 0, n, 0.5, 0.1, o) == E_NULL
    assert q(0, r, w, n, 0.5, 0.1, o) == E_NULL
    assert q(g, r, w, n, 0.0, 0.1, o) == E_THR
    for bad in (-0.1, float("nan"), float("inf")):
        assert q(g, r, w, n, 0.5, bad, o) == E_PARAM
        assert q(g, r, w, 0, 0.5, bad, o) == E_PARAM        # checked even for n == 0
    assert q(g, r, w, 0, 0.5, 0.1, o) == OK                 # n == 0 is a no-op
    assert q(g, r, w + 4, n, 0.5, 0.1, o) == E_ALIGN
    assert q(g, r, g, n, 0.5, 0.1, o) == E_OVERLAP          # w aliases comm_buf
    assert q(g, r, r + 64, n, 0.5, 0.1, o) == E_OVERLAP     # w inside r
    assert q(g, r, w, n, 0.5, 0.1, w + 128) == E_OVERLAP    # words over w
    u = lambda g_, w_, n_, e_: lib.cdsgd_local_update(vp(g_), vp(w_), n_, F(e_), NULL)
    assert u(g, 0, n, 0.1) == E_NULL
    assert u(0, w, n, 0.1) == E_NULL
    assert u(g, w, n, -1.0) == E_PARAM
    assert u(g, w, 0, float("nan")) == E_PARAM
    assert u(g, w, 0, 0.1) == OK
    assert u(g + 8, w, n, 0.1) == E_ALIGN
    assert u(g, w + 4, n, 0.1) == E_ALIGN
    assert u(g, g + 16, n, 0.1) == E_OVERLAP


def test_dequant_reduce_validation(lib):
    n = 4096
    ws = (ctypes.c_void_p * 3)(A, A + (1 << 20), A + (2 << 20))
    acc = A + (3 << 20)
    d = lambda w, W, n_, t, a: lib.gc2_dequant_reduce(w, W, n_, F(t), vp(a), NULL)
    assert d(ws, 0, n, 0.5, acc) == E_PARAM
    assert d(ws, 65, n, 0.5, acc) == E_PARAM
    assert d(ws, 3, n, -0.5, acc) == E_THR
    assert d(ws, 3, n, 0.5, 0) == E_NULL
    assert d(None, 3, n, 0.5, acc) == E_NULL
    bad = (ctypes.c_void_p * 2)(A, 0)
    assert d(bad, 2, n, 0.5, acc) == E_NULL
    mis = (ctypes.c_void_p * 2)(A, A + 2)
    assert d(mis, 2, n, 0.5, acc) == E_ALIGN
    assert d(ws, 3, n, 0.5, acc + 4) == E_ALIGN
    same = (ctypes.c_void_p * 2)(A, A)               # workers may alias each other
    assert d(same, 2, 0, 0.5, acc) == OK
    assert d(ws, 3, n, 0.5, A + (1 << 20) + 256) == E_OVERLAP


def test_qsgd_validation(lib):
    n = 5000
    g, nm, nb, out = A, A + (1 << 20), A + (2 << 20), A + (3 << 20)
    q = lambda g_, n_, d, s, nm_, nb_: lib.qsgd_quantize(vp(g_), n_, d, s, ctypes.c_uint64(1),
                                                         vp(nm_), vp(nb_), NULL)
    assert q(g, n, 0, 7, nm, nb) == E_PARAM
    assert q(g, n, 512, 0, nm, nb) == E_PARAM
    assert q(g, n, 512, 8, nm, nb) == E_PARAM
    assert q(0, n, 512, 7, nm, nb) == E_NULL
    assert q(g + 4, n, 512, 7, nm, nb) == E_ALIGN
    assert q(g, n, 512, 7, nm + 2, nb) == E_ALIGN
    assert q(g, n, 512, 7, g + 64, nb) == E_OVERLAP
    assert q(g, n, 512, 7, nm, nm + 4) == E_OVERLAP
    assert q(0, 0, 512, 7, 0, 0) == OK
    dq = lambda nm_, nb_, n_, d, s, o: lib.qsgd_dequant(vp(nm_), vp(nb_), n_, d, s, vp(o), NULL)
    assert dq(nm, nb, n, 0, 7, out) == E_PARAM
    assert dq(nm, nb, n, 512, 9, out) == E_PARAM
    assert dq(nm, 0, n, 512, 7, out) == E_NULL
    assert dq(nm, nb, n, 512, 7, out + 4) == E_ALIGN
    assert dq(nm, nb, n, 512, 7, nb) == E_OVERLAP


def test_qsgd_maxnorm_and_average_validation(lib):
    n = 1000
    g, nm, nb, out = A, A + (1 << 20), A + (2 << 20), A + (3 << 20)
    q = lambda g_, d, s: lib.qsgd_quantize_maxnorm(vp(g_), n, d, s, ctypes.c_uint64(1), vp(nm),
                                                   vp(nb), NULL)
    assert q(g, 0, 7) == E_PARAM
    assert q(g, 512, 8) == E_PARAM
    assert q(0, 512, 7) == E_NULL
    assert q(g + 4, 512, 7) == E_ALIGN
    arr = lambda xs: (ctypes.c_void_p * len(xs))(*[vp(x) for x in xs])
    sc = [A + (4 << 20) + k * (1 << 16) for k in range(3)]
    nbs = [A + (5 << 20) + k * (1 << 16) for k in range(3)]
    av = lambda s_, n_, K, d, s, o: lib.qsgd_dequant_average(s_, n_, K, n, d, s, vp(o), NULL)
    assert av(arr(sc), arr(nbs), 0, 512, 7, out) == E_PARAM
    assert av(arr(sc), arr(nbs), 65, 512, 7, out) == E_PARAM
    assert av(arr(sc), arr(nbs), 3, 0, 7, out) == E_PARAM
    assert av(arr(sc), arr(nbs), 3, 512, 0, out) == E_PARAM
    assert av(None, arr(nbs), 3, 512, 7, out) == E_NULL
    assert av(arr(sc), arr(nbs), 3, 512, 7, 0) == E_NULL
    assert av(arr([sc[0], 0, sc[2]]), arr(nbs), 3, 512, 7, out) == E_NULL
    assert av(arr(sc), arr(nbs), 3, 512, 7, out + 4) == E_ALIGN
    assert av(arr([sc[0] + 2, sc[1], sc[2]]), arr(nbs), 3, 512, 7, out) == E_ALIGN
    assert av(arr(sc), arr(nbs), 3, 512, 7, nbs[1] - 16) == E_OVERLAP
    assert lib.qsgd_dequant_average(arr(sc), arr(nbs), 3, 0, 512, 7, vp(out), NULL) == OK


def test_saps_validation(lib):
    n = 100_000
    x, m, o, v = A, A + (1 << 20), A + (2 << 20), A + (3 << 20)
    assert lib.saps_mask_words(n) == 3125 and lib.saps_mask_words(33) == 2
    assert lib.saps_num_tiles(n) == 13 and lib.saps_num_tiles(8192) == 1
    mk = lambda n_, c, m_, o_: lib.saps_mask(n_, F(c), ctypes.c_uint64(5), vp(m_), vp(o_), NULL)
    for bad in (0.5, 0.0, -2.0, float("nan"), float("inf")):
        assert mk(n, bad, m, o) == E_PARAM
    assert mk(n, 100.0, 0, o) == E_NULL
    assert mk(0, 100.0, m, 0) == E_NULL
    assert mk(n, 100.0, m + 2, o) == E_ALIGN
    assert mk(n, 100.0, m, o + 4) == E_ALIGN
    assert mk(n, 100.0, m, m + 64) == E_OVERLAP
    g = lambda x_, m_, o_, v_, cap: lib.saps_gather(vp(x_), n, vp(m_), vp(o_), vp(v_), cap, NULL)
    assert g(0, m, o, v, 10) == E_NULL
    assert g(x, m, o, 0, 10) == E_NULL
    assert g(x + 2, m, o, v, 10) == E_ALIGN
    assert g(x, m, o, x + 400, 10) == E_OVERLAP            # values inside x
    assert g(x, m, o, m, 10) == E_OVERLAP                  # values over the mask
    mg = lambda x_, m_, o_, v_, cap: lib.saps_merge(vp(x_), n, vp(m_), vp(o_), vp(v_), cap, NULL)
    assert mg(x, m, o, x + 4000, 10) == E_OVERLAP         # peer values inside x
    assert lib.saps_gather(vp(x), 0, vp(m), vp(o), vp(v), 0, NULL) == OK


def test_elias_validation(lib):
    n = 4096
    nm, nb, of, out = A, A + (1 << 20), A + (2 << 20), A + (3 << 20)
    assert lib.qsgd_elias_max_words(n, 7) == 0 and lib.qsgd_elias_max_words(n, 4096) == 0
    assert lib.qsgd_elias_max_words(n, 512) > n * 24 // 32
    e = lambda d, nm_, nb_, of_, o_, cap: lib.qsgd_elias_encode(vp(nm_), vp(nb_), n, d, vp(of_),
                                                                vp(o_), cap, NULL)
    for bad_d in (0, 4, 12, 2056, 4096):
        assert e(bad_d, nm, nb, of, out, 100) == E_PARAM
    assert e(512, 0, nb, of, out, 100) == E_NULL
    assert e(512, nm, nb, 0, out, 100) == E_NULL
    assert e(512, nm, nb, of + 4, out, 100) == E_ALIGN
    assert e(512, nm, nb, of, out + 2, 100) == E_ALIGN
    assert e(512, nm, nb, of, nb + 64, 100) == E_OVERLAP        # words over the nibbles
    assert e(512, nm, nb, nm, out, 100) == E_OVERLAP            # offsets over the norms
    dd = lambda d, i_, cnt, of_, nm_, nb_: lib.qsgd_elias_decode(vp(i_), cnt, vp(of_), n, d,
                                                                 vp(nm_), vp(nb_), NULL)
    assert dd(100, out, 10, of, nm, nb) == E_PARAM
    assert dd(512, out, 10, of, 0, nb) == E_NULL
    assert dd(512, out, 10, of, nm, out + 4) == E_OVERLAP       # nibbles over the input
    assert lib.qsgd_elias_decode(vp(out), 10, vp(of), 0, 512, vp(nm), vp(nb), NULL) == OK


def test_binding_refuses_host_tensors():
    torch = pytest.importorskip("torch")
    g = torch.zeros(16)
    with pytest.raises(ValueError):
        gcq.gc2_quantize(g, torch.zeros(16), 0.5)


def test_tuning_roundtrip_and_validation(lib):
    t = gcq.Tuning()
    assert lib.gcq_get_tuning(ctypes.byref(t)) == OK
    saved = t.as_dict()
    assert saved["gc2_unroll"] in (1, 2, 4) and saved["gc2_blocks_per_cu"] >= 0
    assert lib.gcq_get_tuning(None) == E_NULL
    assert lib.gcq_set_tuning(None) == E_NULL
    for field, bad in [("gc2_unroll", 3), ("gc2_unroll", 0), ("gc2_nt", -1), ("gc2_nt", 16), ("dq_lds_stores", 5),
                       ("gc2_blocks_per_cu", 1025), ("dq_blocks_per_cu", -3), ("qsgd_nt", 7),
                       ("qsgd_rcp", 2), ("qsgd_dequant_nt", 3), ("dq_fp4_decode", 2),
                       ("qsgd_blocks_per_cu", -1), ("qsgd_dequant_blocks_per_cu", 1025),
                       ("qsgd_buckets_per_wave", 3), ("qsgd_buckets_per_wave", -1),
                       ("dq_words_per_thread", 3), ("dq_words_per_thread", -1),
                       ("dq_resident_per_cu", 1), ("dq_resident_per_cu", 9),
                       ("dq_resident_per_cu", -1), ("gc2_resident_per_cu", 1),
                       ("gc2_resident_per_cu", 9), ("cdsgd_resident_per_cu", 1),
                       ("qsgd_avg_resident_per_cu", 9)]:
        b = gcq.Tuning(**saved)
        setattr(b, field, bad)
        assert lib.gcq_set_tuning(ctypes.byref(b)) == E_PARAM, field
    t2 = gcq.Tuning()
    lib.gcq_get_tuning(ctypes.byref(t2))
    assert t2.as_dict() == saved                      # a rejected set changes nothing
    old = gcq.set_tuning(gc2_blocks_per_cu=7, dq_nt_stores=1)
    assert gcq.get_tuning()["gc2_blocks_per_cu"] == 7
    gcq.set_tuning(**old)
    assert gcq.get_tuning() == saved


def test_element_limit(lib):
    # n above GCQ_MAX_ELEMS = 2^60 is a parameter error for every call; n at the
    # limit passes the size check (a NULL operand then reports itself, so
    # nothing is launched)
    big, top = (1 << 60) + 1, 1 << 60
    header = open(HEADER).read()
    assert "#define GCQ_MAX_ELEMS ((size_t)1 << 60)" in header
    g, r, o, w = A, A + (1 << 20), A + (2 << 20), A + (3 << 20)
    q = lambda n_, g_=g: lib.gc2_quantize(vp(g_), vp(r), n_, F(0.5), vp(o), NULL)
    assert q(big) == E_PARAM and q(top, 0) == E_NULL
    ws = (ctypes.c_void_p * 2)(A, A + (1 << 20))
    d = lambda n_, a: lib.gc2_dequant_reduce(ws, 2, n_, F(0.5), vp(a), NULL)
    assert d(big, w) == E_PARAM and d(top, 0) == E_NULL
    c = lambda n_, g_=g: lib.cdsgd_update_quantize(vp(g_), vp(r), vp(w), n_, F(0.5), F(0.1), vp(o),
                                                   NULL)
    assert c(big) == E_PARAM and c(top, 0) == E_NULL
    u = lambda n_, g_=g: lib.cdsgd_local_update(vp(g_), vp(w), n_, F(0.1), NULL)
    assert u(big) == E_PARAM and u(top, 0) == E_NULL
    for f in (lib.qsgd_quantize, lib.qsgd_quantize_maxnorm):
        qq = lambda n_, g_=g: f(vp(g_), n_, 512, 7, ctypes.c_uint64(1), vp(r), vp(o), NULL)
        assert qq(big) == E_PARAM and qq(top, 0) == E_NULL
    dq = lambda n_, a: lib.qsgd_dequant(vp(r), vp(o), n_, 512, 7, vp(a), NULL)
    assert dq(big, w) == E_PARAM and dq(top, 0) == E_NULL
    arr = lambda xs: (ctypes.c_void_p * len(xs))(*[vp(x) for x in xs])
    av = lambda n_, a: lib.qsgd_dequant_average(arr([r]), arr([o]), 1, n_, 512, 7, vp(a), NULL)
    assert av(big, w) == E_PARAM and av(top, 0) == E_NULL
    assert lib.qsgd_elias_max_words(big, 512) == 0
    e = lambda n_, cap, nm: lib.qsgd_elias_encode(vp(nm), vp(r), n_, 512, vp(o), vp(w), cap, NULL)
    assert e(big, 100, g) == E_PARAM and e(100, big, g) == E_PARAM and e(top, 100, 0) == E_NULL
    dd = lambda n_, cnt, nm: lib.qsgd_elias_decode(vp(w), cnt, vp(o), n_, 512, vp(nm), vp(r), NULL)
    assert dd(big, 10, g) == E_PARAM and dd(100, big, g) == E_PARAM and dd(top, 10, 0) == E_NULL
    mk = lambda n_, m_: lib.saps_mask(n_, F(100.0), ctypes.c_uint64(5), vp(m_), vp(o), NULL)
    assert mk(big, r) == E_PARAM and mk(top, 0) == E_NULL
    for f in (lib.saps_gather, lib.saps_merge):
        sa = lambda n_, cap, x_: f(vp(x_), n_, vp(r), vp(o), vp(w), cap, NULL)
        assert sa(big, 10, g) == E_PARAM and sa(100, big, g) == E_PARAM and sa(top, 10, 0) == E_NULL
    # the fused launch counts every bucket: two of 2^59 + 1 elements are too many together
    half = (1 << 59) + 1
    descs = [(A, A + (1 << 20), A + (2 << 20), half, 0.5), (A, A + (3 << 20), A + (4 << 20), half, 0.5)]
    arrb = (gcq.Gc2Bucket * 2)(*[gcq.Gc2Bucket(*x) for x in descs])
    assert lib.gc2_quantize_buckets(arrb, 2, NULL) == E_PARAM


# The defaults include/gcq.h documents for each knob (and the environment
# variable that overrides it).
DEFAULTS = {"gc2_unroll": 1, "gc2_nt": 7, "gc2_blocks_per_cu": 0, "dq_nt_loads": 1,
            "dq_nt_stores": 1, "dq_lds_stores": 1, "dq_blocks_per_cu": 0, "dq_fp4_decode": 1,
            "qsgd_nt": 1, "qsgd_rcp": 1, "qsgd_dequant_nt": 1, "qsgd_blocks_per_cu": 0,
            "qsgd_dequant_blocks_per_cu": 0, "qsgd_buckets_per_wave": 0, "dq_words_per_thread": 0,
            "dq_resident_per_cu": 3, "gc2_resident_per_cu": 0, "cdsgd_resident_per_cu": 5,
            "qsgd_avg_resident_per_cu": 0}


def _fresh_tuning(extra_env):
    import json
    import subprocess
    import sys

    env = {k: v for k, v in os.environ.items() if not k.startswith("GCQ_")}
    env.update(extra_env)
    code = ("import json, sys; sys.path.insert(0, %r); import gradient_compression_distributed_amd as g; "
            "print(json.dumps(g.get_tuning()))" % ROOT)
    p = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                       timeout=120)
    assert p.returncode == 0, p.stderr
    return json.loads(p.stdout.strip().splitlines()[-1])


def test_tuning_defaults_and_environment():
    assert _fresh_tuning({}) == DEFAULTS
    header = open(HEADER).read()
    for knob in DEFAULTS:
        assert knob in header, knob
        assert "GCQ_" + knob.upper() in header, knob
    t = _fresh_tuning({"GCQ_DQ_WORDS_PER_THREAD": "1", "GCQ_GC2_NT": "99",
                       "GCQ_QSGD_BUCKETS_PER_WAVE": "3", "GCQ_DQ_BLOCKS_PER_CU": "5",
                       "GCQ_DQ_RESIDENT_PER_CU": "1"})
    assert t["dq_resident_per_cu"] == 3            # invalid: the default
    assert _fresh_tuning({"GCQ_DQ_RESIDENT_PER_CU": "0"})["dq_resident_per_cu"] == 0
    assert t["dq_words_per_thread"] == 1
    assert t["gc2_nt"] == 15                       # clamped into 0..15
    assert t["qsgd_buckets_per_wave"] == 0         # invalid: the default
    assert t["dq_blocks_per_cu"] == 5
