"""CPU oracle for the gradient-compression hot path (TEST INFRASTRUCTURE).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never loads it and must fail loudly when the HIP
extension is missing instead of falling back here.

The arithmetic lives in ``gcq_oracle.c`` (plain scalar C, one thread); this
module only marshals numpy arrays through ctypes.  Each wrapper names the
passage of the pages it follows:

* ``gc2_quantize``       -- MXNet PR "2bit gradient compression",
  "Two bit quantization" and "Format of compressed gradient"; CD-SGD 3.4.1.
* ``gc2_dequant_reduce`` -- same PR, "Local kvstore" (device 0 dequantizes
  and sums the other devices' packed data), fixed worker order.
* ``cdsgd_local_update`` / ``cdsgd_update_quantize`` -- CD-SGD 3.4.1
  eq. (11) (w_loc = w - eta g), 3.2.1 Algorithm 1 and Figure 4(b) (the
  local update and the compression both read the same gradient).
* ``qsgd_norms`` / ``qsgd_levels`` / ``qsgd_quantize`` / ``qsgd_dequant``
  -- QSGD summary, Knowl 1 (Q_s), Knowl 2 (norm/sign/level tuple),
  Knowl 8 (bucketing).
* ``qsgd_maxnorms`` / ``qsgd_quantize_maxnorm`` -- Knowl 8, max-norm
  scaling; ``qsgd_dequant_average`` -- Knowl 3 (decode every peer's message
  and average).
* ``saps_keep`` / ``saps_gather`` / ``saps_merge`` -- SAPS ("Communication-
  Efficient Decentralized Learning with Sparsification and Adaptive Peer
  Selection"): the shared-seed Bernoulli(1/c) mask and the single-peer
  exchange.
* ``omega_length`` / ``qsgd_elias_encode`` / ``qsgd_elias_decode`` -- QSGD
  summary Knowl 2 (norm, then omega-coded distances between non-zero
  coordinates with sign and level), Elias' omega code (1975).
* ``philox4x32_10`` / ``uniform`` -- the SC'11 Philox-4x32 generator,
  pinned to its published known-answer vectors (``tests/golden/``).  The
  pages name no random source: which generator, and how (seed, index) map
  to its key and counter, is a frozen reading; the pages accept any
  independent uniforms.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")

_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        from .build import build_oracle

        build_oracle()
    lib = ctypes.CDLL(LIB_PATH)
    vp, sz, u32, u64, f32 = (ctypes.c_void_p, ctypes.c_size_t, ctypes.c_uint32,
                             ctypes.c_uint64, ctypes.c_float)
    lib.oracle_gc2_quantize.argtypes = [vp, vp, sz, f32, vp]
    lib.oracle_gc2_quantize.restype = None
    lib.oracle_gc2_dequant_reduce.argtypes = [vp, u32, sz, f32, vp]
    lib.oracle_cdsgd_local_update.argtypes = [vp, vp, sz, f32]
    lib.oracle_cdsgd_local_update.restype = None
    lib.oracle_cdsgd_update_quantize.argtypes = [vp, vp, vp, sz, f32, f32, vp]
    lib.oracle_cdsgd_update_quantize.restype = None
    lib.oracle_gc2_dequant_reduce.restype = None
    lib.oracle_philox4x32_10.argtypes = [vp, vp, vp]
    lib.oracle_philox4x32_10.restype = None
    lib.oracle_uniform.argtypes = [u64, u64]
    lib.oracle_uniform.restype = f32
    lib.oracle_qsgd_norms.argtypes = [vp, sz, u32, vp]
    lib.oracle_qsgd_norms.restype = None
    lib.oracle_qsgd_levels.argtypes = [vp, sz, u32, u32, u64, u64, vp, vp]
    lib.oracle_qsgd_levels.restype = None
    lib.oracle_qsgd_quantize.argtypes = [vp, sz, u32, u32, u64, vp, vp]
    lib.oracle_qsgd_quantize.restype = None
    lib.oracle_qsgd_dequant.argtypes = [vp, vp, sz, u32, u32, vp]
    lib.oracle_omega_length.argtypes = [u64]
    lib.oracle_omega_length.restype = ctypes.c_uint
    lib.oracle_qsgd_elias_encode.argtypes = [vp, vp, sz, u32, vp, vp, sz]
    lib.oracle_qsgd_elias_encode.restype = u64
    lib.oracle_qsgd_elias_decode.argtypes = [vp, vp, sz, u32, vp, vp]
    lib.oracle_qsgd_elias_decode.restype = None
    lib.oracle_saps_keep.argtypes = [u64, u64, f32]
    lib.oracle_saps_keep.restype = ctypes.c_int
    lib.oracle_saps_keep_range.argtypes = [u64, u64, sz, f32, vp]
    lib.oracle_saps_keep_range.restype = None
    lib.oracle_saps_gather.argtypes = [vp, sz, f32, u64, vp]
    lib.oracle_saps_gather.restype = sz
    lib.oracle_saps_merge.argtypes = [vp, sz, f32, u64, vp]
    lib.oracle_saps_merge.restype = sz
    lib.oracle_qsgd_maxnorms.argtypes = [vp, sz, u32, vp]
    lib.oracle_qsgd_maxnorms.restype = None
    lib.oracle_qsgd_quantize_maxnorm.argtypes = [vp, sz, u32, u32, u64, vp, vp]
    lib.oracle_qsgd_quantize_maxnorm.restype = None
    lib.oracle_qsgd_dequant_average.argtypes = [vp, vp, u32, sz, u32, u32, vp]
    lib.oracle_qsgd_dequant_average.restype = None
    lib.oracle_qsgd_dequant.restype = None
    _lib = lib
    return lib


def _f32(a, name):
    if not (isinstance(a, np.ndarray) and a.dtype == np.float32 and a.flags.c_contiguous):
        raise TypeError(f"{name} must be a C-contiguous float32 numpy array")
    return a


def _u32(a, name):
    if not (isinstance(a, np.ndarray) and a.dtype == np.uint32 and a.flags.c_contiguous):
        raise TypeError(f"{name} must be a C-contiguous uint32 numpy array")
    return a


def _ptr(a):
    return ctypes.c_void_p(a.ctypes.data)


def packed_words(n: int) -> int:
    return (n + 15) // 16


def nibble_words(n: int) -> int:
    return (n + 7) // 8


def num_buckets(n: int, d: int) -> int:
    return (n + d - 1) // d


def gc2_quantize(g: np.ndarray, r: np.ndarray, t: float, out: np.ndarray | None = None):
    """One quantize step: returns packed words; ``r`` is updated in place."""
    lib = _load()
    _f32(g, "g"), _f32(r, "r")
    n = g.size
    if r.size != n:
        raise ValueError("g and r differ in size")
    if out is None:
        out = np.empty(packed_words(n), dtype=np.uint32)
    _u32(out, "out")
    if out.size < packed_words(n):
        raise ValueError("out too small")
    lib.oracle_gc2_quantize(_ptr(g), _ptr(r), n, ctypes.c_float(t), _ptr(out))
    return out


def cdsgd_local_update(g: np.ndarray, w: np.ndarray, eta: float) -> None:
    """w = w - eta * g in float32 (product, then difference); ``w`` in place."""
    lib = _load()
    _f32(g, "g"), _f32(w, "w")
    if w.size != g.size:
        raise ValueError("g and w differ in size")
    lib.oracle_cdsgd_local_update(_ptr(g), _ptr(w), g.size, ctypes.c_float(eta))


def cdsgd_update_quantize(g: np.ndarray, r: np.ndarray, w: np.ndarray, t: float, eta: float,
                          out: np.ndarray | None = None):
    """Local update of ``w`` and one quantize step of (g, r); returns the
    packed words, ``r`` and ``w`` are updated in place."""
    lib = _load()
    _f32(g, "g"), _f32(r, "r"), _f32(w, "w")
    n = g.size
    if r.size != n or w.size != n:
        raise ValueError("g, r and w differ in size")
    if out is None:
        out = np.empty(packed_words(n), dtype=np.uint32)
    _u32(out, "out")
    if out.size < packed_words(n):
        raise ValueError("out too small")
    lib.oracle_cdsgd_update_quantize(_ptr(g), _ptr(r), _ptr(w), n, ctypes.c_float(t),
                                     ctypes.c_float(eta), _ptr(out))
    return out


def gc2_dequant_reduce(words: list, n: int, t: float, acc: np.ndarray | None = None):
    """Sum of W workers' dequantized codes, worker order 0..W-1, float32."""
    lib = _load()
    W = len(words)
    for w in words:
        _u32(w, "words[w]")
        if w.size < packed_words(n):
            raise ValueError("a worker buffer is too small")
    if acc is None:
        acc = np.empty(n, dtype=np.float32)
    _f32(acc, "acc")
    ptrs = (ctypes.c_void_p * max(W, 1))(*[w.ctypes.data for w in words])
    lib.oracle_gc2_dequant_reduce(ctypes.cast(ptrs, ctypes.c_void_p), W, n,
                                  ctypes.c_float(t), _ptr(acc))
    return acc


def philox4x32_10(ctr, key):
    lib = _load()
    c = np.ascontiguousarray(np.asarray(ctr, dtype=np.uint32))
    k = np.ascontiguousarray(np.asarray(key, dtype=np.uint32))
    o = np.empty(4, dtype=np.uint32)
    lib.oracle_philox4x32_10(_ptr(c), _ptr(k), _ptr(o))
    return o


def uniform(seed: int, i: int) -> float:
    return float(_load().oracle_uniform(seed, i))


def qsgd_norms(g: np.ndarray, d: int) -> np.ndarray:
    lib = _load()
    _f32(g, "g")
    norms = np.empty(num_buckets(g.size, d), dtype=np.float32)
    lib.oracle_qsgd_norms(_ptr(g), g.size, d, _ptr(norms))
    return norms


def qsgd_levels(g: np.ndarray, d: int, s: int, seed: int, norms: np.ndarray,
                index_base: int = 0) -> np.ndarray:
    """Nibbles for the slice ``g`` given bucket norms (e.g. a GPU's norms).

    ``index_base`` is the global index of ``g[0]``; it must be a multiple of
    ``d`` and of 8 (buckets and words are counted from the slice start, the
    uniform uses the global index)."""
    lib = _load()
    _f32(g, "g"), _f32(norms, "norms")
    if index_base % d or index_base % 8:
        raise ValueError("index_base must be a multiple of d and 8")
    if norms.size < num_buckets(g.size, d):
        raise ValueError("norms too small")
    nib = np.empty(nibble_words(g.size), dtype=np.uint32)
    lib.oracle_qsgd_levels(_ptr(g), g.size, d, s, ctypes.c_uint64(seed),
                           ctypes.c_uint64(index_base), _ptr(norms), _ptr(nib))
    return nib


def qsgd_quantize(g: np.ndarray, d: int, s: int, seed: int):
    lib = _load()
    _f32(g, "g")
    norms = np.empty(num_buckets(g.size, d), dtype=np.float32)
    nib = np.empty(nibble_words(g.size), dtype=np.uint32)
    lib.oracle_qsgd_quantize(_ptr(g), g.size, d, s, ctypes.c_uint64(seed),
                             _ptr(norms), _ptr(nib))
    return norms, nib


def qsgd_dequant(norms: np.ndarray, nibbles: np.ndarray, n: int, d: int, s: int) -> np.ndarray:
    lib = _load()
    _f32(norms, "norms"), _u32(nibbles, "nibbles")
    if nibbles.size < nibble_words(n) or norms.size < num_buckets(n, d):
        raise ValueError("inputs too small")
    out = np.empty(n, dtype=np.float32)
    lib.oracle_qsgd_dequant(_ptr(norms), _ptr(nibbles), n, d, s, _ptr(out))
    return out


def qsgd_maxnorms(g: np.ndarray, d: int) -> np.ndarray:
    lib = _load()
    _f32(g, "g")
    scales = np.empty(num_buckets(g.size, d), dtype=np.float32)
    lib.oracle_qsgd_maxnorms(_ptr(g), g.size, d, _ptr(scales))
    return scales


def qsgd_quantize_maxnorm(g: np.ndarray, d: int, s: int, seed: int):
    lib = _load()
    _f32(g, "g")
    scales = np.empty(num_buckets(g.size, d), dtype=np.float32)
    nib = np.empty(nibble_words(g.size), dtype=np.uint32)
    lib.oracle_qsgd_quantize_maxnorm(_ptr(g), g.size, d, s, ctypes.c_uint64(seed),
                                     _ptr(scales), _ptr(nib))
    return scales, nib


def qsgd_dequant_average(scales: list, nibbles: list, n: int, d: int, s: int) -> np.ndarray:
    """Mean over K workers of the decoded messages (worker order 0..K-1)."""
    lib = _load()
    K = len(scales)
    if K == 0 or len(nibbles) != K:
        raise ValueError("need K >= 1 scale and nibble arrays")
    for a in scales:
        _f32(a, "scales")
        if a.size < num_buckets(n, d):
            raise ValueError("scales too small")
    for a in nibbles:
        _u32(a, "nibbles")
        if a.size < nibble_words(n):
            raise ValueError("nibbles too small")
    sp = (ctypes.c_void_p * K)(*[_ptr(a) for a in scales])
    npp = (ctypes.c_void_p * K)(*[_ptr(a) for a in nibbles])
    out = np.empty(n, dtype=np.float32)
    lib.oracle_qsgd_dequant_average(sp, npp, K, n, d, s, _ptr(out))
    return out


def saps_keep(seed: int, n: int, c: float, start: int = 0) -> np.ndarray:
    """The mask: keep[i] for start <= i < start + n, as a bool array."""
    lib = _load()
    keep = np.empty(n, dtype=np.uint8)
    lib.oracle_saps_keep_range(ctypes.c_uint64(seed), ctypes.c_uint64(start), n,
                               ctypes.c_float(c), _ptr(keep))
    return keep.view(bool)


def saps_gather(x: np.ndarray, c: float, seed: int) -> np.ndarray:
    lib = _load()
    _f32(x, "x")
    vals = np.empty(x.size, dtype=np.float32)
    k = lib.oracle_saps_gather(_ptr(x), x.size, ctypes.c_float(c), ctypes.c_uint64(seed), _ptr(vals))
    return vals[:k].copy()


def saps_merge(x: np.ndarray, c: float, seed: int, peer: np.ndarray) -> int:
    """x[kept] = (x[kept] + peer) * 0.5 in place; returns the count used."""
    lib = _load()
    _f32(x, "x"), _f32(peer, "peer")
    return int(lib.oracle_saps_merge(_ptr(x), x.size, ctypes.c_float(c), ctypes.c_uint64(seed),
                                     _ptr(peer)))


def omega_length(k: int) -> int:
    return int(_load().oracle_omega_length(k))


def qsgd_elias_encode(norms: np.ndarray, nibbles: np.ndarray, n: int, d: int):
    """Returns (bit_offsets uint64[nb + 1], words uint32[ceil(total/32)])."""
    lib = _load()
    _f32(norms, "norms"), _u32(nibbles, "nibbles")
    nb = num_buckets(n, d)
    if norms.size < nb or nibbles.size < nibble_words(n):
        raise ValueError("inputs too small")
    offs = np.empty(nb + 1, dtype=np.uint64)
    cap = nb + (n * 32 + 31) // 32 + 1          # 32 norm bits + at most 32 bits per element
    out = np.empty(cap, dtype=np.uint32)
    total = lib.oracle_qsgd_elias_encode(_ptr(norms), _ptr(nibbles), n, d, _ptr(offs), _ptr(out),
                                         cap)
    return offs, out[:(total + 31) // 32].copy()


def qsgd_elias_decode(words: np.ndarray, bit_offsets: np.ndarray, n: int, d: int):
    """Returns (norms, nibbles) of the coded buckets."""
    lib = _load()
    _u32(words, "words")
    nb = num_buckets(n, d)
    offs = np.ascontiguousarray(bit_offsets, dtype=np.uint64)
    if offs.size < nb + 1:
        raise ValueError("bit_offsets too small")
    norms = np.empty(nb, dtype=np.float32)
    nib = np.empty(nibble_words(n), dtype=np.uint32)
    lib.oracle_qsgd_elias_decode(_ptr(words), _ptr(offs), n, d, _ptr(norms), _ptr(nib))
    return norms, nib
