"""MI355X (gfx950) gradient-compression hot path: Python binding.

A thin ctypes layer over ``libgcq.so`` (the C ABI of ``include/gcq.h``).
Every step of the path runs in the library's HIP kernels; this module only
checks tensor metadata, passes raw device pointers and the current HIP
stream, and turns a negative status into ``GcqError``.  PyTorch supplies
device memory and streams.  There is no CPU fallback: if the library is
missing, ``load()`` raises.

Packed words (2-bit codes, QSGD nibbles) are held in ``torch.int32``
tensors as raw 32-bit patterns (view them as uint32 on the host).
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "GcqError", "load", "lib_path", "gc2_quantize", "gc2_quantize_buckets",
    "gc2_quantize_buckets_noalloc", "GC2_NOALLOC_MAX_BUCKETS",
    "gc2_dequant_reduce", "qsgd_quantize", "qsgd_dequant", "gc2_packed_words",
    "qsgd_num_buckets", "qsgd_nibble_words", "MAX_WORKERS", "set_tuning", "get_tuning", "BucketList",
    "cdsgd_update_quantize", "cdsgd_local_update", "cdsgd_compresses",
    "qsgd_quantize_maxnorm", "qsgd_dequant_average",
    "saps_mask", "saps_gather", "saps_merge", "saps_mask_words", "saps_num_tiles",
    "qsgd_elias_encode", "qsgd_elias_decode", "qsgd_elias_max_words",
    "probe_stream", "probe_reduce",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_NAME = "libgcq.so"
MAX_WORKERS = 64

_lib = None


class GcqError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = _lib.gcq_status_string(status).decode() if _lib is not None else str(status)
        super().__init__(f"{where}: status {status} ({msg})")


class Tuning(ctypes.Structure):
    """Mirror of ``gcq_tuning`` (launch knobs; results never depend on them)."""
    _fields_ = [(f, ctypes.c_int) for f in (
        "gc2_unroll", "gc2_nt", "gc2_blocks_per_cu", "dq_nt_loads", "dq_nt_stores",
        "dq_lds_stores", "dq_blocks_per_cu", "dq_fp4_decode", "qsgd_nt", "qsgd_rcp",
        "qsgd_dequant_nt", "qsgd_blocks_per_cu", "qsgd_dequant_blocks_per_cu",
        "qsgd_buckets_per_wave", "dq_words_per_thread", "dq_resident_per_cu",
        "gc2_resident_per_cu", "cdsgd_resident_per_cu", "qsgd_avg_resident_per_cu")]

    def as_dict(self):
        return {f: getattr(self, f) for f, _ in self._fields_}


class Gc2Bucket(ctypes.Structure):
    _fields_ = [("g", ctypes.c_void_p), ("r", ctypes.c_void_p), ("out_words", ctypes.c_void_p),
                ("n", ctypes.c_size_t), ("t", ctypes.c_float)]


def lib_path() -> str:
    return os.path.join(_PKG, LIB_NAME)


def load():
    """Load libgcq.so from the package directory (raises if it is absent)."""
    global _lib
    if _lib is not None:
        return _lib
    path = lib_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run __graft_entry__.build() "
                           "(hipcc --offload-arch=gfx950) first")
    lib = ctypes.CDLL(path)
    vp, sz, u32, u64, f32, i32 = (ctypes.c_void_p, ctypes.c_size_t, ctypes.c_uint32,
                                  ctypes.c_uint64, ctypes.c_float, ctypes.c_int)
    lib.gc2_quantize.argtypes = [vp, vp, sz, f32, vp, vp]
    lib.gc2_quantize.restype = i32
    lib.gc2_quantize_buckets.argtypes = [ctypes.POINTER(Gc2Bucket), u32, vp]
    lib.gc2_quantize_buckets.restype = i32
    lib.gc2_quantize_buckets_noalloc.argtypes = [ctypes.POINTER(Gc2Bucket), u32, vp]
    lib.gc2_quantize_buckets_noalloc.restype = i32
    lib.gc2_dequant_reduce.argtypes = [ctypes.POINTER(vp), u32, sz, f32, vp, vp]
    lib.gc2_dequant_reduce.restype = i32
    lib.gcq_probe_reduce.argtypes = [ctypes.POINTER(vp), u32, sz, vp, vp]
    lib.gcq_probe_reduce.restype = i32
    lib.gcq_probe_stream.argtypes = [vp, vp, vp, vp, sz, vp]
    lib.gcq_probe_stream.restype = i32
    lib.qsgd_quantize.argtypes = [vp, sz, u32, u32, u64, vp, vp, vp]
    lib.qsgd_quantize.restype = i32
    lib.qsgd_dequant.argtypes = [vp, vp, sz, u32, u32, vp, vp]
    lib.qsgd_dequant.restype = i32
    lib.cdsgd_update_quantize.argtypes = [vp, vp, vp, sz, f32, f32, vp, vp]
    lib.cdsgd_update_quantize.restype = i32
    lib.qsgd_quantize_maxnorm.argtypes = [vp, sz, u32, u32, u64, vp, vp, vp]
    lib.qsgd_quantize_maxnorm.restype = i32
    lib.qsgd_dequant_average.argtypes = [ctypes.POINTER(vp), ctypes.POINTER(vp), u32, sz, u32,
                                         u32, vp, vp]
    lib.qsgd_dequant_average.restype = i32
    lib.qsgd_elias_max_words.argtypes = [sz, u32]
    lib.qsgd_elias_max_words.restype = sz
    lib.qsgd_elias_encode.argtypes = [vp, vp, sz, u32, vp, vp, sz, vp]
    lib.qsgd_elias_encode.restype = i32
    lib.qsgd_elias_decode.argtypes = [vp, sz, vp, sz, u32, vp, vp, vp]
    lib.qsgd_elias_decode.restype = i32
    lib.saps_mask.argtypes = [sz, f32, u64, vp, vp, vp]
    lib.saps_mask.restype = i32
    lib.saps_gather.argtypes = [vp, sz, vp, vp, vp, sz, vp]
    lib.saps_gather.restype = i32
    lib.saps_merge.argtypes = [vp, sz, vp, vp, vp, sz, vp]
    lib.saps_merge.restype = i32
    lib.saps_mask_words.argtypes = [sz]
    lib.saps_mask_words.restype = sz
    lib.saps_num_tiles.argtypes = [sz]
    lib.saps_num_tiles.restype = sz
    lib.cdsgd_local_update.argtypes = [vp, vp, sz, f32, vp]
    lib.cdsgd_local_update.restype = i32
    lib.gc2_packed_words.argtypes = [sz]
    lib.gc2_packed_words.restype = sz
    lib.qsgd_num_buckets.argtypes = [sz, u32]
    lib.qsgd_num_buckets.restype = sz
    lib.qsgd_nibble_words.argtypes = [sz]
    lib.qsgd_nibble_words.restype = sz
    lib.gcq_status_string.argtypes = [i32]
    lib.gcq_status_string.restype = ctypes.c_char_p
    lib.gcq_get_tuning.argtypes = [ctypes.POINTER(Tuning)]
    lib.gcq_get_tuning.restype = i32
    lib.gcq_set_tuning.argtypes = [ctypes.POINTER(Tuning)]
    lib.gcq_set_tuning.restype = i32
    _lib = lib
    return lib


# ---------------------------------------------------------------- helpers
def gc2_packed_words(n: int) -> int:
    return int(load().gc2_packed_words(n))


def qsgd_num_buckets(n: int, d: int) -> int:
    return int(load().qsgd_num_buckets(n, d))


def qsgd_nibble_words(n: int) -> int:
    return int(load().qsgd_nibble_words(n))


def _dev(x, dtype, name, min_numel=0):
    import torch

    if not isinstance(x, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if x.device.type != "cuda":
        raise ValueError(f"{name} must live in GPU memory (got {x.device})")
    if x.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {x.dtype})")
    if not x.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if x.numel() < min_numel:
        raise ValueError(f"{name} holds {x.numel()} elements, needs {min_numel}")
    return x


def _ptr(x):
    return ctypes.c_void_p(x.data_ptr() if x is not None and x.numel() else 0)


def _stream(device=None):
    import torch

    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check(status: int, where: str):
    if status != 0:
        raise GcqError(status, where)


def get_tuning() -> dict:
    """Current launch knobs as a dict (see ``gcq_tuning`` in include/gcq.h)."""
    t = Tuning()
    _check(load().gcq_get_tuning(ctypes.byref(t)), "gcq_get_tuning")
    return t.as_dict()


def set_tuning(**knobs) -> dict:
    """Change some launch knobs (speed only; results are identical).
    Returns the previous settings, so ``set_tuning(**old)`` restores them."""
    t = Tuning()
    _check(load().gcq_get_tuning(ctypes.byref(t)), "gcq_get_tuning")
    old = t.as_dict()
    for k, v in knobs.items():
        if k not in old:
            raise KeyError(f"unknown tuning knob {k!r}")
        setattr(t, k, int(v))
    _check(load().gcq_set_tuning(ctypes.byref(t)), "gcq_set_tuning")
    return old


# -------------------------------------------------------------- the calls
def gc2_quantize(g, r, t: float, out=None):
    """One 2-bit quantize step: returns the packed words, updates ``r``."""
    import torch

    lib = load()
    _dev(g, torch.float32, "g")
    n = g.numel()
    _dev(r, torch.float32, "r", n)
    if out is None:
        out = torch.empty(gc2_packed_words(n), dtype=torch.int32, device=g.device)
    _dev(out, torch.int32, "out", gc2_packed_words(n))
    _check(lib.gc2_quantize(_ptr(g), _ptr(r), n, ctypes.c_float(t), _ptr(out),
                            _stream(g.device)), "gc2_quantize")
    return out


def cdsgd_compresses(count: int, k: int) -> bool:
    """CD-SGD's k-step switch (Algorithm 1, section 3.2.1): iteration
    ``count`` compresses its gradient unless ``count % k == 0``, when the
    full-precision gradient is pushed instead (host logic only)."""
    if k < 1:
        raise ValueError("k must be >= 1")
    return count % k != 0


def cdsgd_update_quantize(g, r, w, t: float, eta: float, out=None):
    """A compressing CD-SGD iteration on one buffer: ``w -= eta * g`` (local
    update) and one 2-bit quantize step of (g, r); returns the packed words."""
    import torch

    lib = load()
    _dev(g, torch.float32, "g")
    n = g.numel()
    _dev(r, torch.float32, "r", n)
    _dev(w, torch.float32, "w", n)
    if out is None:
        out = torch.empty(gc2_packed_words(n), dtype=torch.int32, device=g.device)
    _dev(out, torch.int32, "out", gc2_packed_words(n))
    _check(lib.cdsgd_update_quantize(_ptr(g), _ptr(r), _ptr(w), n, ctypes.c_float(t),
                                     ctypes.c_float(eta), _ptr(out), _stream(g.device)),
           "cdsgd_update_quantize")
    return out


def cdsgd_local_update(g, w, eta: float):
    """A correction iteration's local update: ``w -= eta * g``."""
    import torch

    lib = load()
    _dev(g, torch.float32, "g")
    _dev(w, torch.float32, "w", g.numel())
    _check(lib.cdsgd_local_update(_ptr(g), _ptr(w), g.numel(), ctypes.c_float(eta),
                                  _stream(g.device)), "cdsgd_local_update")


class BucketList:
    """A checked, reusable descriptor array for gc2_quantize_buckets.

    Holds references to the tensors so their memory outlives the list;
    building it once and reusing it every step keeps per-call host work to
    the library's own checks and one launch."""

    def __init__(self, buckets):
        import torch

        self.tensors = list(buckets)
        self.array = (Gc2Bucket * max(len(buckets), 1))()
        self.device = None
        for i, (g, r, out, t) in enumerate(buckets):
            _dev(g, torch.float32, f"buckets[{i}].g")
            n = g.numel()
            _dev(r, torch.float32, f"buckets[{i}].r", n)
            _dev(out, torch.int32, f"buckets[{i}].out", gc2_packed_words(n))
            self.array[i] = Gc2Bucket(g.data_ptr() if n else 0, r.data_ptr() if n else 0,
                                      out.data_ptr() if n else 0, n, t)
            self.device = self.device or g.device
        self.count = len(buckets)


def gc2_quantize_buckets(buckets):
    """Fused launch over ``[(g, r, out, t), ...]`` (or a ``BucketList``);
    each bucket is quantized exactly as gc2_quantize would."""
    lib = load()
    bl = buckets if isinstance(buckets, BucketList) else BucketList(buckets)
    _check(lib.gc2_quantize_buckets(bl.array, bl.count, _stream(bl.device)),
           "gc2_quantize_buckets")


def gc2_quantize_buckets_noalloc(buckets):
    """gc2_quantize_buckets through the entry point that allocates nothing
    (its descriptor table is a fixed device array of the library, at most
    GC2_NOALLOC_MAX_BUCKETS buckets; calls that may overlap on one device
    race on it)."""
    lib = load()
    bl = buckets if isinstance(buckets, BucketList) else BucketList(buckets)
    _check(lib.gc2_quantize_buckets_noalloc(bl.array, bl.count, _stream(bl.device)),
           "gc2_quantize_buckets_noalloc")


GC2_NOALLOC_MAX_BUCKETS = 4096


def gc2_dequant_reduce(words, n: int, t: float, acc=None):
    """acc = sum over workers 0..W-1 (in order) of the dequantized codes."""
    import torch

    lib = load()
    W = len(words)
    nw = gc2_packed_words(n)
    for i, w in enumerate(words):
        _dev(w, torch.int32, f"words[{i}]", nw)
    if acc is None:
        acc = torch.empty(n, dtype=torch.float32, device=words[0].device)
    _dev(acc, torch.float32, "acc", n)
    ptrs = (ctypes.c_void_p * max(W, 1))(*[w.data_ptr() for w in words])
    _check(lib.gc2_dequant_reduce(ptrs, W, n, ctypes.c_float(t), _ptr(acc),
                                  _stream(acc.device)), "gc2_dequant_reduce")
    return acc


def probe_stream(a, c, b=None, words=None):
    """Measurement probe with the 2-bit quantizer's access pattern and no
    arithmetic: c = a ^ b (bitwise; c = a without b), plus a packed-word
    stream when ``words`` is given.  n = a.numel() must be a multiple of 1024."""
    import torch

    lib = load()
    _dev(a, torch.float32, "a")
    n = a.numel()
    _dev(c, torch.float32, "c", n)
    if b is not None:
        _dev(b, torch.float32, "b", n)
    if words is not None:
        _dev(words, torch.int32, "words", n // 16)
    _check(lib.gcq_probe_stream(_ptr(a), _ptr(b) if b is not None else None, _ptr(c),
                                _ptr(words) if words is not None else None, n,
                                _stream(a.device)), "gcq_probe_stream")


def probe_reduce(words, n: int, acc):
    """Measurement probe: gc2_dequant_reduce's kernel with the decode replaced
    by an XOR (acc[16 i] = XOR of the workers' word i, other sums +0)."""
    import torch

    lib = load()
    W = len(words)
    nw = gc2_packed_words(n)
    for i, w in enumerate(words):
        _dev(w, torch.int32, f"words[{i}]", nw)
    _dev(acc, torch.float32, "acc", n)
    ptrs = (ctypes.c_void_p * max(W, 1))(*[w.data_ptr() for w in words])
    _check(lib.gcq_probe_reduce(ptrs, W, n, _ptr(acc), _stream(acc.device)), "gcq_probe_reduce")
    return acc


def qsgd_quantize(g, d: int, s: int, seed: int, norms=None, nibbles=None, maxnorm: bool = False):
    """Bucketed QSGD: returns (norms float32[ceil(n/d)], nibbles int32[ceil(n/8)]).
    With ``maxnorm`` the bucket scale is the largest magnitude (Knowl 8)."""
    import torch

    lib = load()
    _dev(g, torch.float32, "g")
    n = g.numel()
    nb, nw = qsgd_num_buckets(n, d), qsgd_nibble_words(n)
    if norms is None:
        norms = torch.empty(nb, dtype=torch.float32, device=g.device)
    if nibbles is None:
        nibbles = torch.empty(nw, dtype=torch.int32, device=g.device)
    _dev(norms, torch.float32, "norms", nb)
    _dev(nibbles, torch.int32, "nibbles", nw)
    fn = lib.qsgd_quantize_maxnorm if maxnorm else lib.qsgd_quantize
    _check(fn(_ptr(g), n, d, s, ctypes.c_uint64(seed & 0xFFFFFFFFFFFFFFFF),
              _ptr(norms), _ptr(nibbles), _stream(g.device)), "qsgd_quantize")
    return norms, nibbles


def qsgd_quantize_maxnorm(g, d: int, s: int, seed: int, scales=None, nibbles=None):
    """QSGD with max-norm bucket scales: returns (scales, nibbles)."""
    return qsgd_quantize(g, d, s, seed, norms=scales, nibbles=nibbles, maxnorm=True)


def qsgd_dequant_average(scales, nibbles, n: int, d: int, s: int, out=None):
    """Mean over K workers (order 0..K-1) of their decoded QSGD messages."""
    import torch

    lib = load()
    K = len(scales)
    if K != len(nibbles):
        raise ValueError("scales and nibbles differ in length")
    for i in range(K):
        _dev(scales[i], torch.float32, f"scales[{i}]", qsgd_num_buckets(n, d))
        _dev(nibbles[i], torch.int32, f"nibbles[{i}]", qsgd_nibble_words(n))
    if out is None:
        out = torch.empty(n, dtype=torch.float32, device=scales[0].device)
    _dev(out, torch.float32, "out", n)
    sp = (ctypes.c_void_p * max(K, 1))(*[x.data_ptr() for x in scales])
    npp = (ctypes.c_void_p * max(K, 1))(*[x.data_ptr() for x in nibbles])
    _check(lib.qsgd_dequant_average(sp, npp, K, n, d, s, _ptr(out), _stream(out.device)),
           "qsgd_dequant_average")
    return out


def qsgd_dequant(norms, nibbles, n: int, d: int, s: int, out=None):
    """out = +-(norm * level) / s per element."""
    import torch

    lib = load()
    _dev(norms, torch.float32, "norms", qsgd_num_buckets(n, d))
    _dev(nibbles, torch.int32, "nibbles", qsgd_nibble_words(n))
    if out is None:
        out = torch.empty(n, dtype=torch.float32, device=norms.device)
    _dev(out, torch.float32, "out", n)
    _check(lib.qsgd_dequant(_ptr(norms), _ptr(nibbles), n, d, s, _ptr(out),
                            _stream(out.device)), "qsgd_dequant")
    return out


# ------------------------------------------------------------------ SAPS
def saps_mask_words(n: int) -> int:
    return int(load().saps_mask_words(n))


def saps_num_tiles(n: int) -> int:
    return int(load().saps_num_tiles(n))


def saps_mask(n: int, c: float, seed: int, mask=None, offsets=None, device="cuda"):
    """Shared-seed Bernoulli(1/c) mask: returns (mask words int32, tile
    offsets int64 with the total kept count last)."""
    import torch

    lib = load()
    if mask is None:
        mask = torch.empty(saps_mask_words(n), dtype=torch.int32, device=device)
    if offsets is None:
        offsets = torch.empty(saps_num_tiles(n) + 1, dtype=torch.int64, device=device)
    _dev(mask, torch.int32, "mask", saps_mask_words(n))
    _dev(offsets, torch.int64, "offsets", saps_num_tiles(n) + 1)
    _check(lib.saps_mask(n, ctypes.c_float(c), ctypes.c_uint64(seed & 0xFFFFFFFFFFFFFFFF),
                         _ptr(mask), _ptr(offsets), _stream(offsets.device)), "saps_mask")
    return mask, offsets


def saps_count(offsets) -> int:
    """The total kept count (synchronizes with the device)."""
    return int(offsets[-1].item())


def saps_gather(x, mask, offsets, values=None):
    """The kept components of ``x`` in index order."""
    import torch

    lib = load()
    _dev(x, torch.float32, "x")
    _dev(mask, torch.int32, "mask", saps_mask_words(x.numel()))
    _dev(offsets, torch.int64, "offsets", saps_num_tiles(x.numel()) + 1)
    if values is None:
        values = torch.empty(saps_count(offsets), dtype=torch.float32, device=x.device)
    _dev(values, torch.float32, "values")
    _check(lib.saps_gather(_ptr(x), x.numel(), _ptr(mask), _ptr(offsets), _ptr(values),
                           values.numel(), _stream(x.device)), "saps_gather")
    return values


def saps_merge(x, mask, offsets, peer_values):
    """x[kept] = (x[kept] + peer_values) * 0.5, in place."""
    import torch

    lib = load()
    _dev(x, torch.float32, "x")
    _dev(mask, torch.int32, "mask", saps_mask_words(x.numel()))
    _dev(offsets, torch.int64, "offsets", saps_num_tiles(x.numel()) + 1)
    _dev(peer_values, torch.float32, "peer_values")
    _check(lib.saps_merge(_ptr(x), x.numel(), _ptr(mask), _ptr(offsets), _ptr(peer_values),
                          peer_values.numel(), _stream(x.device)), "saps_merge")


# ------------------------------------------------------- QSGD Elias coding
def qsgd_elias_max_words(n: int, d: int) -> int:
    return int(load().qsgd_elias_max_words(n, d))


def qsgd_elias_encode(norms, nibbles, n: int, d: int, offsets=None, out=None):
    """Elias-omega coded buckets: returns (bit offsets int64[nb + 1], words
    int32[capacity]); the coded length in bits is the last offset."""
    import torch

    lib = load()
    nb = qsgd_num_buckets(n, d)
    _dev(norms, torch.float32, "norms", nb)
    _dev(nibbles, torch.int32, "nibbles", qsgd_nibble_words(n))
    if offsets is None:
        offsets = torch.empty(nb + 1, dtype=torch.int64, device=norms.device)
    if out is None:
        out = torch.empty(max(qsgd_elias_max_words(n, d), 1), dtype=torch.int32,
                          device=norms.device)
    _dev(offsets, torch.int64, "offsets", nb + 1)
    _dev(out, torch.int32, "out")
    _check(lib.qsgd_elias_encode(_ptr(norms), _ptr(nibbles), n, d, _ptr(offsets), _ptr(out),
                                 out.numel(), _stream(out.device)), "qsgd_elias_encode")
    return offsets, out


def qsgd_elias_decode(words, offsets, n: int, d: int, norms=None, nibbles=None):
    """Returns (norms, nibbles) of Elias-coded buckets."""
    import torch

    lib = load()
    nb = qsgd_num_buckets(n, d)
    _dev(words, torch.int32, "words")
    _dev(offsets, torch.int64, "offsets", nb + 1)
    if norms is None:
        norms = torch.empty(nb, dtype=torch.float32, device=words.device)
    if nibbles is None:
        nibbles = torch.empty(qsgd_nibble_words(n), dtype=torch.int32, device=words.device)
    _dev(norms, torch.float32, "norms", nb)
    _dev(nibbles, torch.int32, "nibbles", qsgd_nibble_words(n))
    _check(lib.qsgd_elias_decode(_ptr(words), words.numel(), _ptr(offsets), n, d, _ptr(norms),
                                 _ptr(nibbles), _stream(words.device)), "qsgd_elias_decode")
    return norms, nibbles
