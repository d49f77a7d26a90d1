"""Host-side helpers of the whole-size GPU parity tests (test
infrastructure, no arithmetic of the method).

* ``pmap`` runs a function over items on a pool of host threads.  The
  oracle's C functions are called through ctypes, which releases the GIL,
  so pieces of one oracle pass run in parallel.  The tests only split where
  the oracle's definition is already independent: whole buckets of the
  2-bit quantizer, whole packed words of the reduce, whole QSGD buckets at
  their global indices.
* ``Host`` copies device tensors into page-locked host buffers that are
  allocated once and reused, so a 4 GiB copy per step costs no fresh page
  faults.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np


def threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def pmap(fn, items):
    items = list(items)
    with ThreadPoolExecutor(max_workers=threads()) as ex:
        return list(ex.map(fn, items))


def spans(total: int, piece: int):
    """[lo, hi) ranges covering [0, total) in steps of `piece`."""
    return [(lo, min(lo + piece, total)) for lo in range(0, total, piece)]


class Host:
    """Reusable page-locked host buffers keyed by name."""

    def __init__(self):
        self._bufs = {}

    def copy(self, name: str, t) -> np.ndarray:
        """A host copy of device tensor `t` (synchronous) as numpy; int32
        data is returned as uint32."""
        import torch

        b = self._bufs.get(name)
        if b is None or b.numel() != t.numel() or b.dtype != t.dtype:
            b = torch.empty(t.numel(), dtype=t.dtype, pin_memory=True)
            self._bufs[name] = b
        b.copy_(t.reshape(-1))
        a = b.numpy()
        return a.view(np.uint32) if a.dtype == np.int32 else a

    def release(self):
        self._bufs.clear()


def fbits(a: np.ndarray) -> np.ndarray:
    """float32 bit patterns with every NaN mapped to one canonical pattern
    (IEEE 754 fixes no sign or payload for a NaN an operation generates)."""
    a = np.ascontiguousarray(a)
    b = a.view(np.uint32).copy()
    b[np.isnan(a)] = 0x7FC00000
    return b


def first_mismatches(flags, k: int = 8):
    return [i for i, ok in enumerate(flags) if not ok][:k]
