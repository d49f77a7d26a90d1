"""Seeded synthetic inputs for the gradient-compression hot path.

This module only draws random numbers.  It holds none of the method's
arithmetic (no thresholds, codes, packing or norms), so the oracle and the
HIP path can both be fed from it without sharing any of the computation.

Every host stream is numpy PCG64 keyed by
``SeedSequence([BASE_SEED, stream, step, block])``, where ``stream`` is the
workload's own seed-stream number.  The workloads are stand-ins for the
pages' settings:

GC2_RAGGED_65K (stream 1)
    gc2, W=1: N=65,541 (a ragged tail of 5 elements), g ~ N(0, 0.5^2) fresh
    per step, r = 0, t = 0.5 (the threshold in the MXNet PR's usage
    examples), 3 steps.
GC2_RESNET50 (stream 2)
    gc2 on a ResNet-50-sized flat gradient (25,557,032 elements, ResNet50's
    25M parameters in the QSGD experiments table): 1,048,576-element blocks,
    each N(0, sigma_b^2), sigma_b log-uniform in [1e-4, 1e-1] (fixed per
    block across steps), values fresh per step; t = 0.01; 10 steps.
REDUCE_W16_RESNET50 (stream 3)
    Dequantize-and-reduce: W = 16 packed buffers of 25,557,032 elements whose
    2-bit fields are i.i.d. with P(11) = P(10) = 0.05, P(00) = 0.9; t = 0.01.
QSGD_ALEXNET (stream 4)
    QSGD: 61,100,840 elements (AlexNet's 62M parameters in the same table)
    ~ N(0, 0.01^2); d = 512, s = 7; one hash seed per step.
FUSED_1G (stream 5)
    Fused buckets: 2^30 elements in 128 buckets of 8,388,608, sigma_b
    log-uniform in [1e-5, 1e-2] per bucket, t = 1e-3, 5 steps.
CDSGD_RESNET50 (stream 6)
    CD-SGD local update + quantize on a gradient drawn like GC2_RESNET50's
    (25,557,032 elements, blocked sigmas in [1e-4, 1e-1], t = 0.01): initial
    local weights ~ N(0, 0.05^2), local learning rate 0.1 and k-step 2
    (CD-SGD section 4, ResNet-50 on ImageNet), 4 iterations.
CDSGD_1G (stream 7)
    The same at 2^30 elements with FUSED_1G's gradient layout (t = 1e-3).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

BASE_SEED = 20261202
SIGMA_STREAM = 0xFFFFFFF  # the "step" slot of the per-block sigma stream


def rng(stream: int, step: int, block: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(
        np.random.SeedSequence([BASE_SEED, stream, step, block])))


@dataclass(frozen=True)
class Config:
    stream: int              # seed-stream number (the SeedSequence key)
    name: str
    n: int
    t: float = 0.0
    steps: int = 1
    block: int = 0           # block / bucket length (0: one block)
    sigma: float = 0.0       # fixed sigma (GC2_RAGGED_65K, QSGD_ALEXNET)
    sigma_lo: float = 0.0    # log-uniform sigma range per block
    sigma_hi: float = 0.0
    workers: int = 1
    d: int = 0
    s: int = 0
    eta: float = 0.0         # CD-SGD local learning rate
    k: int = 0               # CD-SGD k-step
    w_sigma: float = 0.0     # spread of the initial local weights


GC2_RAGGED_65K = Config(1, "gc2 quantize+residual, W=1, ragged tail", 65_541, t=0.5, steps=3,
                        sigma=0.5)
GC2_RESNET50 = Config(2, "gc2 quantize+residual, ResNet-50-sized flat gradient", 25_557_032,
                      t=0.01, steps=10, block=1_048_576, sigma_lo=1e-4, sigma_hi=1e-1)
REDUCE_W16_RESNET50 = Config(3, "dequantize-and-reduce, 16 simulated workers", 25_557_032,
                             t=0.01, workers=16)
QSGD_ALEXNET = Config(4, "QSGD stochastic quantize+dequantize", 61_100_840, sigma=0.01, d=512,
                      s=7)
FUSED_1G = Config(5, "fused-bucket gc2 quantize+residual, 1G elements", 1 << 30, t=1e-3,
                  steps=5, block=8_388_608, sigma_lo=1e-5, sigma_hi=1e-2)
CDSGD_RESNET50 = Config(6, "CD-SGD local update + gc2 quantize, ResNet-50-sized", 25_557_032,
                        t=0.01, steps=4, block=1_048_576, sigma_lo=1e-4, sigma_hi=1e-1,
                        eta=0.1, k=2, w_sigma=0.05)
CDSGD_1G = Config(7, "CD-SGD local update + gc2 quantize, 1G elements", 1 << 30, t=1e-3,
                  steps=5, block=8_388_608, sigma_lo=1e-5, sigma_hi=1e-2, eta=0.1, k=2,
                  w_sigma=0.05)
WORKLOADS = (GC2_RAGGED_65K, GC2_RESNET50, REDUCE_W16_RESNET50, QSGD_ALEXNET, FUSED_1G,
             CDSGD_RESNET50, CDSGD_1G)

WEIGHT_STREAM = 0xFFFFFFE  # the "step" slot of the initial-weight stream


def block_sigmas(cfg: Config) -> np.ndarray:
    """Per-block standard deviations, log-uniform in [sigma_lo, sigma_hi]."""
    nblocks = (cfg.n + cfg.block - 1) // cfg.block
    u = rng(cfg.stream, SIGMA_STREAM, 0).uniform(np.log10(cfg.sigma_lo), np.log10(cfg.sigma_hi),
                                              nblocks)
    return (10.0 ** u).astype(np.float64)


def normal_block(stream: int, step: int, block: int, n: int, sigma: float) -> np.ndarray:
    g = rng(stream, step, block).standard_normal(n, dtype=np.float32)
    g *= np.float32(sigma)
    return g


def gradient(cfg: Config, step: int) -> np.ndarray:
    """The whole float32 gradient of a workload at a step (host memory)."""
    if cfg.block == 0:
        return normal_block(cfg.stream, step, 0, cfg.n, cfg.sigma)
    out = np.empty(cfg.n, dtype=np.float32)
    sig = block_sigmas(cfg)
    for b in range(len(sig)):
        lo = b * cfg.block
        hi = min(lo + cfg.block, cfg.n)
        out[lo:hi] = normal_block(cfg.stream, step, b, hi - lo, sig[b])
    return out


def gradient_block(cfg: Config, step: int, b: int) -> np.ndarray:
    """One block (bucket) of a blocked workload's gradient."""
    sig = block_sigmas(cfg)
    lo = b * cfg.block
    hi = min(lo + cfg.block, cfg.n)
    return normal_block(cfg.stream, step, b, hi - lo, sig[b])


def initial_weights(cfg: Config) -> np.ndarray:
    """Initial local weights of a CD-SGD workload, N(0, w_sigma^2)."""
    return normal_block(cfg.stream, WEIGHT_STREAM, 0, cfg.n, cfg.w_sigma)


def iid_field_words(gen: np.random.Generator, nwords: int, p11: float = 0.05,
                    p10: float = 0.05) -> np.ndarray:
    """Random 32-bit words whose sixteen 2-bit fields are i.i.d.:
    0b11 with probability p11, 0b10 with p10, else 0b00 (probabilities
    rounded to multiples of 2^-16).

    Fields are independent and identically distributed, so which field goes
    to which bit pair does not matter; field k is put at bits 2k..2k+1."""
    c11 = int(round(p11 * 65536))
    c10 = int(round((p11 + p10) * 65536))
    out = np.empty(nwords, dtype=np.uint32)
    chunk = 1 << 20
    for lo in range(0, nwords, chunk):
        hi = min(lo + chunk, nwords)
        u = gen.integers(0, 65536, size=(hi - lo) * 16, dtype=np.uint16)
        f = ((u < c10).astype(np.uint8) << 1) | (u < c11).astype(np.uint8)
        f = f.reshape(hi - lo, 4, 4)
        byte = f[:, :, 0] | (f[:, :, 1] << 2) | (f[:, :, 2] << 4) | (f[:, :, 3] << 6)
        out[lo:hi] = np.ascontiguousarray(byte).view("<u4").ravel()
    return out


def worker_words(cfg: Config, worker: int, nwords: int) -> np.ndarray:
    return iid_field_words(rng(cfg.stream, 0, worker), nwords)


def qsgd_seed(step: int) -> int:
    """64-bit hash seed of a QSGD step."""
    return (BASE_SEED << 24) | (step & 0xFFFFFF)


def qsgd_spiky(n: int, d: int, seed: int) -> np.ndarray:
    """Buckets holding 1..8 large entries of random sign over small noise, so
    that every level 0..s occurs (a plain Gaussian bucket almost never goes
    past level 2)."""
    gen = np.random.Generator(np.random.PCG64(np.random.SeedSequence([BASE_SEED, 44, seed])))
    g = gen.standard_normal(n, dtype=np.float32) * np.float32(1e-4)
    nb = (n + d - 1) // d
    for b in range(nb):
        lo, hi = b * d, min(b * d + d, n)
        k = int(gen.integers(1, 9))
        k = min(k, hi - lo)
        pos = lo + gen.choice(hi - lo, size=k, replace=False)
        mag = gen.uniform(0.05, 1.0, size=k).astype(np.float32)
        sgn = np.where(gen.random(k) < 0.5, -1.0, 1.0).astype(np.float32)
        g[pos] = mag * sgn
    return g


# ---------------------------------------------------------------------------
# Device-side generation (torch) for the 1G-element benchmark workload, where
# drawing 4 GiB per step on the host would dominate the run.  Same shapes and
# distributions, a torch (Philox) stream seeded from the same base seed.
# ---------------------------------------------------------------------------

def device_generator(stream: int, step: int, device="cuda"):
    import torch

    gen = torch.Generator(device=device)
    gen.manual_seed((BASE_SEED * 1000 + stream * 100 + step) & 0x7FFFFFFFFFFFFFFF)
    return gen


def fill_bucketed_normal_(out, cfg: Config, step: int):
    """Fill a device float32 tensor of cfg.n elements with the workload's
    per-bucket N(0, sigma_b^2) gradient."""
    import torch

    gen = device_generator(cfg.stream, step, out.device)
    sig = torch.tensor(block_sigmas(cfg), dtype=torch.float32, device=out.device)
    nb = len(sig)
    for b in range(nb):
        lo = b * cfg.block
        hi = min(lo + cfg.block, cfg.n)
        seg = out[lo:hi]
        seg.normal_(0.0, 1.0, generator=gen)
        seg.mul_(sig[b])
    return out


def fill_normal_(out, stream: int, slot: int, sigma: float):
    """Fill a device float32 tensor with N(0, sigma^2) from the workload's
    device stream, at step slot `slot`."""
    gen = device_generator(stream, slot, out.device)
    out.normal_(0.0, 1.0, generator=gen)
    out.mul_(sigma)
    return out


def fill_iid_field_words_(out, stream: int, worker: int, p11: float = 0.05, p10: float = 0.05):
    """Device twin of iid_field_words: fill an int32 tensor with words whose
    16 two-bit fields are i.i.d. (field k at bits 2k..2k+1)."""
    import torch

    gen = device_generator(stream, 1000 + worker, out.device)
    chunk = 1 << 22
    shifts = (2 * torch.arange(16, device=out.device, dtype=torch.int64))
    for lo in range(0, out.numel(), chunk):
        hi = min(lo + chunk, out.numel())
        u = torch.rand((hi - lo, 16), generator=gen, device=out.device)
        f = torch.where(u < p11, 3, torch.where(u < p11 + p10, 2, 0)).to(torch.int64)
        w = (f << shifts).sum(dim=1)
        out[lo:hi] = (w - ((w >> 31) << 32)).to(torch.int32)
    return out
