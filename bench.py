#!/usr/bin/env python3
"""Benchmark of the gradient-compression hot path on one MI355X.

One step = one pass of every hot-path operation over one batch: the 1G
float32 gradient of the fused-bucket workload (2^30 elements, 128 fusion
buckets of 8,388,608, t = 1e-3):
  1. gc2_quantize_buckets   -- 2-bit quantize + residual, one fused launch
  2. gc2_dequant_reduce     -- sum of W = 16 workers' packed buffers (this
                               step's words are worker 0; 15 more are
                               synthetic buffers with i.i.d. codes)
  3. qsgd_quantize          -- bucketed QSGD, d = 512, s = 7 (per-step seed)
  4. qsgd_dequant
Inputs are generated on the device before the timed region (seeded torch
RNG); a new gradient per step, cycling through up to four buffers.

Prints ONE JSON line.  `value` is the fused 2-bit quantizer's throughput
in elements per second (the metric); the whole step's rate is
`step_elements_per_s`.  `ops` breaks each operation down (elements/s, GB/s
of algorithmic traffic, fraction of the 8 TB/s HBM peak and of the
streaming probe with the same access pattern); `roofline` is the dominant
kernel (the fused 2-bit quantizer) timed with HIP events on the stream it
is launched on; `ceiling` holds the measured practical ceilings (the
runtime's 4 GiB device copy and the library's streaming probes);
`configs` times the four smaller workloads (median and best of at least
10 repetitions); `cpu_baseline` is the CPU oracle on a bounded sample of
the same workload, single-threaded on this host.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "gc2_quantize elements/s and achieved HBM GB/s (% of peak) at 1G fp32 elems"
HBM_PEAK_GBPS = 8000.0
W_WORKERS = 16
SAPS_C = 100.0   # the SAPS page's example keeps 1% of the components
QSGD_D, QSGD_S = 512, 7
# algorithmic HBM bytes per element of each operation
BYTES = {
    "gc2_quantize_buckets": 12.25,                         # g, r in; r, 1/4 B of codes out
    "gc2_dequant_reduce": W_WORKERS * 0.25 + 4.0,          # 16 x 1/4 B in, 4 B out
    "qsgd_quantize": 4.0 + 0.5 + 4.0 / QSGD_D,             # g in; nibble + norm share out
    "qsgd_dequant": 0.5 + 4.0 / QSGD_D + 4.0,              # nibble + norm share in; 4 B out
}
OPS = list(BYTES)
PMC_FILE = os.path.join(ROOT, "profiles", "gc2_quantize_buckets_1G_hbm_traffic.json")
CSRC = os.path.join(ROOT, "gradient_compression_distributed_amd", "csrc")
# the fused quantizer's source: the counters are valid only for this text
KERNEL_SRCS = [os.path.join(CSRC, f) for f in ("gc2_quantize.hip", "gcq_device.h",
                                               "gcq_internal.h")]


PHASE = 32768   # offsets of the views are placed modulo this many bytes


def arena(layout, dev):
    """Views of one device allocation, one per (numel, dtype, phase) in
    `layout`: each starts on a 4 KiB boundary whose offset modulo 32 KiB is
    `phase` (two buffers streamed at the same index, like a gradient and its
    residual, run slower when their addresses agree modulo 32 KiB)."""
    import torch

    offs, total = [], 0
    for numel, dt, phase in layout:
        total = (total + 4095) // 4096 * 4096
        total += (phase - total) % PHASE
        offs.append(total)
        total += numel * torch.tensor([], dtype=dt).element_size()
    buf = torch.empty(total, dtype=torch.uint8, device=dev)
    return [buf[o:o + numel * torch.tensor([], dtype=dt).element_size()].view(dt)
            for o, (numel, dt, _) in zip(offs, layout)]


def kernel_source_sha() -> str:
    h = hashlib.sha256()
    for path in KERNEL_SRCS:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per launch of the fused quantizer from the committed
    rocprofv3 counter summary, if it was taken on the current kernel source."""
    try:
        with open(PMC_FILE) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    if d.get("kernel_source_sha") != kernel_source_sha():
        return None
    return d.get("hbm_bytes_per_launch")


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--no-cpu-baseline", action="store_true",
                   help="skip timing the CPU oracle (profiling runs)")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="target CPU work of the oracle sample")
    p.add_argument("--no-per-bucket", action="store_true",
                   help="skip the 128-launch comparison of the fused quantizer")
    p.add_argument("--no-next", action="store_true",
                   help="skip timing CD-SGD's fused local update + quantize")
    p.add_argument("--no-ceiling", action="store_true",
                   help="skip the device copy and the streaming probes")
    p.add_argument("--no-configs", action="store_true",
                   help="skip timing the four smaller workloads")
    p.add_argument("--config-reps", type=int, default=10,
                   help="timed repetitions per smaller workload (at least 10)")
    return p.parse_args()


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} (WORLD_SIZE={world}) is not "
              "supported: the W workers of the reduce are simulated buffers on one GPU and "
              "the library runs no collectives.", file=sys.stderr, flush=True)
        sys.exit(2)

    import numpy as np
    import torch

    import gradient_compression_distributed_amd as gcq
    from gradient_compression_distributed_amd import workloads as wl

    gcq.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cfg = wl.FUSED_1G
    n, nb, blk = cfg.n, cfg.n // cfg.block, cfg.block
    K, Wm = args.steps, args.warmup

    # ---------------------------------------------------------- setup (untimed)
    # Every buffer of the step is a view into one device allocation, as a
    # flat data-parallel gradient buffer would be.  Where each starts modulo
    # 32 KiB was measured in this layout on two boxes, with the same result:
    # the residual at a multiple of 8 KiB from the gradients (here 0; odd
    # multiples of 4 KiB ran the quantizer 1-3% slower), and the sums 16 KiB
    # off the workers' packed buffers (the reduce 1-2% faster than at 0).
    ngrad = min(K + Wm, 4)
    nw = n // 16
    layout = ([(n, torch.float32, 0)] * ngrad + [(n, torch.float32, 0)] +
              [(nw, torch.int32, 0)] * W_WORKERS + [(n, torch.float32, 16384)] +
              [(gcq.qsgd_num_buckets(n, QSGD_D), torch.float32, 0),
               (gcq.qsgd_nibble_words(n), torch.int32, 0), (n, torch.float32, 0)])
    views = arena(layout, dev)
    grads = views[:ngrad]
    r = views[ngrad]
    words = views[ngrad + 1:ngrad + 1 + W_WORKERS]
    acc, norms, nib, qout = views[ngrad + 1 + W_WORKERS:]
    for i, g in enumerate(grads):
        wl.fill_bucketed_normal_(g, cfg, i)
    r.zero_()
    for w in range(1, W_WORKERS):
        wl.fill_iid_field_words_(words[w], cfg.stream, w)
    wpb = blk // 16
    blists = [gcq.BucketList([(g[b * blk:(b + 1) * blk], r[b * blk:(b + 1) * blk],
                               words[0][b * wpb:(b + 1) * wpb], cfg.t) for b in range(nb)])
              for g in grads]
    torch.cuda.synchronize()

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(OPS) + 1)]
          for _ in range(K)]

    def step(i, events=None):
        g = grads[i % ngrad]
        if events:
            events[0].record()
        gcq.gc2_quantize_buckets(blists[i % ngrad])
        if events:
            events[1].record()
        gcq.gc2_dequant_reduce(words, n, cfg.t, acc=acc)
        if events:
            events[2].record()
        gcq.qsgd_quantize(g, QSGD_D, QSGD_S, wl.qsgd_seed(i), norms=norms, nibbles=nib)
        if events:
            events[3].record()
        gcq.qsgd_dequant(norms, nib, n, QSGD_D, QSGD_S, out=qout)
        if events:
            events[4].record()

    for i in range(Wm):
        step(i)
    torch.cuda.synchronize()

    # ---------------------------------------------------------- timed region
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(K):
        step(Wm + k, ev[k])
    torch.cuda.synchronize()
    t1 = time.perf_counter()

    ms_per_step = (t1 - t0) * 1e3 / K
    op_steps = {op: [ev[k][j].elapsed_time(ev[k][j + 1]) for k in range(K)]
                for j, op in enumerate(OPS)}
    op_ms = {op: sum(v) / K for op, v in op_steps.items()}
    ops = {}
    for op in OPS:
        s = op_ms[op] / 1e3
        gbps = BYTES[op] * n / s / 1e9
        ops[op] = {"ms": round(op_ms[op], 4), "ms_median": round(float(np.median(op_steps[op])), 4),
                   "ms_best": round(min(op_steps[op]), 4), "elements_per_s": n / s,
                   "GBps": round(gbps, 1), "frac_of_peak": round(gbps / HBM_PEAK_GBPS, 4),
                   "bytes_per_element": BYTES[op]}

    # the pair the target names: the quantizer plus the reduce, as one rate
    # over both operations' algorithmic bytes
    pair_s = (op_ms["gc2_quantize_buckets"] + op_ms["gc2_dequant_reduce"]) / 1e3
    pair_bpe = BYTES["gc2_quantize_buckets"] + BYTES["gc2_dequant_reduce"]
    gc2_pair = {"ms": round(pair_s * 1e3, 4), "bytes_per_element": pair_bpe,
                "GBps": round(pair_bpe * n / pair_s / 1e9, 1),
                "frac_of_peak": round(pair_bpe * n / pair_s / 1e9 / HBM_PEAK_GBPS, 4)}

    # fused launch vs 128 per-bucket launches of the same quantizer (untimed
    # by the step clock; events on the same stream)
    if not args.no_per_bucket:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = max(3, K // 2)
        g = grads[0]
        e0.record()
        for _ in range(reps):
            for b in range(nb):
                sl = slice(b * blk, (b + 1) * blk)
                gcq.gc2_quantize(g[sl], r[sl], cfg.t, out=words[0][b * wpb:(b + 1) * wpb])
        e1.record()
        torch.cuda.synchronize()
        per_bucket_ms = e0.elapsed_time(e1) / reps
        ops["gc2_quantize_buckets"]["per_bucket_launches_ms"] = round(per_bucket_ms, 4)
        ops["gc2_quantize_buckets"]["fused_speedup"] = round(
            per_bucket_ms / op_ms["gc2_quantize_buckets"], 3)

    # CD-SGD's local update fused with the quantizer (a widening of the path;
    # timed on its own, outside the step): the fused call, the update alone,
    # and the update plus the single-buffer quantizer as two launches
    next_ops = None
    if not args.no_next:
        cds = wl.CDSGD_1G
        g, wloc = grads[0], qout
        wl.fill_normal_(wloc, cds.stream, 999, cds.w_sigma)
        reps = max(3, K // 2)

        def timed(fn):
            fn()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                fn()
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / reps

        fused_ms = timed(lambda: gcq.cdsgd_update_quantize(g, r, wloc, cds.t, cds.eta,
                                                           out=words[0]))
        upd_ms = timed(lambda: gcq.cdsgd_local_update(g, wloc, cds.eta))
        quant_ms = timed(lambda: gcq.gc2_quantize(g, r, cds.t, out=words[0]))
        next_ops = {}
        for name, ms, bpe in (("cdsgd_update_quantize", fused_ms, 20.25),
                              ("cdsgd_local_update", upd_ms, 12.0)):
            gbps = bpe * n / (ms / 1e3) / 1e9
            next_ops[name] = {"ms": round(ms, 4), "elements_per_s": n / (ms / 1e3),
                              "GBps": round(gbps, 1), "frac_of_peak": round(gbps / HBM_PEAK_GBPS, 4),
                              "bytes_per_element": bpe}
        next_ops["cdsgd_update_quantize"]["separate_launches_ms"] = round(upd_ms + quant_ms, 4)
        next_ops["cdsgd_update_quantize"]["config"] = {"eta": cds.eta, "t": cds.t, "n": n}

        # QSGD with max-norm bucket scales, and the 16-worker decode-average
        mx_ms = timed(lambda: gcq.qsgd_quantize_maxnorm(g, QSGD_D, QSGD_S, wl.qsgd_seed(7),
                                                        scales=norms, nibbles=nib))
        Kw = W_WORKERS
        msgs = [gcq.qsgd_quantize(g, QSGD_D, QSGD_S, wl.qsgd_seed(200 + k)) for k in range(Kw)]
        torch.cuda.synchronize()
        avg_ms = timed(lambda: gcq.qsgd_dequant_average([m[0] for m in msgs], [m[1] for m in msgs],
                                                        n, QSGD_D, QSGD_S, out=qout))
        del msgs
        per_msg = 0.5 + 4.0 / QSGD_D
        for name, ms, bpe in (("qsgd_quantize_maxnorm", mx_ms, 4.0 + per_msg),
                              ("qsgd_dequant_average", avg_ms, Kw * per_msg + 4.0)):
            gbps = bpe * n / (ms / 1e3) / 1e9
            next_ops[name] = {"ms": round(ms, 4), "elements_per_s": n / (ms / 1e3),
                              "GBps": round(gbps, 1), "frac_of_peak": round(gbps / HBM_PEAK_GBPS, 4),
                              "bytes_per_element": round(bpe, 4)}
        next_ops["qsgd_dequant_average"]["config"] = {"K": Kw, "d": QSGD_D, "s": QSGD_S, "n": n}

        # SAPS shared-seed sparsification at c = 100 (99% of the components
        # dropped): mask (+ offsets), gather of the kept components, merge of a
        # peer's; algorithmic bytes count the mask bits and the kept elements
        c_saps, seed_saps = SAPS_C, wl.qsgd_seed(9)
        smask = torch.empty(gcq.saps_mask_words(n), dtype=torch.int32, device=dev)
        soffs = torch.empty(gcq.saps_num_tiles(n) + 1, dtype=torch.int64, device=dev)
        mask_ms = timed(lambda: gcq.saps_mask(n, c_saps, seed_saps, mask=smask, offsets=soffs))
        kept = gcq.saps_count(soffs)
        svals = torch.empty(kept, dtype=torch.float32, device=dev)
        gat_ms = timed(lambda: gcq.saps_gather(g, smask, soffs, values=svals))
        mer_ms = timed(lambda: gcq.saps_merge(wloc, smask, soffs, svals))
        kf = kept / n
        for name, ms, bpe in (("saps_mask", mask_ms, 0.125),
                              ("saps_gather", gat_ms, 0.125 + 8.0 * kf),
                              ("saps_merge", mer_ms, 0.125 + 12.0 * kf)):
            gbps = bpe * n / (ms / 1e3) / 1e9
            next_ops[name] = {"ms": round(ms, 4), "elements_per_s": n / (ms / 1e3),
                              "GBps": round(gbps, 1), "bytes_per_element": round(bpe, 4)}
        next_ops["saps_mask"]["config"] = {"c": c_saps, "n": n, "kept": kept}
        del smask, soffs, svals

        # Elias-omega coding of the QSGD output (d = 512, s = 7) and its decode
        gcq.qsgd_quantize(g, QSGD_D, QSGD_S, wl.qsgd_seed(11), norms=norms, nibbles=nib)
        eoffs = torch.empty(gcq.qsgd_num_buckets(n, QSGD_D) + 1, dtype=torch.int64, device=dev)
        ewords = torch.empty(gcq.qsgd_elias_max_words(n, QSGD_D), dtype=torch.int32, device=dev)
        enc_ms = timed(lambda: gcq.qsgd_elias_encode(norms, nib, n, QSGD_D, offsets=eoffs,
                                                     out=ewords))
        coded_bits = int(eoffs[-1].item())
        nib2 = torch.empty_like(nib)
        norms2 = torch.empty_like(norms)
        dec_ms = timed(lambda: gcq.qsgd_elias_decode(ewords, eoffs, n, QSGD_D, norms=norms2,
                                                     nibbles=nib2))
        per_msg = 0.5 + 4.0 / QSGD_D
        for name, ms, bpe in (("qsgd_elias_encode", enc_ms, per_msg + coded_bits / 8 / n),
                              ("qsgd_elias_decode", dec_ms, coded_bits / 8 / n + per_msg)):
            gbps = bpe * n / (ms / 1e3) / 1e9
            next_ops[name] = {"ms": round(ms, 4), "elements_per_s": n / (ms / 1e3),
                              "GBps": round(gbps, 1), "bytes_per_element": round(bpe, 4)}
        next_ops["qsgd_elias_encode"]["config"] = {"d": QSGD_D, "s": QSGD_S, "n": n,
                                                   "coded_bits_per_element": coded_bits / n}
        del eoffs, ewords, nib2, norms2

    # practical ceilings, after everything else (they overwrite the step's
    # buffers): the runtime's 4 GiB device copy, and the library's probes
    # with the exact access patterns of the quantizer and the reduce on the
    # same buffers (no arithmetic)
    ceiling = None
    if not args.no_ceiling:
        ceiling = measure_ceilings(gcq, np, torch, n, grads, r, words, acc, qout)
        ops["gc2_quantize_buckets"]["frac_of_probe"] = round(
            ops["gc2_quantize_buckets"]["GBps"] / ceiling["probe_quantize_GBps"], 4)
        ops["gc2_dequant_reduce"]["frac_of_probe"] = round(
            ops["gc2_dequant_reduce"]["GBps"] / ceiling["probe_reduce_GBps"], 4)

    configs = None
    if not args.no_configs:
        configs = time_configs(args, gcq, wl, np, torch, dev)

    q_ms = op_ms["gc2_quantize_buckets"]
    achieved = BYTES["gc2_quantize_buckets"] * n / (q_ms / 1e3) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                "traffic": measured_traffic(), "kernel": "gc2_quantize_kernel (fused table)",
                "algorithmic_bytes_per_launch": BYTES["gc2_quantize_buckets"] * n,
                "avg_launch_ms": round(q_ms, 4)}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(args, cfg, grads[0], words, np, torch, wl)

    line = {
        "metric": METRIC, "value": ops["gc2_quantize_buckets"]["elements_per_s"],
        "unit": "elements/s",
        "n_gpus": 1, "steps": K, "warmup": Wm, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic (seeded device RNG; per-bucket N(0, sigma_b^2), "
                "sigma_b log-uniform in [1e-5, 1e-2]; i.i.d. worker codes)",
        "config": {"workload": "fused-bucket 2-bit quantize + 16-worker dequant-reduce + "
                               "QSGD d=512 s=7 quantize/dequant over one 1G-element gradient",
                   "n": n, "buckets": nb, "bucket_elems": blk, "t": cfg.t,
                   "workers": W_WORKERS, "qsgd_d": QSGD_D, "qsgd_s": QSGD_S},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "ops": ops,
        "next_ops": next_ops,
        "step_elements_per_s": n / (ms_per_step / 1e3),
        "gc2_quantize_plus_dequant_reduce": gc2_pair,
        "ceiling": ceiling,
        "configs": configs,
        "device": torch.cuda.get_device_name(dev),
    }
    print(json.dumps(line), flush=True)


def measure_ceilings(gcq, np, torch, n, grads, r, words, acc, out, reps=10):
    """GB/s of the runtime's 4 GiB device copy and of the library's probes
    (median of `reps` launches, HIP events on the current stream)."""
    def med(fn, bpe):
        ts = _event_times(torch, lambda i: fn(), 2, reps)
        return round(bpe * n / (float(np.median(ts)) / 1e3) / 1e9, 1)

    return {
        "device_copy_GBps": med(lambda: out.copy_(grads[0]), 8.0),
        "probe_copy_GBps": med(lambda: gcq.probe_stream(grads[0], out), 8.0),
        "probe_quantize_GBps": med(lambda: gcq.probe_stream(grads[0], r, b=r, words=words[0]),
                                   BYTES["gc2_quantize_buckets"]),
        "probe_reduce_GBps": med(lambda: gcq.probe_reduce(words, n, acc),
                                 BYTES["gc2_dequant_reduce"]),
        "note": "device_copy: torch copy_ of 4 GiB (the runtime's copy kernel); probe_copy: "
                "the library's float4 copy in the quantizer's geometry; probe_quantize: the "
                "quantizer's streams (g read, r read and written in place, packed words "
                "written) with no arithmetic; probe_reduce: the reduce's own kernel with the "
                "decode replaced by an XOR; all at 2^30 elements on the step's buffers",
    }


def _event_times(torch, fn, warm, reps):
    """Per-call HIP-event times (ms) of `fn(i)` on the current stream for
    i = warm .. warm + reps - 1, after `warm` untimed calls."""
    for i in range(warm):
        fn(i)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    for k in range(reps):
        ev[k][0].record()
        fn(warm + k)
        ev[k][1].record()
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in ev]


def _summary(np, ts, n, bpe):
    med, best = float(np.median(ts)), float(min(ts))
    gbps = bpe * n / (med / 1e3) / 1e9
    return {"ms_median": round(med, 4), "ms_best": round(best, 4), "reps": len(ts),
            "elements_per_s": n / (med / 1e3), "GBps": round(gbps, 1),
            "frac_of_peak": round(gbps / HBM_PEAK_GBPS, 4), "bytes_per_element": round(bpe, 4)}


def time_configs(args, gcq, wl, np, torch, dev):
    """The four smaller workloads, each op timed per call with HIP events
    (median and best of `reps`; inputs resident on the device; multi-step
    workloads cycle through their steps, the residual carried).  Their
    working sets fit partly in the 256 MB last-level cache, so they are
    reported, not used for the roofline."""
    reps = max(10, args.config_reps)
    out = {}
    # 2-bit quantize + residual, 65,541 elements, 3 steps of fresh g
    c1 = wl.GC2_RAGGED_65K
    g1 = [torch.from_numpy(wl.gradient(c1, s)).to(dev) for s in range(c1.steps)]
    r1 = torch.zeros(c1.n, device=dev)
    o1 = torch.empty(gcq.gc2_packed_words(c1.n), dtype=torch.int32, device=dev)
    ts = _event_times(torch, lambda i: gcq.gc2_quantize(g1[i % c1.steps], r1, c1.t, out=o1), 3, reps)
    out["gc2_ragged_65k"] = {"op": "gc2_quantize", "n": c1.n, "t": c1.t,
                             **_summary(np, ts, c1.n, BYTES["gc2_quantize_buckets"])}
    del g1, r1, o1
    # 2-bit quantize + residual, ResNet-50-sized, 10 steps
    c2 = wl.GC2_RESNET50
    g2 = [torch.from_numpy(wl.gradient(c2, s)).to(dev) for s in range(c2.steps)]
    r2 = torch.zeros(c2.n, device=dev)
    o2 = torch.empty(gcq.gc2_packed_words(c2.n), dtype=torch.int32, device=dev)
    ts = _event_times(torch, lambda i: gcq.gc2_quantize(g2[i % c2.steps], r2, c2.t, out=o2), 3, reps)
    out["gc2_resnet50"] = {"op": "gc2_quantize", "n": c2.n, "t": c2.t,
                           **_summary(np, ts, c2.n, BYTES["gc2_quantize_buckets"])}
    del g2, r2, o2
    # dequantize-and-reduce, 16 workers, ResNet-50-sized
    c3 = wl.REDUCE_W16_RESNET50
    nw3 = gcq.gc2_packed_words(c3.n)
    w3 = [torch.empty(nw3, dtype=torch.int32, device=dev) for _ in range(c3.workers)]
    for k, w in enumerate(w3):
        wl.fill_iid_field_words_(w, c3.stream, k)
    a3 = torch.empty(c3.n, device=dev)
    ts = _event_times(torch, lambda i: gcq.gc2_dequant_reduce(w3, c3.n, c3.t, acc=a3), 3, reps)
    out["reduce_w16_resnet50"] = {"op": "gc2_dequant_reduce", "n": c3.n, "W": c3.workers,
                                  "t": c3.t, **_summary(np, ts, c3.n, c3.workers * 0.25 + 4.0)}
    del w3, a3
    # QSGD quantize and dequant, AlexNet-sized, d = 512, s = 7
    c4 = wl.QSGD_ALEXNET
    g4 = torch.from_numpy(wl.gradient(c4, 0)).to(dev)
    nm4 = torch.empty(gcq.qsgd_num_buckets(c4.n, c4.d), device=dev)
    nb4 = torch.empty(gcq.qsgd_nibble_words(c4.n), dtype=torch.int32, device=dev)
    q4 = torch.empty(c4.n, device=dev)
    ts_q = _event_times(torch, lambda i: gcq.qsgd_quantize(g4, c4.d, c4.s, wl.qsgd_seed(i),
                                                           norms=nm4, nibbles=nb4), 3, reps)
    ts_d = _event_times(torch, lambda i: gcq.qsgd_dequant(nm4, nb4, c4.n, c4.d, c4.s, out=q4),
                        3, reps)
    bq = 4.0 + 0.5 + 4.0 / c4.d
    out["qsgd_alexnet"] = {"n": c4.n, "d": c4.d, "s": c4.s,
                           "qsgd_quantize": _summary(np, ts_q, c4.n, bq),
                           "qsgd_dequant": _summary(np, ts_d, c4.n, bq)}
    del g4, nm4, nb4, q4
    torch.cuda.synchronize()
    return out


def cpu_baseline(args, cfg, g_dev, words, np, torch, wl):
    """The CPU oracle as it stands, one thread pinned to one core, on whole
    buckets of the same workload until about --cpu-seconds of work."""
    import oracle

    try:
        os.sched_setaffinity(0, {sorted(os.sched_getaffinity(0))[0]})
    except (AttributeError, OSError):
        pass
    blk = cfg.block
    wpb = blk // 16
    elems = 0
    total = 0.0
    per_op = {op: 0.0 for op in OPS}
    b = 0
    while total < args.cpu_seconds and b < cfg.n // blk:
        g = g_dev[b * blk:(b + 1) * blk].cpu().numpy()
        ws = [w[b * wpb:(b + 1) * wpb].cpu().numpy().view(np.uint32) for w in words]
        r = np.zeros(blk, np.float32)
        t0 = time.perf_counter()
        ws[0] = oracle.gc2_quantize(g, r, cfg.t)
        t1 = time.perf_counter()
        oracle.gc2_dequant_reduce(ws, blk, cfg.t)
        t2 = time.perf_counter()
        norms, nib = oracle.qsgd_quantize(g, QSGD_D, QSGD_S, wl.qsgd_seed(0))
        t3 = time.perf_counter()
        oracle.qsgd_dequant(norms, nib, blk, QSGD_D, QSGD_S)
        t4 = time.perf_counter()
        for op, dt in zip(OPS, (t1 - t0, t2 - t1, t3 - t2, t4 - t3)):
            per_op[op] += dt
        total += t4 - t0
        elems += blk
        b += 1
    # the widened rows, timed the same way on one whole bucket of the same
    # gradient, 2^23 elements (32 MiB per float array, so the streaming rows
    # do not run from the host's caches; inputs that are another row's output
    # are made untimed)
    m = cfg.block
    gs = g_dev[:m].cpu().numpy()
    cds = wl.CDSGD_1G
    rs = np.random.default_rng(7)
    nxt = {}

    def rate(fn):
        t0 = time.perf_counter()
        fn()
        return m / (time.perf_counter() - t0)

    rr, ww = np.zeros(m, np.float32), (rs.standard_normal(m) * cds.w_sigma).astype(np.float32)
    nxt["cdsgd_update_quantize"] = rate(lambda: oracle.cdsgd_update_quantize(gs, rr, ww, cds.t,
                                                                             cds.eta))
    nxt["cdsgd_local_update"] = rate(lambda: oracle.cdsgd_local_update(gs, ww, cds.eta))
    nxt["qsgd_quantize_maxnorm"] = rate(lambda: oracle.qsgd_quantize_maxnorm(gs, QSGD_D, QSGD_S,
                                                                             wl.qsgd_seed(7)))
    msgs = [oracle.qsgd_quantize(gs, QSGD_D, QSGD_S, wl.qsgd_seed(200 + k)) for k in range(W_WORKERS)]
    nxt["qsgd_dequant_average"] = rate(lambda: oracle.qsgd_dequant_average(
        [x[0] for x in msgs], [x[1] for x in msgs], m, QSGD_D, QSGD_S))
    coded = {}
    nxt["qsgd_elias_encode"] = rate(lambda: coded.setdefault(
        "c", oracle.qsgd_elias_encode(msgs[0][0], msgs[0][1], m, QSGD_D)))
    nxt["qsgd_elias_decode"] = rate(lambda: oracle.qsgd_elias_decode(coded["c"][1], coded["c"][0],
                                                                      m, QSGD_D))
    xs = (rs.standard_normal(m)).astype(np.float32)
    kept = {}
    nxt["saps_mask_and_gather"] = rate(lambda: kept.setdefault(
        "v", oracle.saps_gather(xs, SAPS_C, wl.qsgd_seed(5))))
    peer = rs.standard_normal(kept["v"].size).astype(np.float32)
    nxt["saps_merge"] = rate(lambda: oracle.saps_merge(xs, SAPS_C, wl.qsgd_seed(5), peer))

    model = ""
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                model = ln.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": elems / total, "unit": "elements/s", "cores": 1, "kind": "oracle",
            "sample": f"{b} of {cfg.n // blk} buckets ({elems} elements) of the same step: "
                      "all four operations, single thread pinned to one core",
            "seconds": round(total, 3),
            "ops_elements_per_s": {op: elems / s for op, s in per_op.items()},
            "next_ops_elements_per_s": nxt,
            "next_ops_sample": f"{m} elements (one bucket) of the same gradient, each widened "
                               f"operation once (K = {W_WORKERS} messages for the average, "
                               f"c = {SAPS_C} for SAPS); 32 MiB per float array",
            "host_cpus": os.cpu_count(), "cpu_model": model}


if __name__ == "__main__":
    main()
