"""Host side of bench.py, on the CPU: more than one GPU is refused before
any GPU work, the step buffers are aligned, disjoint views of one
allocation, and the measured HBM traffic is reported only while the
kernel source matches the one the counters were taken on."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


@pytest.mark.parametrize("argv,env", [(["--gpus", "2"], {}), (["--gpus", "8"], {}),
                                      ([], {"WORLD_SIZE": "2"})])
def test_more_than_one_gpu_is_refused(argv, env):
    e = dict(os.environ, **env)
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv], env=e,
                       capture_output=True, text=True, timeout=120)
    assert p.returncode == 2
    assert "one GPU" in p.stderr
    assert p.stdout == ""          # no JSON line


def test_arena_views_are_aligned_and_disjoint():
    import torch

    layout = [(1000, torch.float32, 0), (3, torch.int32, 4096), (4097, torch.float32, 0),
              (1, torch.int64, 28672), (0, torch.float32, 0), (65, torch.int32, 8192)]
    views = bench.arena(layout, "cpu")
    base = views[0].untyped_storage().data_ptr()
    spans = []
    for v, (numel, dt, phase) in zip(views, layout):
        assert v.dtype == dt and v.numel() == numel and v.is_contiguous()
        if numel == 0:                 # an empty view has no address to check
            continue
        start = v.data_ptr() - base
        assert start % 4096 == 0 and start % bench.PHASE == phase
        spans.append((start, start + numel * v.element_size()))
    spans.sort()
    for (a0, a1), (b0, _) in zip(spans, spans[1:]):
        assert a1 <= b0
    for i, v in enumerate(views):      # writes land in their own view only
        v.fill_(i + 1)
    for i, v in enumerate(views):
        assert bool((v == i + 1).all())


def test_traffic_only_for_the_profiled_source(monkeypatch, tmp_path):
    rec = {"kernel_source_sha": "0123456789abcdef", "hbm_bytes_per_launch": 123.0}
    f = tmp_path / "pmc.json"
    f.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "PMC_FILE", str(f))
    monkeypatch.setattr(bench, "kernel_source_sha", lambda: "0123456789abcdef")
    assert bench.measured_traffic() == 123.0
    monkeypatch.setattr(bench, "kernel_source_sha", lambda: "fedcba9876543210")
    assert bench.measured_traffic() is None
    monkeypatch.setattr(bench, "PMC_FILE", str(tmp_path / "absent.json"))
    assert bench.measured_traffic() is None


def test_source_hash_covers_the_quantizer_sources():
    names = sorted(os.path.basename(p) for p in bench.KERNEL_SRCS)
    assert "gc2_quantize.hip" in names
    assert all(os.path.exists(p) for p in bench.KERNEL_SRCS)
    assert len(bench.kernel_source_sha()) == 16
