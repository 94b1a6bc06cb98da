"""Host-side logic of bench.py (no GPU): the one-GPU guard, the counter-measured
traffic read from the committed profile summary, and the clipped pixel count
of listed blocks."""
import os
import re
import subprocess
import sys
from types import SimpleNamespace

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

SUMMARY = os.path.join(ROOT, "profiles", "step_kernels_unet256_pmc_traffic.md")


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_traffic_is_reported_only_for_the_sources_it_was_measured_on(monkeypatch):
    fields = dict(line.split(": ", 1) for line in open(SUMMARY).read().splitlines() if ": " in line)
    stored = {k[len("traffic_bytes."):]: int(v) for k, v in fields.items() if k.startswith("traffic_bytes.")}
    assert set(stored) >= {"diff", "reduce_copy", "fused_layer", "gather", "conv_blocks", "scatter"}
    monkeypatch.setattr(bench, "_csrc_hash", lambda: fields["csrc_sha256"].strip())
    assert bench._measured_kernel_traffic() == stored
    monkeypatch.setattr(bench, "_csrc_hash", lambda: "0" * 64)
    assert bench._measured_kernel_traffic() == {}


def test_traffic_table_follows_its_calibration():
    """Each row's measured MB is FETCH_SIZE x (read factor) + WRITE_SIZE x (write
    factor) KiB, the factors being what the 256 MiB copy's counters give."""
    text = open(SUMMARY).read()
    m = re.search(r"FETCH_SIZE reports ([\d.]+) KiB\s+for it and WRITE_SIZE ([\d.]+) KiB", text)
    fetch_cal, write_cal = float(m.group(1)), float(m.group(2))
    f_fac, w_fac = 262144 / fetch_cal, 262144 / write_cal
    rows = [line for line in text.splitlines() if line.startswith("| `sige::")]
    assert len(rows) == 6
    fields = dict(line.split(": ", 1) for line in text.splitlines() if ": " in line)
    for row in rows:
        cells = [c.strip() for c in row.strip("|").split("|")]
        fetch, write, mb = float(cells[3]), float(cells[4]), float(cells[5])
        assert abs((fetch * f_fac + write * w_fac) * 1024 / 1e6 - mb) < 0.011
    assert sum(int(v) for k, v in fields.items() if k.startswith("traffic_bytes.")) > 0


@pytest.mark.parametrize("b", [2, 6, 8])
def test_active_pixels_clip_edge_blocks(b):
    ho = wo = 20
    nby = nbx = -(-ho // b)
    d = SimpleNamespace(nby=nby, nbx=nbx, ho=ho, wo=wo)
    every = list(range(nby * nbx))
    assert bench._active_pixels(SimpleNamespace(tolist=lambda: every), d, b) == ho * wo
    last = [nby * nbx - 1]
    edge = ho - (nby - 1) * b
    assert bench._active_pixels(SimpleNamespace(tolist=lambda: last), d, b) == edge * edge
