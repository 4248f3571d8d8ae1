"""bench.py's output contract: one JSON line with the fields the driver and
the reader rely on, a roofline for the dominant kernel, and the CPU-oracle
baseline.  Runs a short bench of the 32K workload in a child process."""
import json
import os
import subprocess
import sys

import pytest
import torch

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def line():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    out = subprocess.run(
        [sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "qwen05b_n32k", "--steps", "2",
         "--warmup", "1", "--cpu-seconds", "1", "--decode-steps", "3", "--consensus-steps", "1",
         "--cumulant-steps", "1", "--tree-beam", "4", "--ties-steps", "1"],
        capture_output=True, text=True, timeout=240, cwd=ROOT)
    assert out.returncode == 0, out.stderr[-2000:]
    lines = [l for l in out.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, out.stdout[-2000:]
    return json.loads(lines[0])


def test_bench_line_has_the_contract_fields(line):
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
              "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
              "roofline", "cpu_baseline"):
        assert k in line, k
    assert line["n_gpus"] == 1 and line["steps"] == 2 and line["warmup"] == 1
    assert line["value"] > 0 and line["ms_per_step"] > 0
    assert line["config"]["workload"] == "qwen05b_n32k"


def test_bench_roofline_and_cpu_baseline(line):
    r = line["roofline"]
    for k in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert k in r, k
    assert r["bound"] in ("hbm", "mfma", "alu")
    assert 0 < r["frac"] < 1 and abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-9
    c = line["cpu_baseline"]
    assert c["kind"] == "oracle" and c["cores"] >= 1 and c["value"] > 0 and c["sample"]


def test_bench_variant_legs_present(line):
    for leg in ("consensus", "cumulant", "tree", "decode", "ties"):
        assert line.get(leg), leg


def test_bench_ties_leg_is_exact(line):
    """Every key equal: every row overflows the survivor lists and must still
    take its lowest blocks."""
    t = line["ties"]
    assert t["lowest_ids"] is True
    assert 0 < t["overflow_tiles"] <= t["overflow_rows"] <= t["rows"]
    assert t["ms_per_layer"] > 0
