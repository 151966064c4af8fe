"""bench.py's output contract: one JSON line with the fields the benchmark driver
reads, a roofline object whose fraction is achieved / peak, and a refusal of more
than one GPU (this path runs one GPU's stage)."""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def test_more_than_one_gpu_is_refused_with_a_message():
    res = subprocess.run([sys.executable, BENCH, "--gpus", "2"], capture_output=True, text=True,
                         timeout=300)
    assert res.returncode != 0
    assert res.stdout.strip() == ""
    assert "one GPU" in res.stderr


@pytest.mark.gpu
def test_c2_json_line_has_the_contract_fields():
    res = subprocess.run([sys.executable, "-u", BENCH, "--workload", "c2", "--steps", "2",
                          "--warmup", "1", "--no-cpu-baseline"],
                         capture_output=True, text=True, timeout=600, cwd=ROOT)
    assert res.returncode == 0, res.stderr[-2000:]
    lines = [l for l in res.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, res.stdout
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 2 and d["warmup"] == 1
    assert d["value"] > 0 and d["ms_per_step"] > 0 and d["higher_is_better"] is True
    assert d["dtype"] == "bf16" and "workload" in d["config"]
    r = d["roofline"]
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s" and r["peak"] == 2500.0
    assert abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-3
    assert r["kernel"] == "attn_bf16_kernel" and r["kernel_version"].startswith("attn-")


def test_traffic_tables_are_backed_by_profiles():
    """The HBM traffic bench.py reports is keyed by kernel version: every version in its
    tables has a counter summary under profiles/ that names it, and a library version
    with no entry (the kernel changed since the counters were taken) reports null."""
    import glob
    import re
    sys.path.insert(0, ROOT)
    import bench
    src = open(os.path.join(ROOT, "streaming_causal_video_amd", "csrc", "la_api.cpp")).read()
    tags = re.search(r'la_version\(void\) \{ return "([^"]*)"', src).group(1).split()
    attn = [t for t in tags if t.startswith("attn-")]
    fp8 = [t for t in tags if t.startswith("fp8-")]
    assert len(attn) == 1 and len(fp8) == 1, tags
    profiles = "".join(open(f).read() for f in glob.glob(os.path.join(ROOT, "profiles", "*")))
    for table in (bench.ATTN_TRAFFIC_BYTES, bench.FP8_TRAFFIC_BYTES):
        for version in table:
            assert re.search(rf"\b{re.escape(version)}\b", profiles), version
    assert bench.ATTN_TRAFFIC_BYTES.get("attn-v0") is None
