"""The committed measurement summaries under profiles/ belong to the kernel
source in the tree: every rocprofv3 summary records the sha256 of
gca_kernels.hip it was taken on, and each states the command that made it.
Every bench line is one JSON object with the fields the report contract
names (roofline and, where the oracle was timed, cpu_baseline)."""
import glob
import json
import os

import pytest

from geometric_context_attention_amd.profiling import kernel_source_digest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROFILES = os.path.join(ROOT, "profiles")
TEXTS = sorted(glob.glob(os.path.join(PROFILES, "*.txt")))
LINES = sorted(glob.glob(os.path.join(PROFILES, "bench_line_*.json")))


def test_profiles_present():
    assert TEXTS and LINES
    # text summaries and JSON lines only, each a few KB
    for path in glob.glob(os.path.join(PROFILES, "*")):
        assert path.endswith((".txt", ".json", ".md")), path
        assert os.path.getsize(path) < 16 * 1024, path


@pytest.mark.parametrize("path", TEXTS, ids=os.path.basename)
def test_summary_matches_kernel_source(path):
    text = open(path).read()
    digests = [ln.split(":", 1)[1].strip() for ln in text.splitlines()
               if ln.lstrip("# ").startswith("kernel_source_sha256:")]
    assert digests, "no kernel_source_sha256 line"
    assert all(d == kernel_source_digest() for d in digests), "taken on another kernel source"
    assert "rocprofv3" in text, "the command that made it is not stated"


@pytest.mark.parametrize("path", LINES, ids=os.path.basename)
def test_bench_line_fields(path):
    lines = [ln for ln in open(path).read().splitlines() if ln.strip()]
    assert len(lines) == 1
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["value"] > 0 and "workload" in d["config"]
    r = d["roofline"]
    for key in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert key in r, key
    assert r["bound"] in ("hbm", "mfma", "alu")
    assert abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-3
    if "cpu_baseline" in d:
        c = d["cpu_baseline"]
        assert c["kind"] == "oracle" and c["cores"] >= 1 and c["value"] > 0 and c["sample"]
