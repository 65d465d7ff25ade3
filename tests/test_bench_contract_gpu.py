"""bench.py's output contract, on a short run: one JSON line with the keys a
driver reads, a roofline object for the forward kernel, a CPU baseline of the
oracle (timed on a few heads so the test stays short), and, as the line's
last key, the five workloads with their timing statistics, rooflines and
errors against the whole oracle."""

import json
import os
import subprocess
import sys

import pytest

from tests.gpu_helpers import say

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_prints_one_json_line_with_the_contract():
    say("bench contract")
    cmd = [sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "3", "--warmup", "1", "--no-sweep",
           "--no-backward", "--no-decode", "--no-wide", "--cpu-heads", "4"]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1, r.stdout[-2000:]
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["value"] > 0 and d["ms_per_step"] > 0 and d["higher_is_better"] is True
    assert d["config"]["workload"] == "short_seq_batch"
    roof = d["roofline"]
    for key in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert key in roof, key
    assert roof["bound"] in ("hbm", "mfma") and 0 < roof["frac"] < 1
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-9
    cpu = d["cpu_baseline"]
    assert cpu["kind"] == "oracle" and cpu["value"] > 0 and cpu["cores"] >= 1 and cpu["sample"]

    assert list(d)[-1] == "per_config"
    pc = d["per_config"]
    assert [e["workload"] for e in pc] == ["tiny", "short_seq_batch", "mid_seq_causal", "long_seq_causal",
                                          "single_seq_stress"]
    for e in pc:
        assert e["steps"] >= 20
        assert 0 < e["ms_min"] <= e["ms_median"] <= e["ms_p90"]
        assert e["tflops"] > 0 and e["roofline"]["bound"] in ("hbm", "mfma") and 0 < e["roofline"]["frac"] < 1
        assert e["ok"] is True and e["err_o"] <= 2e-2 and e["err_lse"] <= 1e-3, e
        assert e["oracle_s"] > 0 and e["cores"] >= 1
    # the block stays compact: a reader of the line's last ~2 KB sees it
    assert len(json.dumps(pc)) < 2200, len(json.dumps(pc))
