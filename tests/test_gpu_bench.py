"""The benchmark's one JSON line, produced in this process (bench.main with
its command line patched) on the tiny workload: the keys of the line, the
roofline of the expert-MLP call and the oracle's CPU baseline."""
import json
import sys

import pytest

pytestmark = pytest.mark.gpu

REQUIRED = {"metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
            "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"}


def test_bench_line_tiny(capsys, monkeypatch):
    import bench
    print("[case] bench tiny", flush=True)
    monkeypatch.setattr(sys, "argv", ["bench.py", "--workload", "tiny", "--steps", "3", "--warmup", "1"])
    assert bench.main() == 0
    lines = [l for l in capsys.readouterr().out.splitlines() if l.startswith("{")]
    assert len(lines) == 1
    d = json.loads(lines[0])
    assert REQUIRED <= d.keys()
    assert (d["n_gpus"], d["steps"], d["warmup"]) == (1, 3, 1)
    assert d["value"] > 0 and d["ms_per_step"] > 0 and d["higher_is_better"] is True
    assert d["config"]["workload"] == "tiny" and d["dtype"] == "bf16"
    assert len(d["step_ms_p10_p50_p90"]) == 3
    r = d["roofline"]
    assert r["bound"] in ("hbm", "mfma") and r["unit"] in ("GB/s", "TFLOP/s")
    assert r["achieved"] > 0 and r["peak"] > 0 and r["frac"] == pytest.approx(r["achieved"] / r["peak"], rel=1e-2)
    c = d["cpu_baseline"]
    assert c["kind"] == "oracle" and c["value"] > 0 and c["cores"] >= 1 and c["sample"]
    assert c["cpu_model"]


def test_bench_line_configs_block(capsys, monkeypatch):
    """The default (prefill) line carries the other workloads, each measured the same way with its
    own roofline (here only decode, to keep the test short)."""
    import bench
    print("[case] bench prefill + configs block", flush=True)
    monkeypatch.setattr(bench, "EXTRA_CONFIGS", ("decode",))
    monkeypatch.setattr(sys, "argv", ["bench.py", "--steps", "2", "--warmup", "1", "--no-cpu-baseline"])
    assert bench.main() == 0
    lines = [l for l in capsys.readouterr().out.splitlines() if l.startswith("{")]
    d = json.loads(lines[-1])
    assert d["config"]["workload"] == "prefill" and set(d["configs"]) == {"decode"}
    c = d["configs"]["decode"]
    assert c["workload"] == "decode" and c["active_experts"] > 100 and c["ms_per_step"] > 0
    assert 0 < c["frac_of_hbm_peak"] < 1
    r = c["roofline"]
    assert r["bound"] == "hbm" and r["frac"] == pytest.approx(r["achieved"] / r["peak"], rel=1e-2)
