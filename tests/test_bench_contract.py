"""bench.py's command-line contract: one JSON line with the fields the
measurement is read from (GPU), and a refusal of more than one GPU (CPU)."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


@pytest.mark.gpu
def test_bench_prints_one_json_line():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    print("case bench: --config tiny --configs radix --steps 3 --warmup 1", flush=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--config", "tiny", "--configs", "radix",
                        "--steps", "3", "--warmup", "1", "--append-steps", "2", "--host-steps", "0", "--zip-reps",
                        "1", "--cpu-seconds", "1", "--cpu-seconds-sub", "0.5"],
                       capture_output=True, text=True, timeout=600, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, lines
    b = json.loads(lines[0])
    for key, kind in (("metric", str), ("value", float), ("unit", str), ("n_gpus", int), ("steps", int),
                      ("warmup", int), ("ms_per_step", float), ("higher_is_better", bool), ("scaling", str),
                      ("dtype", str), ("data", str), ("config", dict), ("roofline", dict),
                      ("cpu_baseline", dict), ("configs", list)):
        assert isinstance(b[key], kind), (key, b.get(key))
    assert b["n_gpus"] == 1 and b["steps"] == 3 and b["warmup"] == 1 and b["higher_is_better"] is True
    assert b["vs_baseline"] is None and b["value"] > 0 and b["ms_per_step"] > 0
    assert "workload" in b["config"] and b["config"]["name"] == "tiny"
    for rec in [b] + b["configs"]:
        roof = rec["roofline"]
        assert roof["bound"] == "hbm" and roof["unit"] == "GB/s" and roof["peak"] == 8000.0
        assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-3
        cpu = rec["cpu_baseline"]
        assert cpu["kind"] == "oracle" and cpu["cores"] >= 1 and cpu["value"] > 0 and cpu["sample"]
        chk = cpu["check"]
        assert chk["pass"] is True and chk["pairs"] == chk["of_pairs"] and chk["max_abs"] < 2e-3
        assert rec["stream_read"]["streams"] >= 1 and rec["stream_read"]["GBps"] > 0
        assert rec["split_ms"] > 0 and rec["step_ms_median"] > 0
    assert [c["name"] for c in b["configs"]] == ["radix"]
