"""bench.py: on the host, the one-GPU refusal, the hash that ties the committed
counter summary to the kernel source and the CPU-baseline record; on the GPU, one
short run whose JSON line carries every field of the benchmark contract."""
import json
import os
import subprocess
import sys

import pytest

import bench
import fa_inputs as fi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert msg["n_gpus"] == 2 and "one GPU" in msg["error"]


def test_code_only_ignores_comments_and_whitespace_but_not_code():
    a = "int f(int x) {  // doubles\n  return 2 * x; /* the\n result */\n}\n"
    b = "int f(int x) {\n\treturn 2 * x;\n}"
    c = "int f(int x) { return 3 * x; }"
    assert bench.code_only(a) == bench.code_only(b)
    assert bench.code_only(a) != bench.code_only(c)


def test_traffic_record_is_read_only_for_its_workload():
    # another workload never picks up the headline kernel's counter summary
    assert bench.read_traffic("bf16_causal_b1_h32_n4096_d128") is None
    v = bench.read_traffic("bf16_b2_h32_n4096_d128")
    # present exactly when the summary was taken for the kernel source as it stands
    assert v is None or v > 0


def test_cpu_baseline_record():
    rec, parity = bench.cpu_baseline(fi.FP32_SMALL, budget_s=0.01)
    assert rec["kind"] == "oracle" and rec["unit"] == "TFLOP/s"
    assert rec["value"] > 0 and 1 <= rec["cores"] <= min(16, len(os.sched_getaffinity(0)))
    assert rec["sample"].startswith("1 of 1 (b,h) heads of " + fi.FP32_SMALL.name)
    assert rec["cores_available"] == len(os.sched_getaffinity(0)) and rec["cpu"]
    assert parity is None  # no device result to compare


def test_cpu_baseline_parity_of_a_given_result():
    """Handed the oracle's own result (as float32), the parity record passes; a
    planted error in one output element is reported and fails the bound."""
    import numpy as np
    from oracle import attention_ref
    w = fi.FP32_SMALL
    q, k, v = fi.head_qkv(w, 0, 0)
    o, lse = attention_ref(q, k, v, w.causal, w.scale)
    o32, l32 = o.astype(np.float32)[None, None], lse.astype(np.float32)[None, None]
    _, par = bench.cpu_baseline(w, budget_s=0.01, gpu_out=(o32, l32))
    assert par["heads"] == 1 and par["rows"] == w.N and par["pass"]
    o32 = o32.copy()
    o32[0, 0, 7, 3] += 1e-3
    _, par = bench.cpu_baseline(w, budget_s=0.01, gpu_out=(o32, l32))
    assert not par["pass"] and abs(par["max_abs_dO"] - 1e-3) < 1e-6


@pytest.mark.gpu
def test_bench_line_on_the_gpu():
    """One short bench.py run: the JSON line carries the contract's fields."""
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", fi.FP32_SMALL.name,
                        "--steps", "3", "--warmup", "1"], capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    d = json.loads(r.stdout.strip().splitlines()[-1])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1 and d["value"] > 0
    assert d["config"]["workload"] == fi.FP32_SMALL.name
    rf = d["roofline"]
    assert rf["bound"] in ("mfma", "hbm") and rf["achieved"] > 0 and rf["peak"] > 0
    assert abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3
    # value and the roofline come from the same timed launches
    if rf["bound"] == "mfma":
        assert abs(rf["achieved"] - d["value"]) <= 0.01
    c = d["config"]
    assert c["launch_ms_min"] <= c["launch_ms_median"] <= c["launch_ms_p90"] <= c["launch_ms_max"]
    assert c["shader_clock_mhz"] is not None and 100 < c["shader_clock_mhz"] < 3000
    assert d["cpu_baseline"]["kind"] == "oracle" and d["cpu_baseline"]["cores"] >= 1
    assert d["parity_vs_oracle"]["pass"] and d["parity_vs_oracle"]["rows"] == fi.FP32_SMALL.N
