"""Host-side parts of bench.py: the one-GPU refusal and the HBM-traffic figure
built from two rocprofv3 counter runs (calibrated on a plain copy of known
size, keyed by the kernel source digest)."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr and r.stdout == ""


def _counter_csv(d, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Value"])
        w.writeheader()
        for i, (name, v) in enumerate(rows):
            w.writerow({"Dispatch_Id": i + 1, "Kernel_Name": name, "Counter_Value": v})


@pytest.mark.parametrize("workload", ["decode", "prefill"])
def test_traffic_from_counter_runs(tmp_path, monkeypatch, workload):
    """The copy's counter value fixes bytes per unit: FETCH reads half the copy
    (factor 2), WRITE all of it (factor 1).  Decode averages the timed one-launch
    dispatches; prefill sums the per-kernel means of one moe_expert_ffn call."""
    cal_kib = bench.CAL_BYTES / 1024.0
    if workload == "decode":
        # 2 warmup dispatches, then 3 timed ones, then one past the timed region
        k = "void moe::(anonymous namespace)::ffn_decode_kernel<0, 1>(moe::DecodeArgs)"
        fetch = [("__amd_rocclr_copyBuffer", cal_kib / 2)] + [(k, v) for v in (999, 999, 100, 200, 300, 999)]
        write = [("__amd_rocclr_copyBuffer", cal_kib)] + [(k, v) for v in (999, 999, 10, 20, 30, 999)]
        want_fetch, want_write = 200 * 1024 * 2.0, 20 * 1024.0
        warmup, steps = 2, 3
    else:
        names = ["moe::(anonymous namespace)::schedule_kernel(moe::PrefillArgs, int)",
                 "void moe::(anonymous namespace)::prefill_gate_up_kernel<0, 1, true, true>(moe::PrefillArgs)",
                 "void moe::(anonymous namespace)::prefill_down_kernel<0, 1, true>(moe::PrefillArgs)",
                 "moe::(anonymous namespace)::prefill_combine_kernel(moe::PrefillArgs)",
                 "moe::(anonymous namespace)::plan_kernel(int const*, int, int, int*, int*, int*, int*, int*)"]
        fetch = [("__amd_rocclr_copyBuffer", cal_kib / 2)]
        write = [("__amd_rocclr_copyBuffer", cal_kib)]
        for rep in range(2):  # two calls; per-kernel means are summed (the plan kernel is not counted)
            fetch += [(n, v + rep * 2) for n, v in zip(names, (1, 10, 20, 5, 777))]
            write += [(n, v + rep * 2) for n, v in zip(names, (0, 1, 2, 3, 777))]
        want_fetch = (2 + 11 + 21 + 6) * 1024 * 2.0
        want_write = (1 + 2 + 3 + 4) * 1024.0
        warmup, steps = 0, 2
    fd, wd = str(tmp_path / "fetch"), str(tmp_path / "write")
    _counter_csv(fd, fetch)
    _counter_csv(wd, write)
    tf = str(tmp_path / "traffic.json")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", tf)
    assert bench.traffic_from(fd, wd, workload, warmup, steps) == 0
    r = json.load(open(tf))[workload]
    assert r["fetch_bytes_per_launch"] == pytest.approx(want_fetch)
    assert r["write_bytes_per_launch"] == pytest.approx(want_write)
    assert r["calibration_bytes_per_unit"] == {"FETCH_SIZE": pytest.approx(2.0), "WRITE_SIZE": pytest.approx(1.0)}
    assert bench._traffic(workload) == pytest.approx(want_fetch + want_write)
    # counters taken on other kernel source are not reported
    r["kernel_source_sha"] = "0" * 16
    json.dump({workload: r}, open(tf, "w"))
    assert bench._traffic(workload) is None


def test_source_digest_ignores_comments_only(tmp_path):
    """The traffic file is keyed by the kernel code: comments and blank space
    do not change the key, a changed statement does."""
    a, b, c = tmp_path / "a.hip", tmp_path / "b.hip", tmp_path / "c.hip"
    a.write_text("int f(int x) {\n    return x + 1;  // one more\n}\n")
    b.write_text("/* a note\n   over lines */\nint f(int x) {\n\n    return x + 1;\n}\n")
    c.write_text("int f(int x) {\n    return x + 2;\n}\n")
    assert bench._code_text(str(a)) == bench._code_text(str(b))
    assert bench._code_text(str(a)) != bench._code_text(str(c))
