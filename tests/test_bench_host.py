"""Host-side pieces of bench.py that the reported figures rest on (no GPU):
the algorithmic bytes of a step, the plan -> launch table, the scaling of
rocprofv3 byte counters into HBM bytes, and the single-GPU guard."""

import csv
import json
import os
import subprocess
import sys

import pytest

import bench
from workloads import WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_algorithmic_bytes_of_the_128k_step():
    wl = WORKLOADS["longctx_128k"]
    ab = bench.algorithmic_bytes(wl)
    units = wl.B * wl.Hkv
    # what the method must move per (batch row, KV head) unit: every FP8 code
    # row once (N r bytes) and the M selected K and V rows once (M d 2 2)
    assert units * wl.N * wl.r == 1_073_741_824
    assert units * wl.M * wl.d * 2 * 2 == 268_435_456
    q = wl.B * wl.Hq * wl.d * 2
    P = wl.Hkv * wl.d * wl.r * 4
    assert ab["candidates"] == units * wl.N * wl.r + q + P
    assert ab["select_attend"] == (units * wl.M * 4 + units * wl.M * wl.d * 4 + q
                                   + wl.B * wl.Hq * wl.d * 2)
    # the figure every roofline and GB/s of the 128K step is quoted against
    assert sum(ab.values()) == 1_345_593_472


def test_algorithmic_bytes_scale_with_context_and_budget():
    wl = WORKLOADS["longctx_128k"]
    from workloads import scaled
    a1 = sum(bench.algorithmic_bytes(wl).values())
    a2 = sum(bench.algorithmic_bytes(scaled(wl, N=2 * wl.N)).values())
    a3 = sum(bench.algorithmic_bytes(scaled(wl, M=2 * wl.M)).values())
    units = wl.B * wl.Hkv
    assert a2 - a1 == units * wl.N * wl.r                  # one more N of codes
    assert a3 - a1 == units * wl.M * (wl.d * 4 + 4)        # M more rows and indices


class _StubLib:
    SA_PLAN_CHUNK_EXACT, SA_PLAN_FILTER, SA_PLAN_UNIT, SA_PLAN_SCORES = 0, 1, 2, 3
    SA_STEP_APPEND_BOUND, SA_STEP_CANDIDATES, SA_STEP_MERGE = 1, 2, 3
    SA_STEP_ATTEND, SA_STEP_SELECT_ATTEND = 4, 5

    def __init__(self, plan):
        self.plan = plan

    def sparse_attn_selection_plan(self, sh, n, m):
        return self.plan


@pytest.mark.parametrize("plan,launches,dominant", [
    (2, ["unit_kernel"], "step"),
    (3, ["score_all_kernel", "scores_select_attend_kernel"], "select_attend"),
    (1, ["append_bound_kernel", "filter_kernel", "select_attend_kernel"], "candidates"),
])
def test_step_stages_follow_the_plan(plan, launches, dominant):
    wl = WORKLOADS["longctx_128k"]
    p, stages, nbytes, dom = bench.step_stages(_StubLib(plan), None, wl)
    assert p == plan
    assert [k for _, _, k in stages] == launches
    assert dom == dominant and dom in nbytes
    # every launch plan accounts for the same bytes of the step
    assert sum(nbytes.values()) == sum(bench.algorithmic_bytes(wl).values())


def _counter_csv(path, counter, rows):
    fields = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=fields)
        w.writeheader()
        for disp, name, value in rows:
            w.writerow({"Dispatch_Id": disp, "Kernel_Name": name, "Counter_Name": counter,
                        "Counter_Value": value})


def test_counter_ingestion_scales_by_the_calibration_kernel(tmp_path, monkeypatch):
    calib = "void at::native::vectorized_elementwise_kernel<4, neg_kernel_cuda>(...)"
    kern = "void sa::unit_kernel<128, 32, true>(sa::FilterArgs, ...)"
    fetch, write = tmp_path / "fetch.csv", tmp_path / "write.csv"
    # FETCH_SIZE reads half of the calibration's 1 GiB (scale 2); the kernel's
    # value of one dispatch comes as two rows that must be added
    _counter_csv(fetch, "FETCH_SIZE", [(1, calib, 524288.0), (2, kern, 60.0), (2, kern, 40.0),
                                       (3, kern, 300.0)])
    # WRITE_SIZE reads the calibration's 1 GiB exactly (scale 1)
    _counter_csv(write, "WRITE_SIZE", [(1, calib, 1048576.0), (2, kern, 8.0), (3, kern, 12.0)])
    out = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(out))
    bench.ingest_counters(str(fetch), str(write), 1024)
    e = json.loads(out.read_text())["unit_kernel"]
    assert e["fetch"]["dispatches"] == 2 and e["write"]["dispatches"] == 2
    assert e["fetch"]["scale"] == pytest.approx(2.0) and e["write"]["scale"] == pytest.approx(1.0)
    assert e["fetch"]["bytes_per_launch"] == pytest.approx(200.0 * 1024 * 2.0)
    assert e["write"]["bytes_per_launch"] == pytest.approx(10.0 * 1024)
    assert e["bytes_per_launch"] == round(200.0 * 1024 * 2.0 + 10.0 * 1024)
    # the entry holds for the kernel sources it was taken on, and only those
    assert bench.measured_traffic("unit_kernel", e["source_hash"]) == e["bytes_per_launch"]
    assert bench.measured_traffic("unit_kernel", "0" * 16) is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr or "single MI355X" in r.stderr
