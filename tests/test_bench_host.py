"""Host logic of bench.py (no GPU): the algorithmic flop and byte counts the
roofline divides by, the conversion of HBM counter passes into bytes per
launch, the traffic entry's source check, and the one-GPU guard."""
import csv
import json
import os
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_attention_flops_per_launch_i1536():
    # 4 R I^2 H d (Q K^T and P V) + 2 R I H d c (output projection)
    f = bench.attn_kernel_flops(1536, 1536, 128, 4, 32)
    assert f == 4 * 1536 ** 3 * 128 + 2 * 1536 ** 2 * 128 * 128
    assert abs(f - 1.933e12) < 1e9


def test_projection_bytes_per_launch_i1536():
    # read c bf16 values per position, write q, k, v, g (H d fp16 each) and the H-wide fp16 bias
    b = bench.proj_kernel_bytes(1536, 1536, 128, 4, 32)
    per_pos = 128 * 2 + 4 * 128 * 2 + 4 * 2
    assert b == 1536 * 1536 * per_pos
    assert abs(b - 3.04e9) < 1e7


def test_module_flops_add_up():
    f = bench.tri_module_flops(1536, 1536, 128, 4, 32)
    assert f["total"] == pytest.approx(sum(v for k, v in f.items() if k != "total"))
    assert f["attention"] + f["out_proj"] == bench.attn_kernel_flops(1536, 1536, 128, 4, 32)


def _counter_csv(path, counter, rows):
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for i, (name, value) in enumerate(rows):
            w.writerow({"Dispatch_Id": i, "Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


def test_traffic_from_scales_by_the_copy(tmp_path):
    """A 1 GiB copy whose FETCH_SIZE reads half its bytes gives a fetch scale
    of 2; dispatches of each kernel are averaged and scaled to bytes."""
    attn = "_ZN2pa11attn_kernelILi4ELi128ELb0ELi0EEEvPK"
    proj = "_ZN2pa11proj_kernelILi128ELi128ELi512ELi1EEEvPK"
    copy = "__amd_rocclr_copyBuffer"
    kib = 1024.0 * 1024.0
    fetch, write = tmp_path / "f.csv", tmp_path / "w.csv"
    _counter_csv(fetch, "FETCH_SIZE", [(attn, 1000.0), (attn, 3000.0), (proj, 10.0), (copy, kib / 2), (copy, 1.0)])
    _counter_csv(write, "WRITE_SIZE", [(attn, 50.0), (attn, 50.0), (proj, 400.0), (copy, kib)])
    res = bench.traffic_from(str(fetch), str(write), 1024.0, ["cmd"])
    assert res["fetch_scale"] == pytest.approx(2.0)
    assert res["write_scale"] == pytest.approx(1.0)
    a = res["kernels"]["attention"]
    assert a["dispatches"] == 2
    assert a["fetch_bytes_per_launch"] == pytest.approx(2000.0 * 1024 * 2.0)
    assert a["write_bytes_per_launch"] == pytest.approx(50.0 * 1024)
    assert a["hbm_bytes_per_launch"] == pytest.approx(a["fetch_bytes_per_launch"] + a["write_bytes_per_launch"])
    assert a["source_hash"] == bench.kernel_source_hash("attention")
    assert res["kernels"]["projection"]["write_bytes_per_launch"] == pytest.approx(400.0 * 1024)


def test_traffic_from_needs_the_copy(tmp_path):
    fetch, write = tmp_path / "f.csv", tmp_path / "w.csv"
    _counter_csv(fetch, "FETCH_SIZE", [("_ZN2pa11attn_kernelI", 1.0)])
    _counter_csv(write, "WRITE_SIZE", [("_ZN2pa11attn_kernelI", 1.0)])
    with pytest.raises(SystemExit):
        bench.traffic_from(str(fetch), str(write), 1024.0, [])


def test_traffic_entry_only_for_the_measured_sources():
    """The committed summary is reported while the kernel's sources are the
    ones it was measured on, and null (None) once they have changed."""
    with open(bench.TRAFFIC_FILE) as fh:
        t = json.load(fh)
    for kernel in ("attention", "projection"):
        k = t["kernels"][kernel]
        if k["source_hash"] == bench.kernel_source_hash(kernel):
            assert bench.traffic_entry(kernel) == pytest.approx(k["hbm_bytes_per_launch"])
        else:
            assert bench.traffic_entry(kernel) is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_second_roof_counts():
    # one exp2 per (row, head, query, key): 1536^3 * 4 = 1.45e10 per launch
    assert bench.softmax_elements(1536, 1536, 4) == 1536 ** 3 * 4
    # nominal exp2 issue ceiling: 1024 SIMDs x 64 lanes / 8 cycles at 2.4 GHz
    assert bench.PEAK_EXP2_PER_S == pytest.approx(1.96608e13)


def test_stream_rates_i1536():
    s = bench.stream_rates(1536, 1536, 128, 4, 32, attn_ms=3.0, proj_ms=0.75)
    assert s["bias"]["bytes"] == 2 * 4 * 1536 * 1536                      # fp16 [H][Pp][Pp]
    assert s["gate"]["bytes"] == 2 * 1536 * 1536 * 128                     # fp16, H d per pair
    assert s["bias"]["copied_to_lds_bytes_per_attention_launch"] == s["bias"]["bytes"] * 768
    assert s["gate"]["read_gbs_over_attention"] == pytest.approx(s["gate"]["bytes"] / 3e-3 / 1e9)
    # padded sizes: I = 100 pads to 128 positions
    s = bench.stream_rates(100, 100, 128, 4, 32, 1.0, 1.0)
    assert s["bias"]["bytes"] == 2 * 4 * 128 * 128


class _FakeLib:
    """Records enable calls and returns canned marks (two calls of a step)."""

    def __init__(self, marks):
        self.marks, self.enabled = marks, []

    def pairattn_timing_enable(self, on):
        self.enabled.append(on)

    def pairattn_timing_read(self):
        return self.marks


class _FakeEvent:
    def __init__(self, enable_timing=True):
        pass

    def record(self, stream=None):
        pass

    def elapsed_time(self, other):
        return 8.0


class _FakeTorch:
    class cuda:
        Event = _FakeEvent

        @staticmethod
        def synchronize():
            pass


def test_per_kernel_pass_groups_calls_by_pack_mark():
    marks = [("pack", 0.01), ("projection", 0.7), ("attention", 3.0),
             ("pack", 0.01), ("projection", 0.8), ("mask_bits", 0.02), ("attention", 3.2)] * 2
    L = _FakeLib(marks)
    steps = []
    out = bench.per_kernel_pass(L, _FakeTorch, None, lambda: steps.append(1), 2, ("start_", "end_"))
    assert L.enabled == [True, False] and len(steps) == 2
    assert out["_step_ms"] == 4.0
    assert out["start_attention"] == [3.0, 3.0] and out["end_attention"] == [3.2, 3.2]
    assert out["end_mask_bits"] == [0.02, 0.02] and "start_mask_bits" not in out


def test_cpu_info_names_the_host():
    info = bench.cpu_info()
    assert info["logical_cpus"] >= 1
    assert set(info) == {"cpu_model", "logical_cpus", "affinity_cpus"}
