"""Host-side tools around the benchmark (CPU only): the single-GPU guard of bench.py and the
counter summaries: the fabric-bytes figure bench.py reports only while the kernel sources
still hash to what was profiled, the layer-step gaps and the per-dispatch counter means."""
import argparse
import csv
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from gemm_gate_softmax_amd import profile_summary as ps  # noqa: E402


def _csv(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=list(rows[0]))
        w.writeheader()
        w.writerows(rows)
    return str(path)


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]


def test_code_digest_ignores_comments_and_layout():
    a = "int f(int x) {  // the value\n  return x /* doubled */ * 2;\n}\n"
    b = "int f(int x) {\n\n    return x * 2;   }"
    assert ps._code_only(a) == ps._code_only(b)
    assert ps._code_only(a) != ps._code_only(a.replace("* 2", "* 3"))


def _traffic_files(tmp_path, kernel):
    # three dispatches of the kernel (1000 KiB fetched, 500 KiB written each) among others,
    # and a 1 GiB copy whose FETCH_SIZE reads half its bytes and WRITE_SIZE all of them
    fetch = _csv(tmp_path / "f.csv", [
        {"Kernel_Name": kernel + "<x>(args)", "Dispatch_Id": d, "Counter_Value": v}
        for d, v in ((1, 600), (1, 400), (2, 1000), (3, 1000))] +
        [{"Kernel_Name": "other_kernel(int)", "Dispatch_Id": 9, "Counter_Value": 77}])
    write = _csv(tmp_path / "w.csv", [
        {"Kernel_Name": kernel + "<x>(args)", "Dispatch_Id": d, "Counter_Value": 500}
        for d in (1, 2, 3)])
    cf = _csv(tmp_path / "cf.csv", [{"Kernel_Name": "copy", "Dispatch_Id": 1, "Counter_Value": 524288},
                                     {"Kernel_Name": "fill", "Dispatch_Id": 2, "Counter_Value": 3}])
    cw = _csv(tmp_path / "cw.csv", [{"Kernel_Name": "copy", "Dispatch_Id": 1, "Counter_Value": 1048576}])
    return argparse.Namespace(kernel=kernel, workload="synthetic_case", fetch=fetch, write=write,
                              copy_fetch=cf, copy_write=cw, copy_bytes=1 << 30,
                              command=["rocprofv3 --pmc FETCH_SIZE -- python3 bench.py"])


def test_traffic_summary_scales_by_the_copy_and_is_tied_to_the_sources(tmp_path, monkeypatch):
    a = _traffic_files(tmp_path, "expert_gemm_kernel")
    md = tmp_path / "traffic.md"
    md.write_text(ps.traffic_markdown(a))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(md))
    # fetch: 1000 KiB x 1024 x (2^30 / (524288 KiB x 1024)) = 2,048,000 bytes; write 512,000
    assert bench.recorded_traffic("synthetic_case") == 2048000 + 512000
    assert bench.recorded_traffic("another_workload") is None
    monkeypatch.setattr(bench, "kernel_digest", lambda: "0" * 16)
    assert bench.recorded_traffic("synthetic_case") is None


def test_last_dispatches_of_a_kernel(tmp_path):
    trace = _csv(tmp_path / "t.csv", [
        {"Kernel_Name": name, "Start_Timestamp": s, "End_Timestamp": s + d}
        for name, s, d in (("k_a<1>(int)", 100, 5000), ("k_b(int)", 200, 9000),
                           ("k_a<1>(int)", 300, 7000), ("k_a<1>(int)", 50, 1000))])
    assert ps.last_dispatches(trace, "k_a", 2) == [5.0, 7.0]


def test_layer_steps_durations_and_gaps(tmp_path):
    # two layer steps (a, b, c) with a 2 us and a 3 us gap, one unrelated kernel between,
    # and one step holding an excluded kernel
    rows, t = [], 0
    def k(name, dur, gap):
        nonlocal t
        t += gap
        rows.append({"Kernel_Name": name + "(int)", "Start_Timestamp": t, "End_Timestamp": t + dur})
        t += dur
    for _ in range(2):
        k("first_k", 10000, 1000)
        k("mid_k", 5000, 2000)
        k("last_k", 7000, 3000)
        k("other", 1000, 500)
    k("first_k", 10000, 1000)
    k("skip_me", 1000, 0)
    k("last_k", 7000, 0)
    trace = _csv(tmp_path / "t.csv", rows)
    steps = ps.layer_steps(trace, "first_k", "last_k", exclude=("skip_me",))
    assert len(steps) == 2 and [n for n, _, _ in steps[0]] == ["first_k(int)", "mid_k(int)", "last_k(int)"]
    a = argparse.Namespace(trace=trace, first="first_k", last="last_k", exclude=["skip_me"],
                           last_steps=20, title="t", command="c")
    md = ps.steps_markdown(a)
    assert "| 1 | `mid_k(int)` | 5.0 | 2.0 |" in md and "| 2 | `last_k(int)` | 7.0 | 3.0 |" in md
    assert "Step span 27.0 us: kernels 22.0 us, gaps 5.0 us" in md


def test_layer_steps_overlapping_kernels_report_no_negative_gap(tmp_path):
    # the second kernel starts 10 ns before the first ends (the trace's clocks allow it):
    # the kernels' summed time exceeds the step's span, and the gap total stays at 0
    rows = [{"Kernel_Name": "first_k(int)", "Start_Timestamp": 0, "End_Timestamp": 5000},
            {"Kernel_Name": "last_k(int)", "Start_Timestamp": 4990, "End_Timestamp": 9990}]
    trace = _csv(tmp_path / "t.csv", rows)
    a = argparse.Namespace(trace=trace, first="first_k", last="last_k", exclude=None,
                           last_steps=20, title="t", command="c")
    md = ps.steps_markdown(a)
    assert "Step span 10.0 us: kernels 10.0 us, gaps 0.0 us" in md and "-0.0" not in md


def test_counter_means_sum_instances_and_average_last_dispatches(tmp_path):
    k = "void expert_gemm_kernel<moe::bf16_t, 2, 1, 128, 128, 3, 128, false>(...)"
    rows = []
    for disp, base in ((1, 100.0), (2, 10.0), (3, 20.0)):
        for inst in range(2):                     # two instances (e.g. XCDs) per dispatch
            rows.append({"Kernel_Name": k, "Dispatch_Id": disp, "Counter_Name": "TCC_HIT",
                         "Counter_Value": base + inst})
        rows.append({"Kernel_Name": "other", "Dispatch_Id": disp + 10, "Counter_Name": "TCC_HIT",
                     "Counter_Value": 1e9})
    path = _csv(tmp_path / "c.csv", rows)
    means, n = ps.counter_means(str(path), "expert_gemm_kernel<moe::bf16_t, 2, 1", 2)
    assert n == 2
    # dispatches 2 and 3: (10 + 11) and (20 + 21), mean 31
    assert means == {"TCC_HIT": 31.0}


def test_probe_library_exports_its_entry_point_and_rejects_bad_arguments():
    """libmoe_probe.so (memory-path ceilings for bench.py --memory-ceilings) is built beside
    libmoe.so; argument checks run before any HIP call, so they can be exercised on the CPU."""
    import ctypes

    from gemm_gate_softmax_amd import build as B
    assert os.path.exists(B.PROBE_LIB), "run the build first"
    probe = ctypes.CDLL(B.PROBE_LIB)
    f = probe.moe_probe_stream
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_longlong, ctypes.c_int,
                  ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    good = dict(kind=0, waves=4, buf=4096, region=1 << 20, grid=256, iters=1, sink=8192)
    bad = [dict(kind=3), dict(kind=-1), dict(waves=6), dict(buf=0), dict(buf=4100), dict(region=48 * 1024 - 128),
           dict(region=1 << 40),
           dict(grid=0), dict(grid=5000), dict(iters=0), dict(sink=0)]
    for change in bad:
        a = {**good, **change}
        assert f(a["kind"], a["waves"], a["buf"], a["region"], a["grid"], a["iters"], a["sink"],
                 None) == 1, change
    # the library that the product path loads does not contain the probe
    assert not hasattr(ctypes.CDLL(B.LIB), "moe_probe_stream")


def test_variant_builds_take_library_switches_only():
    """build_variant compiles only with -DMOE_... switches and a plain name (it writes into the
    package's _variants folder); anything else is refused before hipcc runs."""
    import pytest

    from gemm_gate_softmax_amd import build as B
    for name, defines in (("ok", ["-O0"]), ("ok", ["-DOTHER=1"]), ("../x", ["-DMOE_K_ROTATE=0"]),
                          ("a b", [])):
        with pytest.raises(ValueError):
            B.build_variant(name, defines)
