"""Host-side checks of bench.py that need no GPU: every name its functions read is defined, the
--gpus guard, and the parsing of recorded HBM-traffic lines."""

import ast
import builtins
import importlib.util
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def _load():
    spec = importlib.util.spec_from_file_location("bench_under_test", BENCH)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_every_name_read_is_bound():
    """A GPU-only code path that calls a function which no longer exists would only fail on the
    GPU; catch it here from the syntax tree (module-level bindings, imports, arguments, locals)."""
    tree = ast.parse(open(BENCH).read())
    bound = set(dir(builtins)) | {"__file__"}
    for node in ast.walk(tree):
        if isinstance(node, (ast.FunctionDef, ast.ClassDef)):
            bound.add(node.name)
        elif isinstance(node, (ast.Import, ast.ImportFrom)):
            bound.update((a.asname or a.name).split(".")[0] for a in node.names)
        elif isinstance(node, ast.arg):
            bound.add(node.arg)
        elif isinstance(node, ast.Name) and isinstance(node.ctx, (ast.Store, ast.Del)):
            bound.add(node.id)
        elif isinstance(node, ast.ExceptHandler) and node.name:
            bound.add(node.name)
    read = {n.id for n in ast.walk(tree) if isinstance(n, ast.Name) and isinstance(n.ctx, ast.Load)}
    assert read <= bound, f"names read but never bound: {sorted(read - bound)}"


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, BENCH, "--gpus", "2"], capture_output=True, text=True, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def test_recorded_traffic_requires_matching_sources(tmp_path, monkeypatch):
    bench = _load()
    # With the profiles as committed the function returns a number or None, never raises.
    v = bench.recorded_traffic("shard_linear_col_silu_mul", "no_such_workload")
    assert v is None


def test_cpu_baseline_fields():
    """The CPU baseline leg on the tiny workload: all-core and one-core runs, the CPU model, and
    GEMM TFLOP/s and reduce GB/s as separate fields."""
    import torch
    spec = importlib.util.spec_from_file_location("bench_mod", BENCH)
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    from tensor_transformer_linear_amd import workloads as wl
    w = wl.TINY_MLP_T2
    inp = wl.mlp_inputs(w, 16, seed=0)
    out = bench.cpu_baseline(torch, w, (inp["X"], inp["Wgu"], inp["Wd"], inp["R"], inp["gamma"]), 8, 0.2)
    assert out["kind"] == "oracle" and out["unit"] == "TFLOP/s" and out["value"] > 0
    assert out["one_core"]["threads"] == 1 and out["cores"] >= 1
    assert out["affinity_cores"] == len(os.sched_getaffinity(0))
    for run in (out["one_core"], out["all_cores"]):
        assert run["gemm_tflops"] > 0 and run["reduce_gbs"] > 0
    assert out["cpu_model"]


def _counter_csv(path, rows, counter):
    import csv
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.writer(f, quoting=csv.QUOTE_ALL)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"])
        for i, (name, grid, kib) in enumerate(rows):
            w.writerow([i, name, grid, counter, kib])


def test_traffic_record_from_counter_files(tmp_path, capsys):
    """The traffic lines come from counter files, scaled by the copy calibration, summed over the
    distinct dispatches of one call, and stamped with the current sources' hash."""
    spec = importlib.util.spec_from_file_location("bench_mod", BENCH)
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    d = tmp_path / "prof"
    col256 = "void ttl::(anonymous namespace)::gemm_bigwave_kernel<1, false, 128, 256>(ttl::GemmParams)"
    col192 = "void ttl::(anonymous namespace)::gemm_bigwave_kernel<1, false, 128, 192>(ttl::GemmParams)"
    row = "void ttl::(anonymous namespace)::gemm_bigwave_kernel<0, false, 128, 256>(ttl::GemmParams)"
    setup = "void at::native::vectorized_elementwise_kernel<4>(int)"
    for counter, factor in (("FETCH_SIZE", 0.5), ("WRITE_SIZE", 1.0)):
        # a copy of 1 MiB that the counter reads as `factor` of its bytes
        _counter_csv(str(d / f"copy_{counter}" / "c_counter_collection.csv"),
                     [("__amd_rocclr_copyBuffer", 4096, 1024 * factor)], counter)
        (d / f"copy_{counter}.log").write_text('{"copy_bytes_per_launch": 1048576, "launches": 5}\n')
        rows = [(setup, 100, 1e6), (col256, 65536, 1000 * factor), (col256, 65536, 1200 * factor),
                (col192, 65536, 500 * factor), (row, 131072, 700 * factor)]
        _counter_csv(str(d / f"pmc_{counter}_kn" / "b_counter_collection.csv"), rows, counter)
    lines = bench.traffic_record(str(d), "abc123")
    out = capsys.readouterr().out
    # per call: mean of the 256-row dispatches (1100 KiB) + the 192-row dispatch (500 KiB), read and
    # written, each scaled back to true bytes
    want = int(round((1100 + 500) * 1024 * 2))
    assert lines == [f"traffic kernel=shard_linear_col_silu_mul workload=llama3_70b_mlp_tp8_rank0_b4096_kn "
                     f"bytes_per_launch={want} source_sha256={bench.traffic_sources_digest()}"]
    assert "taken at commit abc123" in out and "gemm_bigwave_kernel<0, false, 128, 256> grid 131072" in out


def _trace_csv(path, rows):
    """A rocprofv3 kernel-trace CSV: rows of (kernel name, grid workgroups, start ns, end ns)."""
    import csv
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Kernel_Name", "Grid_Size_X", "Workgroup_Size_X", "Start_Timestamp", "End_Timestamp"])
        for name, grid, t0, t1 in rows:
            w.writerow([name, grid * 256, 256, t0, t1])


def test_trace_summary_from_trace_and_counter_files(tmp_path, capsys):
    """One row per single-kernel run: the library's dispatches grouped by kernel and grid (torch's
    set-up kernels ignored), the per-call sum of their averages, the run's graph and eager times
    from its JSON line, and the HBM bytes per call from the counter runs scaled by the copy."""
    spec = importlib.util.spec_from_file_location("bench_mod", BENCH)
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    d = tmp_path / "ops"
    main = "void ttl::(anonymous namespace)::gemm_bigwave_kernel<2, false, 128, 256, false>(ttl::GemmParams)"
    fin = "void ttl::(anonymous namespace)::splitk_finalize_kernel<0>(ttl::GemmParams)"
    setup = "void at::native::(anonymous namespace)::distribution_elementwise_grid_stride_kernel<4>(int)"
    run = d / "llama3_70b_layer_tp8__qkv"
    # two calls: main 50 and 54 us, finalize 10 and 12 us; a torch kernel that must not count
    _trace_csv(str(run / "trace" / "ct_kernel_trace.csv"),
               [(setup, 2048, 0, 900_000), (main, 225, 1_000_000, 1_050_000), (fin, 2720, 1_051_000, 1_061_000),
                (main, 225, 2_000_000, 2_054_000), (fin, 2720, 2_055_000, 2_067_000)])
    (run / "ct.json").write_text(json.dumps({"workload": "llama3_70b_layer_tp8", "tokens": 2176,
                                             "step_us_graph": 70.0,
                                             "kernels": {"qkv": {"us": 71.0, "gbs": 1000.0}}}) + "\n")
    for counter, factor in (("FETCH_SIZE", 0.5), ("WRITE_SIZE", 1.0)):
        _counter_csv(str(d / f"copy_{counter}" / "c_counter_collection.csv"),
                     [("__amd_rocclr_copyBuffer", 4096, 1024 * factor)], counter)
        (d / f"copy_{counter}.log").write_text('{"copy_bytes_per_launch": 1048576, "launches": 5}\n')
        _counter_csv(str(run / f"pmc_{counter}" / "c_counter_collection.csv"),
                     [(setup, 100, 1e6), (main, 225 * 256, 2000 * factor), (main, 225 * 256, 2000 * factor),
                      (fin, 2720 * 256, 500 * factor), (fin, 2720 * 256, 500 * factor)], counter)
    bench.trace_summary(str(d))
    out = capsys.readouterr().out
    row = next(line for line in out.splitlines() if line.startswith("| llama3_70b_layer_tp8"))
    cells = [c.strip() for c in row.strip("|").split("|")]
    assert cells[2] == "qkv"
    assert "`gemm_bigwave_kernel<2, false, 128, 256, false>` 225: 52.0" in cells[3]
    assert "`splitk_finalize_kernel<0>` 2720: 11.0" in cells[3] and "distribution" not in cells[3]
    assert cells[4:7] == ["63.0", "70.0", "71.0"]
    per_call_mb = (2000 + 500) * 1024 / 1e6  # the true bytes: the calibration undoes the counter scale
    assert cells[7] == f"{per_call_mb:.1f}" and cells[8] == f"{per_call_mb:.1f}"
    assert cells[9] == f"{1000.0 * 71.0 * 1e3 / 1e6:.1f}"
