"""Host-side checks of bench.py that need no GPU: every name its functions read is defined, the
--gpus guard, and the parsing of recorded HBM-traffic lines."""

import ast
import builtins
import importlib.util
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
