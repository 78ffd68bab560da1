#!/usr/bin/env python3
"""Throughput of one tensor-parallel rank's MLP shard on one MI355X (simulated ranks in one HBM).

One step = the whole hot path for rank 0 of t = 8 at the Llama-3-70B shape (hidden 8192,
intermediate 28672, 3584 per rank), over one batch of tokens:
  1. shard_linear_col   gate_up column GEMM with the fused SiLU(gate)·up epilogue -> act [b, 3584]
  2. shard_linear_row   down_proj row GEMM -> rank 0's partial [b, 8192] inside P[8, b, 8192]
  3. reduce_partials_rmsnorm   sum of the 8 partials + residual, RMSNorm -> residual_out, y
The other seven ranks' partials are computed once before timing (their work is identical in
shape to rank 0's and would run on the other GPUs).  The weight is the logical W[k, n] of the
statement Y = X·W, stored as W[k][n] (--layout kn, the default), transposed as W^T[n][k]
(--layout nk, the storage of PyTorch-style Linear weights), or packed in 64 x 128 blocks whose
128-column strips are contiguous (--layout blk, packed once before timing).

The secondary 64-token decode line cycles the simulated rank from step to step, so that successive
steps read different weight slices (1.4 GB in all) and the timing is not served from the 256-MB
Infinity Cache.  It is timed eagerly and, as a decode loop would run it, captured once into a HIP
graph (eight steps, one per rank) and replayed.

Inputs are synthetic and seeded (X, R ~ N(0,1); W ~ N(0,0.02); gamma ~ N(1,0.1); bf16), drawn on the
device and resident in HBM before the timed region.  The JSON line reports whole-step throughput as
algorithmic GEMM TFLOP/s (2·b·k·n per GEMM), each kernel's own time from HIP events recorded on the
stream the kernels run on, the dominant kernel against its roofline, and the CPU oracle timed on a
bounded sample of the same work.
"""

from __future__ import annotations

import argparse
import hashlib
import math
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak (2.5 PFLOP/s)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E (8 TB/s)


# Kernel sources whose HBM traffic counters are recorded under profiles/: the recorded figures
# apply only while these files are unchanged.
TRAFFIC_SOURCES = ("tensor_transformer_linear_amd/csrc/gemm_bigwave.hip",
                   "tensor_transformer_linear_amd/csrc/gemm_bigwave16.hip",
                   "tensor_transformer_linear_amd/csrc/gemm_common.h",
                   "tensor_transformer_linear_amd/csrc/gemm_plan.hip",
                   "tensor_transformer_linear_amd/csrc/kernels.h")


# The Infinity Cache holds 256 MB: HBM-bound kernels whose operands are smaller are timed over
# enough copies of them, used in turn, that each launch reads at least this many distinct bytes.
CACHE_COLD_BYTES = 512e6
MAX_ROTATION_COPIES = 64


def rotation_copies(bytes_per_launch):
    """Copies of a launch's operands that make successive launches read >= CACHE_COLD_BYTES."""
    return int(max(1, min(MAX_ROTATION_COPIES, math.ceil(CACHE_COLD_BYTES / max(bytes_per_launch, 1.0)))))


def cache_label(copies, bytes_per_launch):
    total = copies * bytes_per_launch
    if total >= CACHE_COLD_BYTES:
        return (f"cold: {copies} operand copies used in turn ({total / 1e6:.0f} MB)" if copies > 1 else
                f"cold: operands {bytes_per_launch / 1e6:.0f} MB per launch")
    return (f"warm: {copies} operand copies ({total / 1e6:.1f} MB) fit the 256-MB Infinity Cache; "
            f"a fixed cost bounds this launch")


def gemm_flops(b, k, n):
    return 2.0 * b * k * n


def col_silu_bytes(b, k, n_act):
    # X read once, the rank's gate and up weight columns read once, act written once (bf16)
    return 2.0 * (b * k + k * 2 * n_act + b * n_act)


def row_bytes(b, k_r, n):
    return 2.0 * (b * k_r + k_r * n + b * n)


def reduce_bytes(t, b, n, residual=True):
    # t partials + residual read, gamma read, residual_out and y written (bf16)
    return 2.0 * (t * b * n + (b * n if residual else 0) + n + 2 * b * n)


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--settle-ms", type=float, default=100.0,
                    help="before the warm-up steps, repeat the step for this long (untimed) so that the "
                         "GPU's clock, which starts from idle, reaches its loaded steady state")
    ap.add_argument("--batch", type=int, default=4096, help="tokens per step (4096 prefill; 64 decode)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true", help="skip the secondary 64-token decode line")
    ap.add_argument("--layout", choices=("kn", "nk", "blk"), default="kn",
                    help="weight storage: kn = W[k][n], nk = W^T[n][k], blk = 64 x 128 blocks")
    ap.add_argument("--cpu-rows", type=int, default=32, help="token rows in the CPU oracle sample")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="CPU oracle time per core setting (all cores, then one core): 80 %% GEMMs, 20 %% reduce")
    ap.add_argument("--no-yardstick", action="store_true",
                    help="skip timing torch.matmul (hipBLASLt) on the same GEMM shapes")
    ap.add_argument("--no-power", action="store_true",
                    help="skip sampling socket power and GFX clock while the step repeats (6 s)")
    ap.add_argument("--steady-state", action="store_true",
                    help="only run each b=4096 GEMM (ours and hipBLASLt's) back to back for 2 s, sample "
                         "power and clock, time 30 launches, print one JSON line per GEMM and exit")
    ap.add_argument("--config-table", action="store_true",
                    help="only time every kernel of one rank's step for each of the five workloads "
                         "(tiny MLP, 8B MLP b=1/32/256, 8B attention, 70B MLP b=4096/64, 70B layer), "
                         "print one JSON line per workload and exit")
    ap.add_argument("--workload", default=None,
                    help="with --config-table: only this workload (e.g. llama3_8b_attn_tp4), optionally "
                         "with the token count after a colon (llama3_8b_mlp_tp8:256)")
    ap.add_argument("--op", default=None,
                    help="with --config-table --workload: run and time only this kernel of the step "
                         "(e.g. qkv, o_proj, gate_up_silu, down, reduce_rmsnorm): under a kernel trace, "
                         "every dispatch then belongs to it")
    ap.add_argument("--no-graph", action="store_true",
                    help="with --config-table: skip the HIP-graph replay (for counter runs)")
    ap.add_argument("--trace-summary", metavar="DIR", default=None,
                    help="only summarise rocprofv3 kernel traces found under DIR (one sub-directory per "
                         "--config-table --op run, holding its *_kernel_trace.csv and the run's JSON line "
                         "in ct.json) as markdown rows: the kernels of one call with their average "
                         "durations, their sum, and the call's graph and eager times; then exit")
    ap.add_argument("--traffic-record", metavar="DIR", default=None,
                    help="only summarise rocprofv3 FETCH_SIZE / WRITE_SIZE runs found under DIR "
                         "(pmc_<COUNTER>_<layout>/ of this bench's b=4096 step, copy_<COUNTER>/ of "
                         "--copy-calibration-mib) into HBM bytes per call and print the traffic lines "
                         "for profiles/, stamped with the current kernel sources' hash, then exit")
    ap.add_argument("--commit", default="", help="with --traffic-record: the commit the counters were taken at")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (5 times) and exit: the "
                         "reference for scaling HBM traffic counters")
    return ap.parse_args()


def layout_code(ttl, layout):
    return {"kn": ttl.W_KN, "nk": ttl.W_NK, "blk": ttl.W_BLOCKED}[layout]


def stored_weight(ttl, W, lay):
    """The logical weight W[k, n] in storage `lay` (a copy for nk and blk)."""
    if lay == ttl.W_NK:
        return W.t().contiguous()
    if lay == ttl.W_BLOCKED:
        return ttl.pack_weight_blocked(W)
    return W


def run_mlp(ttl, torch, w, b, steps, warmup, seed, layout, rotate_ranks=False, graph=False, settle_ms=0.0):
    from tensor_transformer_linear_amd import workloads as wl
    dev = "cuda"
    inp = wl.mlp_inputs(w, b, seed=seed, device=dev)
    X, R, gamma, Wgu, Wd = inp["X"], inp["R"], inp["gamma"], inp["Wgu"], inp["Wd"]
    lay = layout_code(ttl, layout)
    # the same logical weights in the chosen storage (set-up, not timed)
    Wgu_s, Wd_s = stored_weight(ttl, Wgu, lay), stored_weight(ttl, Wd, lay)
    t, H, I = w.t, w.hidden, w.intermediate
    Ir = I // t
    sp = ttl.merged_gate_up_split(I, t)
    act = torch.empty((b, Ir), dtype=torch.bfloat16, device=dev)
    P = torch.empty((t, b, H), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()
    # every simulated rank's partial, once
    for r in range(t):
        ttl.shard_linear_col(X, Wgu_s, t, r, sp, ttl.EPI_SILU_MUL, Y=act, stream=stream, w_layout=lay)
        ttl.shard_linear_row(act, Wd_s, t, r, True, P=P[r], stream=stream, w_layout=lay)
    torch.cuda.synchronize()
    # The reduction's operands (partials, residual, outputs) in enough copies, used in turn, that
    # successive steps do not find them in the 256-MB Infinity Cache.
    ncopy = rotation_copies(reduce_bytes(t, b, H))
    Ps = [P] + [P.clone() for _ in range(ncopy - 1)]
    Rs = [R] + [R.clone() for _ in range(ncopy - 1)]
    routs = [torch.empty((b, H), dtype=torch.bfloat16, device=dev) for _ in range(ncopy)]
    ys = [torch.empty((b, H), dtype=torch.bfloat16, device=dev) for _ in range(ncopy)]
    rout, y = routs[0], ys[0]

    def step(i, ev=None, st=None):
        st = stream if st is None else st
        r = i % t if rotate_ranks else 0
        c = i % ncopy
        if ev is not None:
            ev[0].record(st)
        ttl.shard_linear_col(X, Wgu_s, t, r, sp, ttl.EPI_SILU_MUL, Y=act, stream=st, w_layout=lay)
        if ev is not None:
            ev[1].record(st)
        ttl.shard_linear_row(act, Wd_s, t, r, True, P=Ps[c][r], stream=st, w_layout=lay)
        if ev is not None:
            ev[2].record(st)
        ttl.reduce_partials_rmsnorm(Ps[c], gamma, w.eps, Rs[c], residual_out=routs[c], Y=ys[c], stream=st)
        if ev is not None:
            ev[3].record(st)

    # Clock settle: the GPU arrives idle, and its clock governor takes tens of milliseconds of load
    # to reach the steady state of a busy GPU (70B TP=8 step, one box: 702-706 us per step after the
    # 5 warm-up steps alone, 674-677 us after 100 or 400).  The step repeats, untimed, for
    # settle_ms first, synchronising every few steps so that the time is the GPU's.
    t_end = time.perf_counter() + settle_ms / 1e3
    i = 0
    while time.perf_counter() < t_end:
        step(i)
        i += 1
        if i % 4 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    # whole-step timing: nothing but the launches between the two events
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for i in range(steps):
        step(i)
    t1.record(stream)
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / steps
    # per-kernel timing: events recorded on the kernels' stream between the launches, same steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    for i in range(steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    per_step = [[e[j].elapsed_time(e[j + 1]) for e in evs] for j in range(3)]
    k_ms = [sum(v) / steps for v in per_step]
    k_med = [sorted(v)[len(v) // 2] for v in per_step]

    f_col = gemm_flops(b, H, 2 * Ir)
    f_row = gemm_flops(b, Ir, H)
    by_col = col_silu_bytes(b, H, Ir)
    by_row = row_bytes(b, Ir, H)
    by_red = reduce_bytes(t, b, H)
    kern = {
        "shard_linear_col_silu_mul": {"avg_us": k_ms[0] * 1e3, "gflop": f_col / 1e9, "mbytes": by_col / 1e6,
                                      "tflops": f_col / (k_ms[0] * 1e9), "gbs": by_col / (k_ms[0] * 1e6)},
        "shard_linear_row": {"avg_us": k_ms[1] * 1e3, "gflop": f_row / 1e9, "mbytes": by_row / 1e6,
                             "tflops": f_row / (k_ms[1] * 1e9), "gbs": by_row / (k_ms[1] * 1e6)},
        "reduce_partials_rmsnorm": {"avg_us": k_ms[2] * 1e3, "mbytes": by_red / 1e6,
                                    "gbs": by_red / (k_ms[2] * 1e6)},
    }
    for j, (name, d) in enumerate(kern.items()):
        d["median_us"] = k_med[j] * 1e3
        d["frac_mfma_peak"] = d.get("tflops", 0.0) / PEAK_BF16_TFLOPS
        d["frac_hbm_peak"] = d["gbs"] / PEAK_HBM_GBS
    wbytes = 2.0 * H * 2 * I + 2.0 * I * H  # both full weights; each step reads rank r's slices
    kern["shard_linear_col_silu_mul"]["cache"] = kern["shard_linear_row"]["cache"] = (
        f"cold: ranks cycled, {t} weight slices ({wbytes / 1e6:.0f} MB) in turn" if rotate_ranks else
        (f"cold: weights ({wbytes / t / 1e6:.0f} MB) exceed the Infinity Cache" if wbytes / t > CACHE_COLD_BYTES
         else "warm: one weight slice every step"))
    kern["reduce_partials_rmsnorm"]["cache"] = cache_label(ncopy, reduce_bytes(t, b, H))
    res = {"ms_per_step": ms_step, "flops": f_col + f_row, "kernels": kern,
           "tensors": (X, Wgu, Wd, R, gamma), "step": step}
    if graph:
        # The same steps captured once into a HIP graph (one step per simulated rank, as a decode
        # loop would replay them) and replayed: the step time without host launch overhead.  The
        # split-K workspace was allocated by the eager steps above.
        cycle = t if rotate_ranks else 1
        cycle = cycle * ncopy // math.gcd(cycle, ncopy)  # every rank and every operand copy
        g = torch.cuda.CUDAGraph()
        gs = torch.cuda.Stream()
        gs.wait_stream(stream)
        with torch.cuda.stream(gs):  # eager once on the capturing stream: its split-K workspace
            for i in range(cycle):
                step(i, st=gs)
        torch.cuda.synchronize()
        with torch.cuda.stream(gs):
            with torch.cuda.graph(g, stream=gs):
                for i in range(cycle):
                    step(i, st=gs)
        stream.wait_stream(gs)
        g.replay()
        torch.cuda.synchronize()
        replays = max(1, steps // cycle)
        t0.record(stream)
        for _ in range(replays):
            g.replay()
        t1.record(stream)
        torch.cuda.synchronize()
        res["ms_per_step_graph"] = t0.elapsed_time(t1) / (replays * cycle)
    return res


def yardstick(torch, w, layout):
    """torch.matmul (hipBLASLt) on this rank's GEMM shapes, as an off-path reference: the plain
    products only (no SiLU·up, no column map: the rank's weight slice is a separate dense tensor).
    Decode shapes cycle through 8 weight copies so that the Infinity Cache does not hold them."""
    H, Ir = w.hidden, w.intermediate // w.t
    layout = "nk" if layout == "nk" else "kn"  # no blocked storage in hipBLASLt: W[k][n] stands in
    out = {}
    for M, K, N, name in ((4096, H, 2 * Ir, "gate_up_b4096"), (4096, Ir, H, "down_b4096"),
                          (64, H, 2 * Ir, "gate_up_b64"), (64, Ir, H, "down_b64")):
        X = torch.randn(M, K, device="cuda").to(torch.bfloat16)
        copies = 8 if M < 512 else 1
        Ws = [(torch.randn(N, K, device="cuda") * 0.02).to(torch.bfloat16) if layout == "nk"
              else (torch.randn(K, N, device="cuda") * 0.02).to(torch.bfloat16) for _ in range(copies)]
        mm = (lambda i: torch.matmul(X, Ws[i % copies].t())) if layout == "nk" else \
             (lambda i: torch.matmul(X, Ws[i % copies]))
        for i in range(5):
            mm(i)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        n = 20
        e0.record()
        for i in range(n):
            mm(i)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / n * 1e3
        out[name] = {"us": us, "tflops": 2.0 * M * K * N / (us * 1e6)}
        del X, Ws
    return {"library": "torch.matmul (hipBLASLt)", "weight_storage": layout, "shapes": out}


RIDGE_FLOP_PER_BYTE = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)


def _time_chain(torch, ops, reps, warmup):
    """ops: list of (name, fn(i), flops, bytes, cache).  Runs the chain `reps` times (step i passes
    i to every op, which picks its simulated rank and operand copy from it) with HIP events recorded
    between the launches on the launching stream; returns {name: average microseconds}."""
    stream = torch.cuda.current_stream()
    for i in range(warmup):
        for op in ops:
            op[1](i)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(ops) + 1)] for _ in range(reps)]
    for i in range(reps):
        evs[i][0].record(stream)
        for j, op in enumerate(ops):
            op[1](i)
            evs[i][j + 1].record(stream)
    torch.cuda.synchronize()
    return {op[0]: sum(e[j].elapsed_time(e[j + 1]) for e in evs) / reps * 1e3 for j, op in enumerate(ops)}


def config_table(ttl, torch, layout, reps=20, warmup=3, only=None, only_op=None, graph=True):
    """Every kernel of one rank's step for each workload, one JSON line each.  Decode-size batches
    (b < 512) cycle the simulated rank from repetition to repetition, so that the weight slices are
    not served from the Infinity Cache; the reductions rotate their operands (partials, residual,
    outputs) among enough copies that each launch reads at least 512 MB of distinct bytes (at most
    64 copies: the smallest decode reductions stay cache-resident, and say so)."""
    from tensor_transformer_linear_amd import workloads as wl
    dev = "cuda"
    names = {ttl.W_KN: "kn", ttl.W_NK: "nk", ttl.W_BLOCKED: "blk"}

    def storage_for(t, weights):
        """The requested storage, or W[k][n] where a blocked weight would not fit the shapes
        (k % 64, n % 128, and (k / t) % 64 for row weights).  weights: (W, is_row) pairs."""
        lay = layout_code(ttl, layout)
        if lay == ttl.W_BLOCKED and not all(W.shape[0] % 64 == 0 and W.shape[1] % 128 == 0 and
                                            (not row or (W.shape[0] // t) % 64 == 0)
                                            for W, row in weights):
            return ttl.W_KN
        return lay

    def bf(*shape):
        # With a single kernel timed (--op) the chain is not run to fill the buffers, so that a
        # kernel trace holds that kernel's dispatches only: they get random values instead.
        if only_op is not None:
            return torch.randn(shape, device=dev).to(torch.bfloat16)
        return torch.empty(shape, dtype=torch.bfloat16, device=dev)

    class Chain:
        """One rank's chain: the GEMMs cycle the simulated rank when `cycle` > 1; each reduction
        has its own rotation of partial-sum buffers, shared with the row GEMM that fills it."""

        def __init__(self, t, b, H, cycle):
            self.t, self.b, self.H, self.cycle = t, b, H, cycle
            self.ops = []

        def rank(self, i, r=None):
            return i % self.cycle if r is None else r

        def col(self, name, X_of, W, split, epi, Y, n_w, n_out, lay, wbytes):
            b, k = self.b, W.shape[0] if lay != ttl.W_NK else W.shape[1]
            cache = (f"cold: ranks cycled, {self.t} weight slices ({wbytes / 1e6:.0f} MB) in turn" if self.cycle > 1
                     else "as in the step chain (weight slice re-read every repetition)")
            self.ops.append((name, lambda i, r=None: ttl.shard_linear_col(X_of(i), W, self.t, self.rank(i, r), split,
                                                                          epi, Y=Y, w_layout=lay),
                             gemm_flops(b, k, n_w), 2.0 * (b * k + k * n_w + b * n_out), cache))

        def partials(self):
            """A rotation of [t, b, H] partial buffers with their residual and outputs."""
            rb = reduce_bytes(self.t, self.b, self.H)
            n = rotation_copies(rb)
            return {"P": [bf(self.t, self.b, self.H) for _ in range(n)], "rout": [bf(self.b, self.H) for _ in range(n)],
                    "y": [bf(self.b, self.H) for _ in range(n)], "n": n, "bytes": rb}

        def row(self, name, X_of, W, part, k, n, parallel, lay, wbytes):
            b, kr = self.b, k // self.t
            cache = (f"cold: ranks cycled, {self.t} weight slices ({wbytes / 1e6:.0f} MB) in turn" if self.cycle > 1
                     else "as in the step chain (weight slice re-read every repetition)")
            self.ops.append((name, lambda i, r=None: ttl.shard_linear_row(
                X_of(i), W, self.t, self.rank(i, r), parallel, P=part["P"][i % part["n"]][self.rank(i, r)],
                w_layout=lay),
                             gemm_flops(b, kr, n), 2.0 * (b * kr + kr * n + b * n), cache))

        def red(self, name, part, gamma, eps, R_of):
            self.ops.append((name, lambda i, r=None: ttl.reduce_partials_rmsnorm(
                part["P"][i % part["n"]], gamma, eps, R_of(i), residual_out=part["rout"][i % part["n"]],
                Y=part["y"][i % part["n"]]), 0.0, part["bytes"], cache_label(part["n"], part["bytes"])))

    def graph_step_us(ops, cycle, replays=10):
        """The chain for steps 0..cycle-1 captured once into a HIP graph and replayed: the step time
        without host launch overhead (small shapes are otherwise bound by the launch rate)."""
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):  # eager once on the capturing stream: its split-K workspace
            for i in range(cycle):
                for op in ops:
                    op[1](i)
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                for i in range(cycle):
                    for op in ops:
                        op[1](i)
        torch.cuda.current_stream().wait_stream(s)
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(replays):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / (replays * cycle) * 1e3

    def report(wname, b, t, us, ops, graph_us, lay, us_alone=None):
        kern = {}
        for name, _, fl, by, cache in ops:
            u = us[name]
            tf, gbs = fl / (u * 1e6), by / (u * 1e3)
            bound = "mfma" if fl / by > RIDGE_FLOP_PER_BYTE else "hbm"
            frac = lambda tf, gbs: tf / PEAK_BF16_TFLOPS if bound == "mfma" else gbs / PEAK_HBM_GBS
            kern[name] = {"us": u, "tflops": tf, "gbs": gbs, "bound": bound, "frac": frac(tf, gbs), "cache": cache}
            if us_alone is not None:
                # the call alone, repeated in a replayed graph: no host launch cost and no events
                # between launches (the events of the chain's timing add a few us per kernel)
                ua = us_alone[name]
                kern[name].update({"us_graph": ua, "frac_graph": frac(fl / (ua * 1e6), by / (ua * 1e3))})
        print(json.dumps({"workload": wname, "tokens": b, "t": t, "weight_storage": names[lay],
                          "step_us": sum(us.values()), "step_us_graph": graph_us, "kernels": kern}),
              flush=True)

    def run(wname, b, t, chain, parts, lay, keep):
        # every rank's partials into every copy of the rotations, in chain order (not with --op,
        # whose buffers hold random values)
        copies = max(p["n"] for p in parts)
        if only_op is None:
            for c in range(copies):
                for r in range(t):
                    for op in chain.ops:
                        op[1](c, r)
        torch.cuda.synchronize()
        # a whole number of rank cycles and operand rotations per graph
        gcycle = chain.cycle
        for p in parts:
            gcycle = gcycle * p["n"] // math.gcd(gcycle, p["n"])
        ops = chain.ops
        if only_op is not None:
            ops = [op for op in chain.ops if op[0] == only_op]
            if not ops:
                raise SystemExit(f"{wname}: no kernel named {only_op!r} (one of {[op[0] for op in chain.ops]})")
        us = _time_chain(torch, ops, max(reps, gcycle if gcycle <= 64 else reps), warmup)
        alone = {op[0]: graph_step_us([op], min(gcycle, 64)) for op in ops} if graph else None
        report(wname, b, t, us, ops, graph_step_us(ops, min(gcycle, 64)) if graph else float("nan"), lay, alone)

    def wanted(w, b):
        if only is None:
            return True
        name, _, tokens = only.partition(":")
        return w.name == name and (not tokens or int(tokens) == b)

    for w in (wl.TINY_MLP_T2, wl.LLAMA3_8B_MLP_TP8, wl.LLAMA3_70B_MLP_TP8):
        for b in w.batches:
            if not wanted(w, b):
                continue
            inp = wl.mlp_inputs(w, b, seed=0, device=dev)
            t, H, I = w.t, w.hidden, w.intermediate
            Ir = I // t
            lay = storage_for(t, ((inp["Wgu"], False), (inp["Wd"], True)))
            Wgu, Wd = stored_weight(ttl, inp["Wgu"], lay), stored_weight(ttl, inp["Wd"], lay)
            act = bf(b, Ir)
            sp = ttl.merged_gate_up_split(I, t)
            ch = Chain(t, b, H, t if b < 512 else 1)
            part = ch.partials()
            X, R = inp["X"], inp["R"]
            ch.col("gate_up_silu", lambda i: X, Wgu, sp, ttl.EPI_SILU_MUL, act, 2 * Ir, Ir, lay, 2.0 * H * 2 * I)
            ch.row("down", lambda i: act, Wd, part, I, H, True, lay, 2.0 * I * H)
            ch.red("reduce_rmsnorm", part, inp["gamma"], w.eps, lambda i: R)
            run(w.name, b, t, ch, [part], lay, None)
            del inp, Wgu, Wd, act, part, ch
            torch.cuda.empty_cache()

    for w in (wl.LLAMA3_8B_ATTN_TP4, wl.LLAMA3_70B_LAYER_TP8):
        for b in w.batches:
            if not wanted(w, b):
                continue
            is_layer = isinstance(w, wl.LayerShard)
            inp = (wl.layer_inputs if is_layer else wl.attn_inputs)(w, b, seed=0, device=dev)
            t, H = w.t, w.hidden
            nq, nkv, hd = w.n_q_heads, w.n_kv_heads, w.head_dim
            sp = ttl.qkv_split(nq, nkv, hd, t)
            n_qkv = (nq + 2 * nkv) * hd
            w_r = ttl.split_width(sp, n_qkv, t)
            weights = [(inp["Wqkv"], False), (inp["Wo"], True)]
            if is_layer:
                weights += [(inp["Wgu"], False), (inp["Wd"], True)]
            lay = storage_for(t, weights)
            Wqkv, Wo = stored_weight(ttl, inp["Wqkv"], lay), stored_weight(ttl, inp["Wo"], lay)
            qkv = bf(b, w_r)
            gamma = inp["gamma_attn"] if is_layer else inp["gamma"]
            ch = Chain(t, b, H, t if b < 512 else 1)
            pa = ch.partials()
            X, A, R = inp["X"], inp["A"], inp["R"]
            ch.col("qkv", lambda i: X, Wqkv, sp, ttl.EPI_NONE, qkv, w_r, w_r, lay, 2.0 * H * n_qkv)
            ch.row("o_proj", lambda i: A, Wo, pa, nq * hd, H, False, lay, 2.0 * nq * hd * H)
            ch.red("reduce_rmsnorm_attn", pa, gamma, w.eps, lambda i: R)
            parts = [pa]
            keep = [Wqkv, Wo, qkv]
            if is_layer:
                I = w.intermediate
                Ir = I // t
                Wgu, Wd = stored_weight(ttl, inp["Wgu"], lay), stored_weight(ttl, inp["Wd"], lay)
                act = bf(b, Ir)
                pm = ch.partials()
                gsp = ttl.merged_gate_up_split(I, t)
                # the MLP half reads the attention half's outputs of the same step
                ch.col("gate_up_silu", lambda i: pa["y"][i % pa["n"]], Wgu, gsp, ttl.EPI_SILU_MUL, act,
                       2 * Ir, Ir, lay, 2.0 * H * 2 * I)
                ch.row("down", lambda i: act, Wd, pm, I, H, True, lay, 2.0 * I * H)
                ch.red("reduce_rmsnorm_mlp", pm, inp["gamma_mlp"], w.eps, lambda i: pa["rout"][i % pa["n"]])
                parts.append(pm)
                keep += [Wgu, Wd, act]
            run(w.name, b, t, ch, parts, lay, keep)
            del inp, ch, keep, parts, pa
            torch.cuda.empty_cache()


def read_power_clock():
    """(socket power W, mean GFX clock MHz) from amd-smi, or None."""
    import subprocess
    try:
        out = subprocess.run(["amd-smi", "metric", "-p", "-c", "--json"], capture_output=True, text=True,
                             timeout=30).stdout
        d = json.loads(out)
        g = d["gpu_data"][0] if isinstance(d, dict) else d[0]
        clocks = [v["clk"]["value"] for k, v in g["clock"].items() if k.startswith("gfx_")]
        return g["power"]["socket_power"]["value"], sum(clocks) / len(clocks)
    except Exception:  # pragma: no cover - tool missing or output not as expected
        return None


def steady_state(ttl, torch, w, layout):
    """Each b=4096 GEMM of the rank, ours and hipBLASLt's, at the power limit: run back to back for
    2 s, sample power and clock once in the middle, then time 30 launches."""
    lay = layout_code(ttl, layout)
    b, H, I, t = 4096, w.hidden, w.intermediate, w.t
    Ir = I // t
    X = torch.randn(b, H, device="cuda").to(torch.bfloat16)
    Wgu = (torch.randn(H, 2 * I, device="cuda") * 0.02).to(torch.bfloat16)
    Wd = (torch.randn(I, H, device="cuda") * 0.02).to(torch.bfloat16)
    act = torch.randn(b, Ir, device="cuda").to(torch.bfloat16)
    P = torch.empty(b, H, device="cuda", dtype=torch.bfloat16)
    sp = ttl.merged_gate_up_split(I, t)
    # rank 0's slices as separate dense tensors for torch.matmul
    Wg_r = torch.cat([Wgu[:, :Ir], Wgu[:, I:I + Ir]], dim=1).contiguous()  # [H, 2*Ir]
    Wd_r = Wd[:Ir].contiguous()                                            # [Ir, H]
    if lay == ttl.W_NK:
        Wgu, Wd = Wgu.t().contiguous(), Wd.t().contiguous()
        Wg_r, Wd_r = Wg_r.t().contiguous(), Wd_r.t().contiguous()
        mm_g = lambda: torch.matmul(X, Wg_r.t())
        mm_d = lambda: torch.matmul(act, Wd_r.t())
    else:  # hipBLASLt has no blocked storage: its products read W[k][n]
        if lay == ttl.W_BLOCKED:
            Wgu, Wd = ttl.pack_weight_blocked(Wgu), ttl.pack_weight_blocked(Wd)
        mm_g = lambda: torch.matmul(X, Wg_r)
        mm_d = lambda: torch.matmul(act, Wd_r)
    cases = (("ours_gate_up_silu", 2.0 * b * H * 2 * Ir,
              lambda: ttl.shard_linear_col(X, Wgu, t, 0, sp, ttl.EPI_SILU_MUL, Y=act, w_layout=lay)),
             ("ours_down", 2.0 * b * Ir * H, lambda: ttl.shard_linear_row(act, Wd, t, 0, P=P, w_layout=lay)),
             ("hipblaslt_gate_up_plain", 2.0 * b * H * 2 * Ir, mm_g),
             ("hipblaslt_down", 2.0 * b * Ir * H, mm_d))
    for name, flops, fn in cases:
        t0 = time.perf_counter()
        pc = None
        while time.perf_counter() - t0 < 2.0:
            for _ in range(10):
                fn()
            torch.cuda.synchronize()
            if pc is None and time.perf_counter() - t0 > 1.0:
                pc = read_power_clock() or (None, None)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(30):
            fn()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / 30 * 1e3
        print(json.dumps({"gemm": name, "weight_storage": layout, "us": us, "tflops": flops / (us * 1e6),
                          "socket_power_w": pc[0] if pc else None,
                          "gfx_clock_mhz_mean": pc[1] if pc else None}), flush=True)


def sample_power_clock(torch, step, seconds=6.0):
    """Socket power and GFX clock reported by amd-smi once while `step` runs back to back (the GPU
    settles at its power limit within a fraction of a second).  The repetition lasts longer than a
    5-s utilisation sampler's period, so an outside observer sees the GPU busy during the bench.
    None if amd-smi is unavailable."""
    t0 = time.perf_counter()
    pc, i = None, 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(20):
            step(i)
            i += 1
        torch.cuda.synchronize()
        if pc is None and time.perf_counter() - t0 > seconds / 2:
            pc = read_power_clock() or (None, None)
    if not pc or pc[0] is None:
        return None
    return {"socket_power_w": pc[0], "gfx_clock_mhz_mean": pc[1],
            "sampled": "amd-smi metric -p -c --json, once, while the step repeated for %.1f s" % seconds}


def traffic_sources_digest():
    h = hashlib.sha256()
    for rel in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def read_counter_csv(path, counter):
    """{kernel name: [value per dispatch]} of one rocprofv3 --pmc counter_collection.csv."""
    import csv
    out = {}
    with open(path, newline="") as f:
        for row in csv.DictReader(f):
            if row.get("Counter_Name") == counter:
                out.setdefault((row["Kernel_Name"], int(row["Grid_Size"])), []).append(float(row["Counter_Value"]))
    return out


def classify_dispatch(name):
    """Which entry point of the bench step a dispatch belongs to (None for the set-up kernels)."""
    if ("gemm_bigwave_kernel<1," in name or "gemm_bigwave16_kernel<1," in name or "gemm_skinny_kernel<1," in name
            or "splitk_finalize_kernel<1>" in name):
        return "shard_linear_col_silu_mul"
    if ("gemm_bigwave_kernel<0," in name or "gemm_bigwave16_kernel<0," in name or "gemm_skinny_kernel<0," in name
            or "splitk_finalize_kernel<0>" in name):
        return "shard_linear_row"
    if "reduce_rmsnorm_kernel" in name:
        return "reduce_partials_rmsnorm"
    return None


def _short_kernel_name(name):
    """The library's kernel name without namespaces and arguments (template arguments kept)."""
    m = re.search(r"ttl::\(anonymous namespace\)::(\w+)(<[^>]*>)?", name)
    return (m.group(1) + (m.group(2) or "")) if m else None


def trace_summary(directory):
    """Markdown rows from rocprofv3 kernel traces of single-kernel config-table runs (--op): for each
    run, the library's dispatches grouped by kernel and grid, their counts and average durations; one
    call dispatches each group once, so the per-call kernel time is the sum of the averages.  The
    run's JSON line (ct.json) gives the same call's time in a replayed HIP graph (kernels plus the
    gaps between them, no host launch cost) and eagerly launched (HIP events around each call)."""
    import csv
    import glob
    import statistics
    csv.field_size_limit(1 << 30)
    factor = None
    if os.path.isdir(os.path.join(directory, "copy_FETCH_SIZE")):
        factor = copy_factors(directory)
        print(f"HBM counters scaled by {factor['FETCH_SIZE']:.4f} (FETCH_SIZE) and {factor['WRITE_SIZE']:.4f} "
              f"(WRITE_SIZE) from a plain device copy; sources sha256 {traffic_sources_digest()}")
        print()
    print("| workload | tokens | kernel call | dispatches per call: kernel, grid, average us | "
          "sum of kernels us | graph us | eager us | read MB | written MB | algorithmic MB |")
    print("|---|---|---|---|---|---|---|---|---|---|")
    for run in sorted(d for d in glob.glob(os.path.join(directory, "*")) if os.path.isdir(d)):
        traces = glob.glob(os.path.join(run, "**", "*kernel_trace.csv"), recursive=True)
        if not traces:
            continue
        groups = {}
        for path in traces:
            for r in csv.DictReader(open(path)):
                name = _short_kernel_name(r["Kernel_Name"])
                if name is None:
                    continue
                grid = int(r["Grid_Size_X"]) // max(1, int(r["Workgroup_Size_X"]))
                dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
                groups.setdefault((name, grid), []).append(dur)
        if not groups:
            continue
        calls = max(len(v) for v in groups.values())
        order = sorted(groups, key=lambda k: -statistics.mean(groups[k]))
        parts = [f"`{k[0]}` {k[1]}: {statistics.mean(groups[k]):.1f}" +
                 ("" if len(groups[k]) == calls else f" ({len(groups[k])} of {calls} calls)") for k in order]
        total = sum(statistics.mean(v) * len(v) / calls for v in groups.values())
        meta = {}
        ct = os.path.join(run, "ct.json")
        if os.path.exists(ct):
            for line in open(ct):
                if line.startswith("{"):
                    meta = json.loads(line)
        kern = next(iter(meta.get("kernels", {}).items()), (os.path.basename(run), {}))
        traffic = ["", ""]
        if factor is not None and os.path.isdir(os.path.join(run, "pmc_FETCH_SIZE")):
            for i, counter in enumerate(("FETCH_SIZE", "WRITE_SIZE")):
                d = {k: v for k, v in _counter_run(run, f"pmc_{counter}", counter).items()
                     if _short_kernel_name(k[0]) is not None}
                n = max(len(v) for v in d.values())
                per_call = sum(sum(v) / n for v in d.values()) * 1024.0 * factor[counter]
                traffic[i] = f"{per_call / 1e6:.1f}"
        alg = kern[1].get("gbs", float("nan")) * kern[1].get("us", float("nan")) * 1e3
        print(f"| {meta.get('workload', os.path.basename(run))} | {meta.get('tokens', '')} | {kern[0]} | "
              f"{'; '.join(parts)} | {total:.1f} | {meta.get('step_us_graph', float('nan')):.1f} | "
              f"{kern[1].get('us', float('nan')):.1f} | {traffic[0]} | {traffic[1]} | {alg / 1e6:.1f} |")


def _counter_run(directory, sub, counter):
    """{(kernel name, grid): [KiB per dispatch]} of the counter run under directory/sub."""
    import glob
    files = glob.glob(os.path.join(directory, sub, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no counter_collection.csv under {os.path.join(directory, sub)}")
    return read_counter_csv(files[0], counter)


def copy_factors(directory):
    """Bytes per counted KiB for FETCH_SIZE and WRITE_SIZE: the plain device copy's known size (its
    JSON line in directory/copy_<COUNTER>*.log) over what the counter read for it (copy_<COUNTER>/)."""
    import glob
    factor = {}
    for counter in ("FETCH_SIZE", "WRITE_SIZE"):
        d = _counter_run(directory, f"copy_{counter}", counter)
        copies = [(k, v) for k, v in d.items() if "copyBuffer" in k[0] or "copy" in k[0].lower()]
        (name, _), vals = max(copies, key=lambda kv: kv[0][1])
        nbytes = None
        for log in glob.glob(os.path.join(directory, f"copy_{counter}*.log")):
            for line in open(log):
                if line.startswith("{") and "copy_bytes_per_launch" in line:
                    nbytes = json.loads(line)["copy_bytes_per_launch"]
        if nbytes is None:
            raise RuntimeError(f"copy size not found in {directory}/copy_{counter}*.log")
        kib = sum(vals) / len(vals)
        factor[counter] = nbytes / (kib * 1024.0)
    return factor


def traffic_record(directory, commit, b=4096, t=8, H=8192, I=28672):
    """HBM bytes per call of each entry point from FETCH_SIZE and WRITE_SIZE counter runs.  Each
    counter is scaled by what it reads for a plain device copy of known size; a call's traffic is the
    sum, over the distinct dispatches (kernel, grid) one call issues, of their mean per dispatch."""
    def one(sub, counter):
        return _counter_run(directory, sub, counter)

    factor = copy_factors(directory)
    alg = {"shard_linear_col_silu_mul": col_silu_bytes(b, H, I // t),
           "shard_linear_row": row_bytes(b, I // t, H),
           "reduce_partials_rmsnorm": reduce_bytes(t, b, H)}
    digest = traffic_sources_digest()
    rows, lines = [], []
    for lay in ("kn", "nk"):
        if not os.path.isdir(os.path.join(directory, f"pmc_FETCH_SIZE_{lay}")):
            continue
        per_call = {}
        for counter in ("FETCH_SIZE", "WRITE_SIZE"):
            for (name, grid), vals in one(f"pmc_{counter}_{lay}", counter).items():
                ep = classify_dispatch(name)
                if ep is None:
                    continue
                mean_bytes = sum(vals) / len(vals) * 1024.0 * factor[counter]
                per_call.setdefault(ep, {"FETCH_SIZE": 0.0, "WRITE_SIZE": 0.0, "dispatches": []})
                per_call[ep][counter] += mean_bytes
                if counter == "FETCH_SIZE":
                    m = re.search(r"(\w+_kernel<[^>]*>)", name)
                    per_call[ep]["dispatches"].append(f"{m.group(1) if m else name[:40]} grid {grid}")
        for ep, d in per_call.items():
            total = d["FETCH_SIZE"] + d["WRITE_SIZE"]
            rows.append(f"| {ep} | {lay} | {d['FETCH_SIZE'] / 1e6:.1f} | {d['WRITE_SIZE'] / 1e6:.1f} | "
                        f"{total / 1e6:.1f} | {alg[ep] / 1e6:.1f} | {total / alg[ep]:.2f} | "
                        f"{'; '.join(d['dispatches'])} |")
            if ep == "shard_linear_col_silu_mul":
                lines.append(f"traffic kernel={ep} workload=llama3_70b_mlp_tp8_rank0_b{b}_{lay} "
                             f"bytes_per_launch={int(round(total))} source_sha256={digest}")
    print(f"counters scaled by a {factor['FETCH_SIZE']:.4f} (FETCH_SIZE) and {factor['WRITE_SIZE']:.4f} "
          f"(WRITE_SIZE) factor from the plain device copy; sources sha256 {digest}"
          + (f"; taken at commit {commit}" if commit else ""))
    print("| entry point (per call) | weight storage | read MB | written MB | traffic MB | algorithmic MB "
          "| ratio | dispatches |")
    print("|---|---|---|---|---|---|---|---|")
    for r in rows:
        print(r)
    print()
    for line in lines:
        print(line)
    return lines


def recorded_traffic(kernel, workload):
    """HBM bytes per launch recorded from the FETCH_SIZE / WRITE_SIZE counters in profiles/, or None
    when no record exists or the kernel sources changed since the counters were taken."""
    digest = traffic_sources_digest()
    pat = re.compile(r"^traffic\s+kernel=(\S+)\s+workload=(\S+)\s+bytes_per_launch=(\d+)\s+"
                     r"source_sha256=([0-9a-f]{64})\s*$")
    pdir = os.path.join(ROOT, "profiles")
    if not os.path.isdir(pdir):
        return None
    for name in sorted(os.listdir(pdir)):
        if not name.endswith((".md", ".txt")):
            continue
        with open(os.path.join(pdir, name)) as f:
            for line in f:
                m = pat.match(line.strip())
                if m and m.group(1) == kernel and m.group(2) == workload and m.group(4) == digest:
                    return float(m.group(3))
    return None


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(torch, w, tensors, rows, seconds):
    """The oracle as it stands, on rank 0's work for `rows` token rows (rows are independent), timed
    on the host's cores twice: with every core this process may run on (os.sched_getaffinity) as
    numpy's BLAS threads, and with one.  Each run times the two GEMM steps (gate_up + SiLU·up, then
    the down partial) and the reduction (8 partials + residual + RMSNorm) separately, each repeated
    until its share of `seconds` has passed."""
    import numpy as np
    import oracle
    from tensor_transformer_linear_amd import workloads as wl
    from threadpoolctl import threadpool_info, threadpool_limits
    X, Wgu, Wd, R, gamma = tensors
    t, H, I = w.t, w.hidden, w.intermediate
    Ir = I // t
    # inputs to host memory and the oracle's decoding (not timed: input preparation)
    Xs = oracle.bf16_bits_to_f64(wl.bf16_bits(X[:rows].cpu()))
    Rs = oracle.bf16_bits_to_f64(wl.bf16_bits(R[:rows].cpu()))
    gs = oracle.bf16_bits_to_f64(wl.bf16_bits(gamma.cpu()))
    Wgu64 = oracle.bf16_bits_to_f64(wl.bf16_bits(Wgu.cpu()))
    Wd64 = oracle.bf16_bits_to_f64(wl.bf16_bits(Wd.cpu()))
    split = oracle.merged_gate_up_split(I, t)
    rng = np.random.default_rng(0)
    others = oracle.round_bf16(rng.standard_normal((t - 1, rows, H)))  # the other ranks' partials

    def gemms():
        act = oracle.round_bf16(oracle.silu_mul(oracle.col_shard(Xs, Wgu64, split, t, 0)))
        return oracle.round_bf16(oracle.row_shard(act, Wd64, t, 0, x_is_parallel=True))

    p0 = gemms()
    P = np.concatenate([p0[None], others])

    def timed(fn, budget):
        n, t0 = 0, time.perf_counter()
        while True:
            fn()
            n += 1
            dt = time.perf_counter() - t0
            if dt >= budget:
                return n, dt

    gemm_flops_pass = gemm_flops(rows, H, 2 * Ir) + gemm_flops(rows, Ir, H)
    red_bytes_pass = reduce_bytes(t, rows, H)
    affinity = len(os.sched_getaffinity(0))
    runs = {}
    for label, limit in (("all_cores", affinity), ("one_core", 1)):
        with threadpool_limits(limits=limit):
            threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
            ng, tg = timed(gemms, 0.4 * seconds)
            nr, tr = timed(lambda: oracle.reduce_partials_rmsnorm(P, Rs, gs, w.eps), 0.1 * seconds)
        runs[label] = {"threads": int(threads), "gemm_tflops": ng * gemm_flops_pass / tg / 1e12,
                       "gemm_passes": ng, "gemm_seconds": tg,
                       "reduce_gbs": nr * red_bytes_pass / tr / 1e9, "reduce_passes": nr, "reduce_seconds": tr,
                       "step_tflops": gemm_flops_pass / (tg / ng + tr / nr) / 1e12}
    allc = runs["all_cores"]
    return {"value": allc["step_tflops"], "unit": "TFLOP/s", "cores": allc["threads"], "kind": "oracle",
            "cpu_model": cpu_model(), "affinity_cores": affinity,
            "gemm_tflops": allc["gemm_tflops"], "reduce_gbs": allc["reduce_gbs"],
            "one_core": runs["one_core"], "all_cores": allc,
            "seconds": sum(r["gemm_seconds"] + r["reduce_seconds"] for r in runs.values()),
            "sample": f"rank 0 of t={t} over {rows} of the {tensors[0].shape[0]} token rows: gate_up+SiLU*up and "
                      f"the down partial (GEMM TFLOP/s), the reduction of {t} partials + residual + RMSNorm "
                      f"(GB/s of its algorithmic bytes); value = the step's GEMM flops over the step's time "
                      f"(both parts) with all cores; float64 numpy oracle; rows are independent, so the rates "
                      f"apply to the full batch"}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU's share of the tensor-parallel work (ranks are simulated in one "
              "HBM); runs on more than one GPU are not part of this benchmark.", file=sys.stderr)
        return 2
    if args.traffic_record:
        traffic_record(args.traffic_record, args.commit)
        return 0
    if args.trace_summary:
        trace_summary(args.trace_summary)
        return 0
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    if args.copy_calibration_mib:
        n = args.copy_calibration_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").random_(0, 255)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_per_launch": n, "launches": 5}), flush=True)
        return 0
    from tensor_transformer_linear_amd import ttl
    from tensor_transformer_linear_amd import workloads as wl
    w = wl.LLAMA3_70B_MLP_TP8
    if args.steady_state:
        steady_state(ttl, torch, w, args.layout)
        return 0
    if args.config_table:
        config_table(ttl, torch, args.layout, only=args.workload, only_op=args.op, graph=not args.no_graph)
        return 0
    b = args.batch
    workload = f"llama3_70b_mlp_tp8_rank0_b{b}_{args.layout}"
    res = run_mlp(ttl, torch, w, b, args.steps, args.warmup, seed=0, layout=args.layout, settle_ms=args.settle_ms,
                  rotate_ranks=(b < 512))
    ms = res["ms_per_step"]
    value = res["flops"] / (ms * 1e9)
    kcol = res["kernels"]["shard_linear_col_silu_mul"]
    traffic = recorded_traffic("shard_linear_col_silu_mul", workload)
    if b >= 512:
        roof = {"kernel": "shard_linear_col_silu_mul", "bound": "mfma", "achieved": kcol["tflops"],
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": kcol["tflops"] / PEAK_BF16_TFLOPS,
                "traffic": traffic}
    else:
        roof = {"kernel": "shard_linear_col_silu_mul", "bound": "hbm", "achieved": kcol["gbs"],
                "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": kcol["gbs"] / PEAK_HBM_GBS,
                "traffic": traffic}
    roof["algorithmic_gflop_per_launch"] = kcol["gflop"]
    power = None if args.no_power else sample_power_clock(torch, res["step"])
    roof["algorithmic_mbytes_per_launch"] = kcol["mbytes"]
    out = {
        "metric": "TFLOP/s and % bf16 MFMA peak, 1-rank shard of Llama-3-70B MLP at TP=8 shape",
        "value": value,
        "unit": "TFLOP/s",
        "pct_bf16_peak": 100.0 * value / PEAK_BF16_TFLOPS,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_ms": args.settle_ms,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": workload, "hidden": w.hidden,
                   "intermediate": w.intermediate, "t": w.t, "tokens": b, "weight_storage": args.layout,
                   "step": "gate_up+SiLU*up (col) -> down (row partial) -> reduce 8 partials + residual + RMSNorm"},
        "roofline": roof,
        "power_clock": power,
        "kernels": res["kernels"],
    }
    if not args.no_decode and b != 64:
        dec = run_mlp(ttl, torch, w, 64, args.steps, args.warmup, seed=1, layout=args.layout, settle_ms=args.settle_ms,
                      rotate_ranks=True, graph=True)
        out["decode64"] = {"ms_per_step": dec["ms_per_step"], "ranks": "cycled 0..7 step by step",
                           "tflops": dec["flops"] / (dec["ms_per_step"] * 1e9),
                           "ms_per_step_graph": dec["ms_per_step_graph"],
                           "tflops_graph": dec["flops"] / (dec["ms_per_step_graph"] * 1e9),
                           "kernels": dec["kernels"]}
        del dec
    out["yardstick"] = None if args.no_yardstick else yardstick(torch, w, args.layout)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(torch, w, res["tensors"], args.cpu_rows, args.cpu_seconds)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
