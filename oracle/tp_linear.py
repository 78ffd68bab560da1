"""Plain CPU oracle of the tensor-parallel sharded linear path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg
of ``bench.py`` may import or call this module.  The HIP library never routes through it, and it
shares no code, header, table or helper with ``tensor_transformer_linear_amd``: it receives raw bf16
bit patterns (numpy ``uint16``) and works on its own decoding of them.

Arithmetic is float64 throughout.  Inputs are bf16, so every product of two inputs is exact in
float64 and sums of them carry only float64 rounding, far below the bf16-in / fp32-accumulate error
of the device path.  Matrix products use numpy's float64 ``@`` as one step (a library primitive);
nothing is blocked, fused or reordered beyond the definitions cited below.

Sources (page title, then section):
  [VLLM-TP]  "vLLM 源码完全拆解（十一）：模型并行与 Worker 层" (pinghaoyang.com.cn), sections
             "一个矩阵乘法如何被切开" (Y = XW with X[b,k], W[k,n]; column split W_i[k,n/t], Y_i = XW_i;
             row split W_i[k/t,n], X_i[b,k/t], Y = sum_i X_i W_i), "ColumnParallelLinear"
             (divide() asserts exact division; rank r takes columns [r*n/t, (r+1)*n/t)),
             "MergedColumnParallelLinear / QkvParallelLinear" (output_sizes=[I, I]; q heads / t per
             rank; kv heads split or replicated when t >= n_kv), "RowParallelLinear"
             (input_is_parallel; split along the last dim; partial sums reduced).
  [VLLM-CR5] "vLLM Code Reading (Section 5): GPUWorker.execute_model 与 PP/TP 通信"
             (jeremyguo.space), sections 12 (Y_i = X_i A_i, Y = sum_i Y_i) and 14 (activation runs on
             the local shard).
  [MLXCEL]   "Tensor Parallelism" (mlxcel.ai manual), sections "Vocab Parallel" (each rank owns a
             contiguous vocabulary slice; logits all-gathered) and "Communication Patterns"
             (reduce-scatter leaves each rank one reduced chunk).
  [UNDERCUR] "Tensor & pipeline parallelism" (wrynx.github.io, Undercurrent docs), sections
             "residual_stream" (post_attention_layernorm(hidden, residual) returns the updated pair;
             the residual stream is hidden + residual) and "final_norm" (RMSNorm(hidden, eps), not
             sharded across TP ranks).

Readings where the pages are silent (each is also listed in the design notes):
  * SiLU is not defined on the pages: silu(x) = x / (1 + exp(-x)) (the standard definition).
  * RMSNorm's formula is not printed: y = h / sqrt(mean_j(h_j^2) + eps) * gamma over the full
    hidden dimension, eps inside the root.
  * The merged gate_up weight is sliced per output_size: rank r owns gate columns
    [r*I/t, (r+1)*I/t) and the matching up columns [I + r*I/t, I + (r+1)*I/t).
  * KV heads when t >= n_kv: rank r takes kv head floor(r * n_kv / t) (vLLM's replica rule).
  * Partials are summed in ascending rank order; the residual is added after the sum; the norm reads
    the unrounded sum h, and the updated residual stream is h.
  * No bias: Llama's projections carry none.

Parity status: every function below is pinned by CPU tests (brute-force dot products on tiny
inputs, the column-concatenation and row-sum invariants, closed forms of SiLU and RMSNorm, the head
arithmetic printed on the pages).  Only the tolerance constant 2e-2 * rms(ref) is not from the pages.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "bf16_bits_to_f64", "f64_to_bf16_bits", "round_bf16", "divide", "qkv_local_heads",
    "column_split", "merged_gate_up_split", "qkv_split", "plain_split", "rank_columns",
    "col_shard", "silu", "silu_mul", "row_shard", "reduce_partials_rmsnorm", "mlp_rank_chain",
    "col_gathered", "reduce_scatter_partials_rmsnorm",
]


# ----------------------------------------------------------------------------------------------
# bf16 encoding (the storage type of every tensor that crosses the library boundary)
# ----------------------------------------------------------------------------------------------

def bf16_bits_to_f64(bits) -> np.ndarray:
    """Decode raw bf16 bit patterns: a bf16 is the high half of an IEEE binary32."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


_BF16_MAX = float.fromhex("0x1.fep127")  # largest finite bf16


def round_bf16(x) -> np.ndarray:
    """Round float64 values to the nearest bf16 value (ties to even), returned as float64.

    bf16 keeps 8 significant bits and binary32's exponent range, so a normal value with exponent e
    (x = m * 2**e, 0.5 <= |m| < 1) is rounded to a multiple of 2**(e-8); below 2**-126 the spacing is
    the subnormal quantum 2**-133.  Values past the rounding threshold of the largest finite bf16
    become infinities.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    finite = np.isfinite(x)
    out[~finite] = x[~finite]
    xf = x[finite]
    m, e = np.frexp(xf)
    e = np.maximum(e, -125)  # below the normal range the quantum stays 2**-133
    quantum = np.ldexp(1.0, e - 8)
    r = np.rint(xf / quantum) * quantum  # np.rint rounds halfway cases to even
    # Overflow: anything that rounds beyond the largest finite bf16 is infinite.
    big = np.abs(r) > _BF16_MAX
    r[big] = np.copysign(np.inf, xf[big])
    out[finite] = r
    return out


def f64_to_bf16_bits(x) -> np.ndarray:
    """Encode float64 values as bf16 bit patterns (round to nearest, ties to even)."""
    r = round_bf16(x)
    return (r.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


# ----------------------------------------------------------------------------------------------
# Shard arithmetic  [VLLM-TP] "ColumnParallelLinear", "MergedColumnParallelLinear / QkvParallelLinear"
# ----------------------------------------------------------------------------------------------

def divide(numerator: int, denominator: int) -> int:
    """Exact division, refusing anything that does not divide (vLLM's divide() asserts)."""
    if denominator <= 0 or numerator % denominator != 0:
        raise ValueError(f"{numerator} is not divisible by {denominator}")
    return numerator // denominator


def qkv_local_heads(total_q_heads: int, total_kv_heads: int, t: int):
    """Per-rank head counts of the QKV projection: (q heads, kv heads, kv replicas).

    q heads are split evenly.  When t >= total kv heads each rank holds one kv head and every kv head
    is replicated t / n_kv times; otherwise kv heads are split evenly with no replica.
    """
    q = divide(total_q_heads, t)
    if t >= total_kv_heads:
        return q, 1, divide(t, total_kv_heads)
    return q, divide(total_kv_heads, t), 1


def column_split(seg_n, seg_parts):
    """A column split: segments packed side by side along n, segment i cut into seg_parts[i] slices."""
    seg_n = tuple(int(v) for v in seg_n)
    seg_parts = tuple(int(v) for v in seg_parts)
    if len(seg_n) != len(seg_parts) or not seg_n:
        raise ValueError("segments and part counts must pair up")
    return seg_n, seg_parts


def plain_split(n: int, t: int):
    return column_split((n,), (t,))


def merged_gate_up_split(intermediate: int, t: int):
    """gate_up built with output_sizes=[I, I]: each output size is its own segment."""
    return column_split((intermediate, intermediate), (t, t))


def qkv_split(n_q_heads: int, n_kv_heads: int, head_dim: int, t: int):
    """q | k | v segments; kv segments have min(t, n_kv) distinct slices."""
    kv_parts = n_kv_heads if t >= n_kv_heads else t
    return column_split((n_q_heads * head_dim, n_kv_heads * head_dim, n_kv_heads * head_dim),
                        (t, kv_parts, kv_parts))


def rank_columns(split, t: int, rank: int) -> np.ndarray:
    """Columns of the full W owned by `rank`, in output order (segment by segment).

    Segment i of width n_i with p_i slices: rank r takes slice q = floor(r * p_i / t), i.e. columns
    [off_i + q * n_i/p_i, off_i + (q+1) * n_i/p_i).  With p_i = t this is the plain
    start_idx = tp_rank * shard_size rule of weight_loader.
    """
    seg_n, seg_parts = split
    if not (0 <= rank < t):
        raise ValueError("rank out of range")
    cols = []
    off = 0
    for n_i, p_i in zip(seg_n, seg_parts):
        w = divide(n_i, p_i)
        if p_i < t:
            divide(t, p_i)  # a replicated slice must be shared by a whole number of ranks
        elif p_i != t:
            raise ValueError("a segment cannot have more slices than ranks")
        q = (rank * p_i) // t
        cols.append(np.arange(off + q * w, off + (q + 1) * w))
        off += n_i
    return np.concatenate(cols)


# ----------------------------------------------------------------------------------------------
# The four operations
# ----------------------------------------------------------------------------------------------

def col_shard(X, W, split, t: int, rank: int) -> np.ndarray:
    """Column-parallel output of one rank: Y_r = X @ W[:, C_r]  ([VLLM-TP] column split).

    X: [b, k] float64, W: [k, n] float64 (the full, unsharded weight).  Returns [b, |C_r|].
    """
    X = np.asarray(X, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    if X.shape[1] != W.shape[0]:
        raise ValueError("inner dimensions differ")
    if sum(split[0]) != W.shape[1]:
        raise ValueError("segments do not cover W's columns")
    cols = rank_columns(split, t, rank)
    return X @ W[:, cols]


def silu(x) -> np.ndarray:
    """silu(x) = x * sigmoid(x) = x / (1 + exp(-x))."""
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore"):
        return x / (1.0 + np.exp(-x))


def silu_mul(Y) -> np.ndarray:
    """Gated activation on the local shard ([VLLM-CR5] section 14): left half gate, right half up."""
    Y = np.asarray(Y, dtype=np.float64)
    h = Y.shape[1] // 2
    if 2 * h != Y.shape[1]:
        raise ValueError("gate and up halves must have equal width")
    return silu(Y[:, :h]) * Y[:, h:]


def row_shard(X, W, t: int, rank: int, x_is_parallel: bool) -> np.ndarray:
    """Row-parallel partial of one rank: P_r = X_r @ W[r*k/t:(r+1)*k/t, :]  ([VLLM-TP] row split).

    W is the full [k, n] weight.  X is either already the rank's slice [b, k/t] (input_is_parallel)
    or the full [b, k], whose columns [r*k/t, (r+1)*k/t) are the slice (split along the last dim).
    """
    X = np.asarray(X, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    k = W.shape[0]
    w = divide(k, t)
    if not (0 <= rank < t):
        raise ValueError("rank out of range")
    rows = slice(rank * w, (rank + 1) * w)
    Xr = X if x_is_parallel else X[:, rows]
    if Xr.shape[1] != w:
        raise ValueError("input width does not match k/t")
    return Xr @ W[rows, :]


def reduce_partials_rmsnorm(P, residual, gamma, eps: float):
    """Sum of t rank partials, residual add, RMSNorm over the full hidden dimension.

    P: [t, b, n]; residual: [b, n] or None (then h = sum); gamma: [n].
    s = P_0 + P_1 + ... + P_{t-1} (ascending rank); h = s + residual;
    y = h / sqrt(mean_j h_j^2 + eps) * gamma.  Returns (h, y): h is the updated residual stream.
    ([UNDERCUR] "residual_stream", "final_norm"; [VLLM-TP] "RowParallelLinear" all-reduce.)
    """
    P = np.asarray(P, dtype=np.float64)
    s = np.zeros(P.shape[1:], dtype=np.float64)
    for r in range(P.shape[0]):
        s = s + P[r]
    h = s if residual is None else s + np.asarray(residual, dtype=np.float64)
    ms = np.mean(h * h, axis=-1, keepdims=True)
    y = h / np.sqrt(ms + eps) * np.asarray(gamma, dtype=np.float64)
    return h, y


def col_gathered(X, W, split, t: int, epi_silu_mul: bool = False) -> np.ndarray:
    """ColumnParallelLinear with gather_output=True: the all-gather of the t rank outputs, i.e. their
    concatenation along the last dimension in rank order.  ([VLLM-TP] "ColumnParallelLinear"
    forward, gather_output branch, and "all-gather"; [MLXCEL] "Vocab Parallel": logits of the
    vocabulary slices all-gathered.)"""
    outs = []
    for r in range(t):
        y = col_shard(X, W, split, t, r)
        outs.append(silu_mul(y) if epi_silu_mul else y)
    return np.concatenate(outs, axis=-1)


def reduce_scatter_partials_rmsnorm(P, residual_shard, gamma, eps: float, t: int, rank: int):
    """Sequence-parallel reduction: rank `rank` reduces and normalises only its chunk of b/t token
    rows, [rank*b/t, (rank+1)*b/t), with its shard of the residual stream.  ([MLXCEL]
    "Communication Patterns": after reduce-scatter each rank holds one reduced chunk;
    [VLLM-CR5] section 4, PP + SP: the residual stays scattered over the ranks.)  Returns (h, y) of
    the chunk."""
    P = np.asarray(P, dtype=np.float64)
    b = P.shape[1]
    rows = divide(b, t)
    chunk = P[:, rank * rows:(rank + 1) * rows]
    return reduce_partials_rmsnorm(chunk, residual_shard, gamma, eps)


def mlp_rank_chain(X, Wgu, Wd, t: int, intermediate: int, store_bf16: bool = True):
    """gate_up (column, merged) -> silu*up -> down (row) for every rank.

    Returns (acts, P, acts_stored, P_stored).  acts[r] and P[r] are each step's exact value given
    the inputs that step reads; with store_bf16 those inputs are the bf16 values the library
    boundary stores between steps (the rank's act tensor, its partial), i.e. acts_stored[r] =
    round_bf16(acts[r]) feeds the down projection and P_stored = round_bf16(P) feeds the reduction.
    Without store_bf16 the stored values equal the exact ones.
    """
    split = merged_gate_up_split(intermediate, t)
    acts, parts, acts_s, parts_s = [], [], [], []
    for r in range(t):
        act = silu_mul(col_shard(X, Wgu, split, t, r))
        act_s = round_bf16(act) if store_bf16 else act
        p = row_shard(act_s, Wd, t, r, x_is_parallel=True)
        p_s = round_bf16(p) if store_bf16 else p
        acts.append(act)
        acts_s.append(act_s)
        parts.append(p)
        parts_s.append(p_s)
    return acts, np.stack(parts), acts_s, np.stack(parts_s)
