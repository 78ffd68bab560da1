"""ctypes binding of libttl (argument marshalling only: every step runs in the HIP library).

The names mirror the C ABI in include/ttl.h.  Tensors are torch bf16 tensors on the GPU; torch is
used for device memory and streams only.  Importing this module loads libttl.so and raises
ImportError if it has not been built, so the compute path can never silently fall back to anything
else.
"""

from __future__ import annotations

import contextlib
import ctypes
import os
from typing import Optional, Sequence, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libttl.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python -m tensor_transformer_linear_amd.build` "
                      "(or __graft_entry__.build()) before using the HIP path")

_lib = ctypes.CDLL(LIB_PATH)

OK = 0
ERR_NULL, ERR_SHAPE, ERR_NOT_DIVISIBLE, ERR_RANK, ERR_ALIGN, ERR_UNSUPPORTED, ERR_HIP = range(1, 8)
EPI_NONE = 0
EPI_SILU_MUL = 1
W_KN = 0  # weight stored [k][n] (row stride n)
W_NK = 1  # weight stored transposed, [n][k] (row stride k), as PyTorch-style Linear weights are
W_BLOCKED = 2  # [k][n] in 64 x 128 blocks, 128-column strips contiguous (see pack_weight_blocked)
MAX_SEGMENTS = 3
MAX_PEERS = 16
EXPORTED = ("shard_linear_col", "shard_linear_col_stored", "shard_linear_col_noalloc", "shard_linear_col_gathered",
            "shard_linear_row", "shard_linear_row_stored",
            "reduce_partials_rmsnorm", "reduce_scatter_partials_rmsnorm", "reduce_partials_rmsnorm_peers",
            "ttl_pack_weight_blocked", "ttl_last_error", "ttl_version", "ttl_set_gemm_override")
# GEMM kernel families ttl_set_gemm_override can force (tests and measurements only)
GEMM_KERNELS = {"auto": 0, "tiled": 1, "splitk": 2, "eightwave": 3, "tilesplit": 4, "narrow": 5,
                "narrowsplit": 6, "short": 7, "mixed": 8, "persist": 9, "tiled16": 10,
                "appended": 11, "streamnk": 12}


class ColSplit(ctypes.Structure):
    _fields_ = [("nseg", ctypes.c_int32),
                ("seg_n", ctypes.c_int64 * MAX_SEGMENTS),
                ("seg_parts", ctypes.c_int32 * MAX_SEGMENTS)]


_c_u16p = ctypes.c_void_p
_I32, _I64 = ctypes.c_int32, ctypes.c_int64
_lib.shard_linear_col.restype = _I32
_lib.shard_linear_col.argtypes = [_c_u16p, _I64, _I64, _c_u16p, _I64, _I32, _I32,
                                  ctypes.POINTER(ColSplit), _I32, _c_u16p, ctypes.c_void_p]
_lib.shard_linear_col_stored.restype = _I32
_lib.shard_linear_col_stored.argtypes = [_c_u16p, _I64, _I64, _c_u16p, _I64, _I32, _I32, _I32,
                                         ctypes.POINTER(ColSplit), _I32, _c_u16p, ctypes.c_void_p]
_lib.shard_linear_col_noalloc.restype = _I32
_lib.shard_linear_col_noalloc.argtypes = _lib.shard_linear_col_stored.argtypes
NOALLOC_SCRATCH_BYTES = 64 << 20
_lib.shard_linear_col_gathered.restype = _I32
_lib.shard_linear_col_gathered.argtypes = _lib.shard_linear_col_stored.argtypes
_lib.shard_linear_row.restype = _I32
_lib.shard_linear_row.argtypes = [_c_u16p, _I64, _I64, _I32, _c_u16p, _I64, _I32, _I32, _c_u16p,
                                  ctypes.c_void_p]
_lib.shard_linear_row_stored.restype = _I32
_lib.shard_linear_row_stored.argtypes = [_c_u16p, _I64, _I64, _I32, _c_u16p, _I64, _I32, _I32, _I32,
                                         _c_u16p, ctypes.c_void_p]
_lib.ttl_set_gemm_override.restype = _I32
_lib.ttl_set_gemm_override.argtypes = [_I32, _I32, _I32, _I32]
_lib.reduce_partials_rmsnorm.restype = ctypes.c_int32
_lib.reduce_partials_rmsnorm.argtypes = [_c_u16p, ctypes.c_int32, ctypes.c_int64, ctypes.c_int64,
                                         _c_u16p, _c_u16p, ctypes.c_float, _c_u16p, _c_u16p,
                                         ctypes.c_void_p]
_lib.reduce_scatter_partials_rmsnorm.restype = ctypes.c_int32
_lib.reduce_scatter_partials_rmsnorm.argtypes = [_c_u16p, ctypes.c_int32, ctypes.c_int64, ctypes.c_int64,
                                                 ctypes.c_int32, _c_u16p, _c_u16p, ctypes.c_float,
                                                 _c_u16p, _c_u16p, ctypes.c_void_p]
_lib.reduce_partials_rmsnorm_peers.restype = ctypes.c_int32
_lib.reduce_partials_rmsnorm_peers.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_int32, ctypes.c_int64,
                                               ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, _c_u16p, _c_u16p,
                                               ctypes.c_float, _c_u16p, _c_u16p, ctypes.c_void_p]
_lib.ttl_pack_weight_blocked.restype = ctypes.c_int32
_lib.ttl_pack_weight_blocked.argtypes = [_c_u16p, ctypes.c_int64, ctypes.c_int64, _c_u16p, ctypes.c_void_p]
_lib.ttl_last_error.restype = ctypes.c_char_p
_lib.ttl_last_error.argtypes = []
_lib.ttl_version.restype = ctypes.c_int32
_lib.ttl_version.argtypes = []


def lib() -> ctypes.CDLL:
    """The loaded library (raw C entry points, for callers that marshal pointers themselves)."""
    return _lib


class TTLError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


def last_error() -> str:
    return (_lib.ttl_last_error() or b"").decode()


def _check(status: int):
    if status != OK:
        raise TTLError(status, last_error())


def make_split(seg_n: Sequence[int], seg_parts: Sequence[int]) -> ColSplit:
    if not 1 <= len(seg_n) <= MAX_SEGMENTS or len(seg_n) != len(seg_parts):
        raise ValueError("1..3 segments with one part count each")
    s = ColSplit()
    s.nseg = len(seg_n)
    for i, (w, q) in enumerate(zip(seg_n, seg_parts)):
        s.seg_n[i] = int(w)
        s.seg_parts[i] = int(q)
    return s


def merged_gate_up_split(intermediate: int, t: int) -> ColSplit:
    """gate_up with output_sizes=[I, I]: gate and up are separate segments, each cut into t slices."""
    return make_split((intermediate, intermediate), (t, t))


def qkv_split(n_q_heads: int, n_kv_heads: int, head_dim: int, t: int) -> ColSplit:
    """q | k | v segments; k and v have min(t, n_kv) distinct slices (replicated when t > n_kv)."""
    kv_parts = n_kv_heads if t >= n_kv_heads else t
    return make_split((n_q_heads * head_dim, n_kv_heads * head_dim, n_kv_heads * head_dim),
                      (t, kv_parts, kv_parts))


def split_width(split: Optional[ColSplit], n: int, t: int) -> int:
    """Output columns of one rank under `split` (None: n / t)."""
    if split is None:
        return n // t
    return sum(split.seg_n[i] // split.seg_parts[i] for i in range(split.nseg))


def _dev_ptr(x: Optional[torch.Tensor], name: str) -> Optional[int]:
    if x is None:
        return None
    if not isinstance(x, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if x.dtype != torch.bfloat16:
        raise TypeError(f"{name} must be bfloat16, got {x.dtype}")
    if not x.is_cuda:
        raise ValueError(f"{name} must live on the GPU (the library has no host path)")
    if not x.is_contiguous():
        raise ValueError(f"{name} must be contiguous (row-major, dense)")
    return x.data_ptr()


def _stream_handle(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _weight_dims(W: torch.Tensor, w_layout: int):
    """(k, n) of the logical W[k, n] given its storage."""
    if w_layout == W_NK:
        n, k = W.shape
    else:
        k, n = W.shape
    return k, n


def _expect_shape(x: Optional[torch.Tensor], name: str, shape) -> None:
    """Reject a tensor whose shape is not the one the call will read or write (before any launch:
    the library only sees pointers and sizes)."""
    if x is not None and tuple(x.shape) != tuple(shape):
        raise ValueError(f"{name} must be {list(shape)}, got {list(x.shape)}")


def _expect_2d(x: torch.Tensor, name: str) -> None:
    if not isinstance(x, torch.Tensor) or x.dim() != 2:
        raise ValueError(f"{name} must be a 2-D tensor")


def pack_weight_blocked(W: torch.Tensor, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """The [k, n] weight W re-laid out for W_BLOCKED (64 x 128 blocks, 128-column strips); the
    result is a [k, n] tensor whose memory holds that layout.  k % 64 == 0 and n % 128 == 0."""
    _expect_2d(W, "W")
    k, n = W.shape
    if out is None:
        out = torch.empty((k, n), dtype=torch.bfloat16, device=W.device)
    _expect_shape(out, "out", (k, n))
    _check(_lib.ttl_pack_weight_blocked(_dev_ptr(W, "W"), k, n, _dev_ptr(out, "out"), _stream_handle(stream)))
    return out


def _col_dims(X: torch.Tensor, W: torch.Tensor, w_layout: int, split, t: int, epi: int):
    _expect_2d(X, "X")
    _expect_2d(W, "W")
    b, k = X.shape
    kw, n = _weight_dims(W, w_layout)
    if kw != k:
        raise ValueError(f"X is [{b},{k}] but W is {tuple(W.shape)} (layout {w_layout})")
    width = split_width(split, n, t) if t >= 1 else 0
    ncols = width // 2 if epi == EPI_SILU_MUL else width
    return b, k, n, ncols


def shard_linear_col(X: torch.Tensor, W: torch.Tensor, t: int, rank: int,
                     split: Optional[ColSplit] = None, epi: int = EPI_NONE,
                     Y: Optional[torch.Tensor] = None, stream=None,
                     w_layout: int = W_KN) -> torch.Tensor:
    """Column-parallel output of `rank`: X[b,k] · W[:, C_rank] (optionally SiLU(gate)·up).

    W is the logical [k, n] weight stored as `w_layout` says: a [k, n] tensor (W_KN, the C entry
    point shard_linear_col), its transpose as an [n, k] tensor (W_NK) or the blocked storage
    (W_BLOCKED; both through shard_linear_col_stored)."""
    b, k, n, ncols = _col_dims(X, W, w_layout, split, t, epi)
    if Y is None:
        Y = torch.empty((b, max(ncols, 0)), dtype=torch.bfloat16, device=X.device)
    _expect_shape(Y, "Y", (b, ncols))
    sp = ctypes.byref(split) if split is not None else None
    if w_layout == W_KN:
        st = _lib.shard_linear_col(_dev_ptr(X, "X"), b, k, _dev_ptr(W, "W"), n, t, rank, sp, epi,
                                   _dev_ptr(Y, "Y"), _stream_handle(stream))
    else:
        st = _lib.shard_linear_col_stored(_dev_ptr(X, "X"), b, k, _dev_ptr(W, "W"), n, w_layout, t, rank,
                                          sp, epi, _dev_ptr(Y, "Y"), _stream_handle(stream))
    _check(st)
    return Y


def shard_linear_col_noalloc(X: torch.Tensor, W: torch.Tensor, t: int, rank: int,
                             split: Optional[ColSplit] = None, epi: int = EPI_NONE,
                             Y: Optional[torch.Tensor] = None, stream=None,
                             w_layout: int = W_KN) -> torch.Tensor:
    """shard_linear_col with split-K partials kept in the library's static device scratch instead of
    an allocated workspace (the C entry point shard_linear_col_noalloc).  Pass Y to keep the call
    itself free of allocation."""
    b, k, n, ncols = _col_dims(X, W, w_layout, split, t, epi)
    if Y is None:
        Y = torch.empty((b, max(ncols, 0)), dtype=torch.bfloat16, device=X.device)
    _expect_shape(Y, "Y", (b, ncols))
    _check(_lib.shard_linear_col_noalloc(_dev_ptr(X, "X"), b, k, _dev_ptr(W, "W"), n, w_layout, t, rank,
                                         ctypes.byref(split) if split is not None else None, epi,
                                         _dev_ptr(Y, "Y"), _stream_handle(stream)))
    return Y


def shard_linear_col_gathered(X: torch.Tensor, W: torch.Tensor, t: int, rank: int,
                              split: Optional[ColSplit] = None, epi: int = EPI_NONE,
                              Y_all: Optional[torch.Tensor] = None, stream=None,
                              w_layout: int = W_KN) -> torch.Tensor:
    """Like shard_linear_col with gather_output=True: writes the rank's output into its column block
    [rank*w, (rank+1)*w) of the all-gathered Y_all[b, t*w]."""
    b, k, n, ncols = _col_dims(X, W, w_layout, split, t, epi)
    if Y_all is None:
        Y_all = torch.empty((b, max(ncols * t, 0)), dtype=torch.bfloat16, device=X.device)
    _expect_shape(Y_all, "Y_all", (b, ncols * t))
    _check(_lib.shard_linear_col_gathered(_dev_ptr(X, "X"), b, k, _dev_ptr(W, "W"), n, w_layout, t, rank,
                                          ctypes.byref(split) if split is not None else None, epi,
                                          _dev_ptr(Y_all, "Y_all"), _stream_handle(stream)))
    return Y_all


def shard_linear_row(X: torch.Tensor, W: torch.Tensor, t: int, rank: int,
                     x_is_parallel: bool = True, P: Optional[torch.Tensor] = None,
                     stream=None, w_layout: int = W_KN) -> torch.Tensor:
    """Row-parallel partial of `rank`: X_rank · W[rank*k/t:(rank+1)*k/t, :] (W stored per w_layout;
    W_KN through the C entry point shard_linear_row, the others through shard_linear_row_stored).
    X is [b, k/t] when x_is_parallel, else the full [b, k]."""
    _expect_2d(X, "X")
    _expect_2d(W, "W")
    k, n = _weight_dims(W, w_layout)
    b = X.shape[0]
    if t >= 1 and k % t == 0:  # otherwise the library rejects the split (NOT_DIVISIBLE)
        _expect_shape(X, "X", (b, k // t if x_is_parallel else k))
    if P is None:
        P = torch.empty((b, n), dtype=torch.bfloat16, device=X.device)
    _expect_shape(P, "P", (b, n))
    if w_layout == W_KN:
        st = _lib.shard_linear_row(_dev_ptr(X, "X"), b, k, 1 if x_is_parallel else 0, _dev_ptr(W, "W"), n,
                                   t, rank, _dev_ptr(P, "P"), _stream_handle(stream))
    else:
        st = _lib.shard_linear_row_stored(_dev_ptr(X, "X"), b, k, 1 if x_is_parallel else 0, _dev_ptr(W, "W"),
                                          n, w_layout, t, rank, _dev_ptr(P, "P"), _stream_handle(stream))
    _check(st)
    return P


def reduce_partials_rmsnorm(P: torch.Tensor, gamma: torch.Tensor, eps: float,
                            residual: Optional[torch.Tensor] = None,
                            residual_out: Optional[torch.Tensor] = None,
                            Y: Optional[torch.Tensor] = None,
                            stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Sum of the t partials P[t,b,n] + residual, then RMSNorm; returns (residual_out, Y)."""
    if not isinstance(P, torch.Tensor) or P.dim() != 3:
        raise ValueError("P must be a 3-D [t, b, n] tensor")
    t, b, n = P.shape
    if residual_out is None:
        residual_out = torch.empty((b, n), dtype=torch.bfloat16, device=P.device)
    if Y is None:
        Y = torch.empty((b, n), dtype=torch.bfloat16, device=P.device)
    for x, name, shape in ((residual, "residual", (b, n)), (gamma, "gamma", (n,)),
                           (residual_out, "residual_out", (b, n)), (Y, "Y", (b, n))):
        _expect_shape(x, name, shape)
    _check(_lib.reduce_partials_rmsnorm(_dev_ptr(P, "P"), t, b, n, _dev_ptr(residual, "residual"),
                                        _dev_ptr(gamma, "gamma"), float(eps),
                                        _dev_ptr(residual_out, "residual_out"), _dev_ptr(Y, "Y"),
                                        _stream_handle(stream)))
    return residual_out, Y


def reduce_scatter_partials_rmsnorm(P: torch.Tensor, gamma: torch.Tensor, eps: float, rank: int,
                                    residual: Optional[torch.Tensor] = None,
                                    residual_out: Optional[torch.Tensor] = None,
                                    Y: Optional[torch.Tensor] = None,
                                    stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Sequence-parallel reduction: rank `rank`'s chunk of b/t rows of the sum of P[t,b,n] + its
    residual shard, then RMSNorm; returns (residual_out, Y), each [b/t, n]."""
    if not isinstance(P, torch.Tensor) or P.dim() != 3:
        raise ValueError("P must be a 3-D [t, b, n] tensor")
    t, b, n = P.shape
    rows = b // t if t > 0 else 0
    if residual_out is None:
        residual_out = torch.empty((rows, n), dtype=torch.bfloat16, device=P.device)
    if Y is None:
        Y = torch.empty((rows, n), dtype=torch.bfloat16, device=P.device)
    if t > 0 and b % t == 0:  # otherwise the library rejects the row split (NOT_DIVISIBLE)
        for x, name, shape in ((residual, "residual", (rows, n)), (residual_out, "residual_out", (rows, n)),
                               (Y, "Y", (rows, n))):
            _expect_shape(x, name, shape)
    _expect_shape(gamma, "gamma", (n,))
    _check(_lib.reduce_scatter_partials_rmsnorm(_dev_ptr(P, "P"), t, b, n, rank,
                                                _dev_ptr(residual, "residual"), _dev_ptr(gamma, "gamma"),
                                                float(eps), _dev_ptr(residual_out, "residual_out"),
                                                _dev_ptr(Y, "Y"), _stream_handle(stream)))
    return residual_out, Y


def reduce_partials_rmsnorm_peers(P_ranks, gamma: torch.Tensor, eps: float, row0: int = 0,
                                  rows: Optional[int] = None,
                                  residual: Optional[torch.Tensor] = None,
                                  residual_out: Optional[torch.Tensor] = None,
                                  Y: Optional[torch.Tensor] = None,
                                  stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """The reduction over rows [row0, row0 + rows) of t partials held in t separate [b, n]
    tensors (one per rank); returns (residual_out, Y), each [rows, n]."""
    P_ranks = list(P_ranks)
    t = len(P_ranks)
    b, n = P_ranks[0].shape if t else (0, 0)
    for P in P_ranks:
        if tuple(P.shape) != (b, n):
            raise ValueError(f"every partial must be [{b}, {n}], got {tuple(P.shape)}")
    rows = b - row0 if rows is None else rows
    dev = P_ranks[0].device if t else gamma.device
    if residual_out is None:
        residual_out = torch.empty((max(rows, 0), n), dtype=torch.bfloat16, device=dev)
    if Y is None:
        Y = torch.empty((max(rows, 0), n), dtype=torch.bfloat16, device=dev)
    for x, name, shape in ((residual, "residual", (rows, n)), (gamma, "gamma", (n,)),
                           (residual_out, "residual_out", (rows, n)), (Y, "Y", (rows, n))):
        _expect_shape(x, name, shape)
    ptrs = (ctypes.c_void_p * max(t, 1))(*[_dev_ptr(P, f"P_ranks[{r}]") for r, P in enumerate(P_ranks)])
    _check(_lib.reduce_partials_rmsnorm_peers(ptrs, t, b, n, row0, rows, _dev_ptr(residual, "residual"),
                                              _dev_ptr(gamma, "gamma"), float(eps),
                                              _dev_ptr(residual_out, "residual_out"), _dev_ptr(Y, "Y"),
                                              _stream_handle(stream)))
    return residual_out, Y


def version() -> int:
    return int(_lib.ttl_version())


def set_gemm_override(kernel: str = "auto", splits: int = 0, plan_cus: int = 0, trace: bool = False) -> None:
    """Force a GEMM kernel family for every later call in the process (tests and measurements only;
    ttl_set_gemm_override).  kernel="auto", splits=0, plan_cus=0 restore the choice by shape."""
    if kernel not in GEMM_KERNELS:
        raise ValueError(f"unknown kernel family {kernel!r}; one of {sorted(GEMM_KERNELS)}")
    _check(_lib.ttl_set_gemm_override(GEMM_KERNELS[kernel], int(splits), int(plan_cus), 1 if trace else 0))


@contextlib.contextmanager
def gemm_override(kernel: str = "auto", splits: int = 0, plan_cus: int = 0, trace: bool = False):
    """set_gemm_override for the duration of a with-block, then the choice by shape again."""
    set_gemm_override(kernel, splits, plan_cus, trace)
    try:
        yield
    finally:
        set_gemm_override()
