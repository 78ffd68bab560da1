"""The C ABI without a GPU: the library loads, exports every entry point the header declares, and
rejects bad arguments with the documented status before touching the device.

Every call below fails validation, so no kernel is launched and no HIP call is made.  Pointers are
fake, suitably aligned integers that are never dereferenced.
"""

import os
import re
import subprocess

import pytest

from tensor_transformer_linear_amd import ttl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ttl.h")

A, B, C, D = 0x10000, 0x20000, 0x30000, 0x40000  # fake 16-byte-aligned device addresses


def _gpu_present():
    import torch
    return torch.cuda.device_count() > 0  # counts devices without initialising one


# With a GPU present, a validation rule that regressed would launch a kernel on the fake pointers;
# these checks therefore run only where there is no device.
no_device = pytest.mark.skipif(_gpu_present(), reason="passes fake device pointers; CPU-only check")


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:ttl_status|const char\*|int32_t)\s+(\w+)\s*\(", text, re.M)))


def test_header_declares_the_boundary():
    assert declared_functions() == sorted(ttl.EXPORTED)


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", ttl.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(ttl.lib(), name)


def test_status_codes_match_header():
    text = open(HEADER).read()
    codes = dict((m[0], int(m[1])) for m in re.findall(r"#define (TTL_\w+) (\d+)", text))
    assert codes["TTL_OK"] == ttl.OK
    assert codes["TTL_ERR_NULL"] == ttl.ERR_NULL
    assert codes["TTL_ERR_SHAPE"] == ttl.ERR_SHAPE
    assert codes["TTL_ERR_NOT_DIVISIBLE"] == ttl.ERR_NOT_DIVISIBLE
    assert codes["TTL_ERR_RANK"] == ttl.ERR_RANK
    assert codes["TTL_ERR_ALIGN"] == ttl.ERR_ALIGN
    assert codes["TTL_ERR_UNSUPPORTED"] == ttl.ERR_UNSUPPORTED
    assert codes["TTL_ERR_HIP"] == ttl.ERR_HIP
    assert codes["TTL_EPI_SILU_MUL"] == ttl.EPI_SILU_MUL
    assert codes["TTL_W_KN"] == ttl.W_KN and codes["TTL_W_NK"] == ttl.W_NK
    assert codes["TTL_W_BLOCKED"] == ttl.W_BLOCKED
    assert codes["TTL_MAX_SEGMENTS"] == ttl.MAX_SEGMENTS
    assert ttl.version() >= 100


def _col(X=A, b=16, k=256, W=B, n=1376, t=2, rank=0, split=None, epi=0, Y=C, lay=None):
    """shard_linear_col (the [k][n] form of the statement) when lay is None, else
    shard_linear_col_stored with that storage."""
    sp = None if split is None else ttl.ctypes.byref(split)
    if lay is None:
        return ttl.lib().shard_linear_col(X, b, k, W, n, t, rank, sp, epi, Y, None)
    return ttl.lib().shard_linear_col_stored(X, b, k, W, n, lay, t, rank, sp, epi, Y, None)


def _colg(X=A, b=16, k=256, W=B, n=1376, t=2, rank=0, split=None, epi=0, Y=C, lay=0):
    sp = None if split is None else ttl.ctypes.byref(split)
    return ttl.lib().shard_linear_col_gathered(X, b, k, W, n, lay, t, rank, sp, epi, Y, None)


def _noalloc(X=A, b=16, k=256, W=B, n=1376, t=2, rank=0, split=None, epi=0, Y=C, lay=0):
    sp = None if split is None else ttl.ctypes.byref(split)
    return ttl.lib().shard_linear_col_noalloc(X, b, k, W, n, lay, t, rank, sp, epi, Y, None)


def _rs(P=A, t=2, b=16, n=256, rank=0, R=B, gamma=D, eps=1e-5, Rout=B, Y=C):
    return ttl.lib().reduce_scatter_partials_rmsnorm(P, t, b, n, rank, R, gamma, eps, Rout, Y, None)


def _row(X=A, b=16, k=688, par=1, W=B, n=256, t=2, rank=0, P=C, lay=None):
    if lay is None:
        return ttl.lib().shard_linear_row(X, b, k, par, W, n, t, rank, P, None)
    return ttl.lib().shard_linear_row_stored(X, b, k, par, W, n, lay, t, rank, P, None)


# far-apart fake buffers for the overlap rules (the defaults above sit 64 KiB apart)
FX, FW, FY = 0x1000000, 0x2000000, 0x3000000


def _pack(W=A, k=256, n=1024, out=B):
    return ttl.lib().ttl_pack_weight_blocked(W, k, n, out, None)


def _red(P=A, t=2, b=16, n=256, R=B, gamma=D, eps=1e-5, Rout=B, Y=C):
    return ttl.lib().reduce_partials_rmsnorm(P, t, b, n, R, gamma, eps, Rout, Y, None)


PEERS = [0x100000 + 0x10000 * r for r in range(17)]  # fake, 16-byte aligned, 64 KiB apart


def _peers(ptrs=None, t=2, b=16, n=256, row0=0, rows=16, R=B, gamma=D, eps=1e-5, Rout=B, Y=C):
    ptrs = PEERS[:t] if ptrs is None else ptrs
    arr = None if ptrs == "null" else (ttl.ctypes.c_void_p * max(len(ptrs), 1))(*ptrs)
    return ttl.lib().reduce_partials_rmsnorm_peers(arr, t, b, n, row0, rows, R, gamma, eps, Rout, Y, None)


@pytest.mark.parametrize("call,status,needle", [
    (lambda: _col(X=None), ttl.ERR_NULL, "non-NULL"),
    (lambda: _col(Y=None), ttl.ERR_NULL, "non-NULL"),
    (lambda: _col(b=0), ttl.ERR_SHAPE, "b=0"),
    (lambda: _col(k=-8), ttl.ERR_SHAPE, ""),
    (lambda: _col(t=0), ttl.ERR_RANK, "t=0"),
    (lambda: _col(rank=2), ttl.ERR_RANK, "rank=2"),
    (lambda: _col(rank=-1), ttl.ERR_RANK, ""),
    (lambda: _col(n=1370, t=4), ttl.ERR_NOT_DIVISIBLE, "not divisible"),
    (lambda: _col(split=ttl.make_split((688, 680), (2, 2))), ttl.ERR_NOT_DIVISIBLE, "sum to 1368"),
    (lambda: _col(split=ttl.make_split((688, 688), (2, 3)), t=6), ttl.ERR_NOT_DIVISIBLE, "divisible by 3"),
    (lambda: _col(split=ttl.make_split((688, 688), (4, 4)), t=2), ttl.ERR_NOT_DIVISIBLE, "divisor"),
    (lambda: _col(X=A + 8), ttl.ERR_ALIGN, "aligned"),
    (lambda: _col(k=252), ttl.ERR_ALIGN, "multiples of 8"),
    (lambda: _col(n=1376, t=4, split=ttl.make_split((688, 688), (4, 4))), ttl.ERR_ALIGN, "slice width 172"),
    (lambda: _col(epi=1), ttl.ERR_UNSUPPORTED, "two equal segments"),
    (lambda: _col(epi=1, split=ttl.make_split((704, 672), (2, 2))), ttl.ERR_UNSUPPORTED, "two equal"),
    (lambda: _col(epi=7), ttl.ERR_UNSUPPORTED, "epilogue"),
    (lambda: _col(lay=3), ttl.ERR_UNSUPPORTED, "weight layout"),
    (lambda: _col(lay=ttl.W_KN, X=None), ttl.ERR_NULL, "shard_linear_col_stored"),
    (lambda: _col(X=FX, W=FW, Y=FW + 4096), ttl.ERR_UNSUPPORTED, "overlap"),       # Y inside W
    (lambda: _col(X=FX, W=FW, Y=FX + 16), ttl.ERR_UNSUPPORTED, "overlap"),         # Y inside X
    (lambda: _col(X=FX, W=FW, Y=FW - 16, lay=ttl.W_NK, n=1376, k=256), ttl.ERR_UNSUPPORTED, "overlap"),
    (lambda: _colg(X=FX, W=FW, Y=FX + 32), ttl.ERR_UNSUPPORTED, "overlap"),
    (lambda: _row(X=FX, W=FW, P=FW + 1024), ttl.ERR_UNSUPPORTED, "overlap"),       # P inside W
    (lambda: _row(X=FX, W=FW, P=FX + 16, par=0), ttl.ERR_UNSUPPORTED, "overlap"),  # P inside full X
    (lambda: _row(X=FX, W=FW, P=FW + 1024, lay=ttl.W_NK), ttl.ERR_UNSUPPORTED, "overlap"),
    (lambda: _col(lay=ttl.W_BLOCKED), ttl.ERR_ALIGN, "blocked weight"),          # n % 128 != 0
    (lambda: _col(k=200, n=1536, lay=ttl.W_BLOCKED), ttl.ERR_ALIGN, "blocked weight"),
    (lambda: _col(k=16384, n=131072, t=1, lay=ttl.W_BLOCKED), ttl.ERR_UNSUPPORTED, "2 GiB"),
    (lambda: _col(k=16384, n=65536, t=1, lay=1), ttl.ERR_UNSUPPORTED, "2 GiB"),
    (lambda: _col(k=16384, n=131072, t=2, lay=1), ttl.ERR_UNSUPPORTED, "2 GiB"),
    (lambda: _noalloc(X=None), ttl.ERR_NULL, "shard_linear_col_noalloc"),
    (lambda: _noalloc(rank=2), ttl.ERR_RANK, "rank=2"),
    (lambda: _noalloc(epi=1), ttl.ERR_UNSUPPORTED, "two equal segments"),
    (lambda: _noalloc(lay=3), ttl.ERR_UNSUPPORTED, "weight layout"),
    (lambda: _noalloc(X=FX, W=FW, Y=FW + 4096), ttl.ERR_UNSUPPORTED, "overlap"),
    (lambda: _colg(Y=None), ttl.ERR_NULL, "non-NULL"),
    (lambda: _colg(rank=2), ttl.ERR_RANK, "rank=2"),
    (lambda: _colg(n=1370, t=4), ttl.ERR_NOT_DIVISIBLE, "not divisible"),
    (lambda: _colg(epi=1), ttl.ERR_UNSUPPORTED, "two equal segments"),
    (lambda: _colg(k=252), ttl.ERR_ALIGN, "multiples of 8"),
    (lambda: _row(lay=-1), ttl.ERR_UNSUPPORTED, "weight layout"),
    (lambda: _row(lay=ttl.W_KN, P=None), ttl.ERR_NULL, "shard_linear_row_stored"),
    (lambda: ttl.lib().ttl_set_gemm_override(13, 0, 0, 0), ttl.ERR_UNSUPPORTED, "unknown kernel"),
    (lambda: ttl.lib().ttl_set_gemm_override(2, -1, 0, 0), ttl.ERR_UNSUPPORTED, "splits=-1"),
    (lambda: ttl.lib().ttl_set_gemm_override(0, 0, -4, 0), ttl.ERR_UNSUPPORTED, "plan_cus=-4"),
    (lambda: _row(lay=ttl.W_BLOCKED), ttl.ERR_ALIGN, "blocked weight"),          # k % 64 != 0
    (lambda: _row(k=1024, t=32, lay=ttl.W_BLOCKED), ttl.ERR_ALIGN, "blocked weight"),  # k/t = 32
    (lambda: _row(k=16384, n=65536, t=1, lay=ttl.W_BLOCKED), ttl.ERR_UNSUPPORTED, "2 GiB"),
    (lambda: _pack(W=None), ttl.ERR_NULL, "non-NULL"),
    (lambda: _pack(k=0), ttl.ERR_SHAPE, ""),
    (lambda: _pack(k=65536, n=65536), ttl.ERR_SHAPE, "2^31"),
    (lambda: _pack(k=100), ttl.ERR_ALIGN, "k % 64"),
    (lambda: _pack(n=1000), ttl.ERR_ALIGN, "n % 128"),
    (lambda: _pack(out=B + 8), ttl.ERR_ALIGN, "aligned"),
    (lambda: _pack(out=A + 16), ttl.ERR_UNSUPPORTED, "overlap"),
    (lambda: _row(P=None), ttl.ERR_NULL, "non-NULL"),
    (lambda: _row(n=0), ttl.ERR_SHAPE, ""),
    (lambda: _row(rank=5), ttl.ERR_RANK, ""),
    (lambda: _row(k=689), ttl.ERR_NOT_DIVISIBLE, "not divisible"),
    (lambda: _row(k=680, t=4), ttl.ERR_ALIGN, "k/t=170"),
    (lambda: _row(W=B + 2), ttl.ERR_ALIGN, "aligned"),
    (lambda: _red(P=None), ttl.ERR_NULL, ""),
    (lambda: _red(gamma=None), ttl.ERR_NULL, ""),
    (lambda: _red(t=0), ttl.ERR_RANK, ""),
    (lambda: _red(n=65544), ttl.ERR_SHAPE, "65536"),
    (lambda: _red(b=0), ttl.ERR_SHAPE, ""),
    (lambda: _red(eps=-1.0), ttl.ERR_SHAPE, "eps"),
    (lambda: _red(n=252), ttl.ERR_ALIGN, "multiple of 8"),
    (lambda: _red(Y=C + 4), ttl.ERR_ALIGN, "aligned"),
    (lambda: _red(Y=A + 16), ttl.ERR_UNSUPPORTED, "overlap"),
    (lambda: _red(Rout=A), ttl.ERR_UNSUPPORTED, "alias"),
    (lambda: _red(R=B, Rout=B + 16), ttl.ERR_UNSUPPORTED, "alias"),
    (lambda: _peers(t=0), ttl.ERR_RANK, "t=0"),
    (lambda: _peers(t=17), ttl.ERR_UNSUPPORTED, "17"),
    (lambda: _peers(ptrs="null"), ttl.ERR_NULL, "P_ranks"),
    (lambda: _peers(ptrs=[PEERS[0], None]), ttl.ERR_NULL, "P_ranks[1]"),
    (lambda: _peers(ptrs=[PEERS[0], PEERS[1] + 8]), ttl.ERR_ALIGN, "P_ranks[1]"),
    (lambda: _peers(b=0), ttl.ERR_SHAPE, ""),
    (lambda: _peers(row0=8, rows=9), ttl.ERR_SHAPE, "rows [8, 17)"),
    (lambda: _peers(rows=0), ttl.ERR_SHAPE, ""),
    (lambda: _peers(row0=-1), ttl.ERR_SHAPE, ""),
    (lambda: _peers(n=252), ttl.ERR_ALIGN, "multiple of 8"),
    (lambda: _peers(gamma=None), ttl.ERR_NULL, ""),
    (lambda: _peers(Y=PEERS[1] + 64), ttl.ERR_UNSUPPORTED, "P_ranks[1]"),
    (lambda: _peers(Rout=PEERS[0]), ttl.ERR_UNSUPPORTED, ""),
    (lambda: _rs(P=None), ttl.ERR_NULL, ""),
    (lambda: _rs(rank=2), ttl.ERR_RANK, "rank=2"),
    (lambda: _rs(rank=-1), ttl.ERR_RANK, ""),
    (lambda: _rs(b=15), ttl.ERR_NOT_DIVISIBLE, "not divisible by t=2"),
    (lambda: _rs(n=65544), ttl.ERR_SHAPE, "65536"),
    (lambda: _rs(n=252), ttl.ERR_ALIGN, "multiple of 8"),
    (lambda: _rs(Y=A + 16), ttl.ERR_UNSUPPORTED, "overlap"),
], ids=lambda v: v if isinstance(v, (int, str)) else "")
@no_device
def test_validation_rejects_before_launch(call, status, needle):
    got = call()
    assert got == status, (got, ttl.last_error())
    assert needle in ttl.last_error()


def test_binding_refuses_host_tensors():
    import torch
    X = torch.zeros(16, 256, dtype=torch.bfloat16)
    W = torch.zeros(256, 1376, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        ttl.shard_linear_col(X, W, 2, 0, ttl.merged_gate_up_split(688, 2), ttl.EPI_SILU_MUL)
    with pytest.raises(TypeError, match="bfloat16"):
        ttl.shard_linear_row(X[:, :128].float().contiguous(), W, 2, 0)


@no_device
def test_noalloc_refuses_a_call_beyond_its_scratch():
    """A call whose split-K partials would exceed the static scratch (64 k-splits of 256 x 16384
    fp32 = 1 GiB) is refused before anything is launched: the plan is sized by a dry pass."""
    with ttl.gemm_override("splitk", splits=64):
        got = _noalloc(X=FX, b=256, k=8192, W=FW, n=16384, t=1, Y=0x40000000)
    assert got == ttl.ERR_UNSUPPORTED, (got, ttl.last_error())
    assert "static scratch" in ttl.last_error() and str(64 * 256 * 16384 * 4) in ttl.last_error()
    assert ttl.NOALLOC_SCRATCH_BYTES == 64 << 20


def test_exact_and_stored_forms_validate_alike():
    """The statement's [k][n] form and the storage-taking form apply the same rules."""
    for kw in (dict(b=0), dict(rank=3), dict(n=1370, t=4), dict(X=A + 8)):
        assert _col(**kw) == _col(lay=ttl.W_KN, **kw)
    for kw in (dict(k=689), dict(rank=2), dict(P=None)):
        assert _row(**kw) == _row(lay=ttl.W_KN, **kw)


def _cpu(*shape):
    import torch
    return torch.zeros(*shape, dtype=torch.bfloat16)


@pytest.mark.parametrize("call,needle", [
    # caller-supplied outputs of the wrong shape
    (lambda: ttl.shard_linear_col(_cpu(16, 256), _cpu(256, 1376), 2, 0, ttl.merged_gate_up_split(688, 2),
                                  ttl.EPI_SILU_MUL, Y=_cpu(16, 688)), "Y must be [16, 344]"),
    (lambda: ttl.shard_linear_col(_cpu(16, 256), _cpu(256, 1376), 2, 0, Y=_cpu(8, 688)), "Y must be [16, 688]"),
    (lambda: ttl.shard_linear_col_gathered(_cpu(16, 256), _cpu(256, 1376), 2, 1, Y_all=_cpu(16, 688)),
     "Y_all must be [16, 1376]"),
    (lambda: ttl.shard_linear_row(_cpu(16, 344), _cpu(688, 256), 2, 0, P=_cpu(16, 255)), "P must be [16, 256]"),
    # the row GEMM's input must be [b, k/t] (parallel) or [b, k] (full)
    (lambda: ttl.shard_linear_row(_cpu(16, 344), _cpu(688, 256), 2, 0, x_is_parallel=False), "X must be [16, 688]"),
    (lambda: ttl.shard_linear_row(_cpu(16, 688), _cpu(688, 256), 2, 0, x_is_parallel=True), "X must be [16, 344]"),
    (lambda: ttl.shard_linear_row(_cpu(16, 688), _cpu(256, 688), 2, 0, x_is_parallel=False, w_layout=ttl.W_NK,
                                  P=_cpu(16, 200)), "P must be [16, 256]"),
    # X and W disagree on k
    (lambda: ttl.shard_linear_col(_cpu(16, 200), _cpu(256, 1376), 2, 0), "X is [16,200]"),
    # the reduction's operands
    (lambda: ttl.reduce_partials_rmsnorm(_cpu(2, 16, 256), _cpu(255), 1e-5), "gamma must be [256]"),
    (lambda: ttl.reduce_partials_rmsnorm(_cpu(2, 16, 256), _cpu(256), 1e-5, residual=_cpu(16, 128)),
     "residual must be [16, 256]"),
    (lambda: ttl.reduce_partials_rmsnorm(_cpu(2, 16, 256), _cpu(256), 1e-5, Y=_cpu(15, 256)), "Y must be [16, 256]"),
    (lambda: ttl.reduce_partials_rmsnorm(_cpu(16, 256), _cpu(256), 1e-5), "3-D"),
    (lambda: ttl.reduce_scatter_partials_rmsnorm(_cpu(2, 16, 256), _cpu(256), 1e-5, 0, residual=_cpu(16, 256)),
     "residual must be [8, 256]"),
    (lambda: ttl.reduce_partials_rmsnorm_peers([_cpu(16, 256)] * 2, _cpu(256), 1e-5, row0=8, rows=8,
                                               Y=_cpu(16, 256)), "Y must be [8, 256]"),
    (lambda: ttl.pack_weight_blocked(_cpu(256, 1024), out=_cpu(1024, 256)), "out must be [256, 1024]"),
])
def test_binding_checks_shapes_before_any_call(call, needle):
    """Every tensor's shape is checked against the sizes the call will read and write before the C
    entry point is reached: these host tensors would otherwise be refused later, as host memory."""
    with pytest.raises(ValueError, match=re.escape(needle)):
        call()


def test_gemm_override_setter():
    """The test-only kernel override is set and cleared through its entry point; no environment
    variable is read by the library."""
    with ttl.gemm_override("splitk", splits=3):
        pass
    with pytest.raises(ValueError):
        ttl.set_gemm_override("bogus")
    out = subprocess.run(["nm", "-D", "--undefined-only", ttl.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    assert "getenv" not in out


def test_split_helpers_match_header_rule():
    sp = ttl.qkv_split(64, 8, 128, 8)
    assert ttl.split_width(sp, 10240, 8) == 1280
    sp = ttl.qkv_split(32, 4, 128, 8)
    assert [sp.seg_parts[i] for i in range(3)] == [8, 4, 4]
    assert ttl.split_width(ttl.merged_gate_up_split(28672, 8), 57344, 8) == 7168
