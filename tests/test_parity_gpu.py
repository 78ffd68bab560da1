"""Parity of the HIP path (through the C ABI) with the CPU oracle, on seeded synthetic inputs.

Small cases compare every element; they span several 256-wide tiles and ragged tails in all three
GEMM dimensions.  Each GEMM case runs through every kernel the library has, forced with
the library's test-only override (256 x 256 tiles by the four-wave kernel where K is a multiple of 64, by the
eight-wave kernel, the four-wave kernel's tiles cut along k, its 256 x 128 tiles, its 192 x 256
tiles, and the split-K kernel for short M), and through the shape-based choice; the split-free kernel for
[n][k] weights and few rows has tests of its own.  Tolerance, per output tensor: the error beyond the bf16 rounding of each output
element is at most 2e-2 * rms(ref), the reference being the oracle's unrounded float64 value (bf16
inputs, so the device-side error is fp32 accumulation and fp32 elementwise math).  Integer-exact
special cases (identity and one-hot operands) are compared bit for bit.
"""

import numpy as np
import pytest
import torch

import oracle
from tensor_transformer_linear_amd import workloads as wl
from tests.util import assert_close, f64, from_gpu, gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ttl():
    from tensor_transformer_linear_amd import ttl as lib
    assert torch.cuda.is_available()
    return lib


LAYOUTS = pytest.mark.parametrize("layout", ["kn", "nk"])


@pytest.fixture(params=["auto", "tiled", "tiled16", "eightwave", "tilesplit", "narrow", "short", "splitk"])
def gemm_path(request, gemm_force):
    """Which GEMM kernel the library uses for the test (auto = its choice by shape)."""
    if request.param == "auto":
        gemm_force.set(kernel="auto")
    else:
        gemm_force.set(kernel=request.param)
    gemm_force.set(splits=0)
    return request.param


def _stored(ttl, W, layout):
    """Device copy of the logical W[k, n] in the requested storage layout."""
    return (gpu(W), ttl.W_KN) if layout == "kn" else (gpu(W.t().contiguous()), ttl.W_NK)


def _col_case(ttl, b, k, split_np, split_c, t, seed, epi=0, layout="kn"):
    n = sum(split_np[0])
    X = wl.random_bf16((b, k), seed)
    W = wl.random_bf16((k, n), seed + 1, std=0.05)
    Xd = gpu(X)
    Wd, lay = _stored(ttl, W, layout)
    Xo, Wo = f64(X), f64(W)
    for r in range(t):
        Y = ttl.shard_linear_col(Xd, Wd, t, r, split_c, epi, w_layout=lay)
        ref = oracle.col_shard(Xo, Wo, split_np, t, r)
        if epi == ttl.EPI_SILU_MUL:
            ref = oracle.silu_mul(ref)
        assert_close(from_gpu(Y), ref, f"col b={b} k={k} n={n} t={t} r={r} epi={epi} {layout}")


@pytest.mark.parametrize("b,k,I,t", [
    (16, 256, 688, 2),      # the tiny workload's gate_up shape
    (1, 64, 128, 2),        # single row, one k-tile
    (300, 200, 344, 1),     # ragged in M (300), K (200) and N (344 act columns)
    (257, 512, 1024, 4),    # one row past a 256 tile
    (513, 1024, 2048, 8),   # several tiles in every dimension
])
@LAYOUTS
def test_col_silu_mul(ttl, gemm_path, b, k, I, t, layout):
    _col_case(ttl, b, k, oracle.merged_gate_up_split(I, t), ttl.merged_gate_up_split(I, t), t,
              seed=10 + b, epi=ttl.EPI_SILU_MUL, layout=layout)


@pytest.mark.parametrize("b,k,n,t", [(16, 256, 1376, 2), (300, 136, 520, 1), (260, 512, 2048, 4)])
@LAYOUTS
def test_col_plain(ttl, gemm_path, b, k, n, t, layout):
    _col_case(ttl, b, k, oracle.plain_split(n, t), None, t, seed=20 + b, layout=layout)


@pytest.mark.parametrize("b,k,nq,nkv,hd,t", [
    (70, 256, 8, 4, 32, 4),    # t == n_kv
    (70, 256, 16, 8, 16, 4),   # t < n_kv: 2 kv heads per rank
    (33, 128, 8, 2, 32, 4),    # t > n_kv: one kv head per rank, replicated twice
    (300, 512, 32, 8, 128, 4), # the 8B attention head layout at a small batch
])
@LAYOUTS
def test_col_qkv(ttl, gemm_path, b, k, nq, nkv, hd, t, layout):
    _col_case(ttl, b, k, oracle.qkv_split(nq, nkv, hd, t), ttl.qkv_split(nq, nkv, hd, t), t, seed=30 + b,
              layout=layout)


@pytest.mark.parametrize("b,k,n,t", [(16, 688, 256, 2), (300, 344, 520, 1), (257, 1024, 768, 4),
                                     (5, 2048, 264, 8)])
@pytest.mark.parametrize("x_is_parallel", [True, False])
@LAYOUTS
def test_row(ttl, gemm_path, b, k, n, t, x_is_parallel, layout):
    w = k // t
    X = wl.random_bf16((b, k), 40 + b)
    W = wl.random_bf16((k, n), 41 + b, std=0.05)
    Xd = gpu(X)
    Wd, lay = _stored(ttl, W, layout)
    Xo, Wo = f64(X), f64(W)
    for r in range(t):
        xin = Xd[:, r * w:(r + 1) * w].contiguous() if x_is_parallel else Xd
        P = ttl.shard_linear_row(xin, Wd, t, r, x_is_parallel, w_layout=lay)
        ref = oracle.row_shard(Xo, Wo, t, r, x_is_parallel=False)
        assert_close(from_gpu(P), ref, f"row b={b} k={k} n={n} t={t} r={r} par={x_is_parallel} {layout}")


@pytest.mark.parametrize("t,b,n,with_residual", [(2, 16, 256, True), (8, 5, 4096, True),
                                                  (1, 3, 8, True), (4, 33, 8192, False),
                                                  (3, 7, 4104, True), (2, 4, 16384, True),
                                                  (2, 2, 65536, True),
                                                  # the many-row launch shapes of n = 4096 and 8192
                                                  (4, 1100, 4096, True), (2, 2600, 4096, False),
                                                  (8, 1030, 8192, True), (3, 4100, 8192, True)])
def test_reduce_rmsnorm(ttl, t, b, n, with_residual):
    P = wl.random_bf16((t, b, n), 50 + n)
    R = wl.random_bf16((b, n), 51 + n) if with_residual else None
    gamma = wl.random_bf16((n,), 52 + n, mean=1.0, std=0.1)
    Rd = gpu(R) if with_residual else None
    rout, y = ttl.reduce_partials_rmsnorm(gpu(P), gpu(gamma), 1e-5, Rd)
    h, yref = oracle.reduce_partials_rmsnorm(f64(P), f64(R) if with_residual else None, f64(gamma), 1e-5)
    assert_close(from_gpu(rout), h, f"reduce residual_out t={t} b={b} n={n}", literal=True)
    assert_close(from_gpu(y), yref, f"reduce y t={t} b={b} n={n}", literal=True)


def test_reduce_residual_in_place(ttl):
    t, b, n = 4, 9, 1024
    P, R = wl.random_bf16((t, b, n), 60), wl.random_bf16((b, n), 61)
    gamma = wl.random_bf16((n,), 62, mean=1.0, std=0.1)
    Rd = gpu(R)
    rout, y = ttl.reduce_partials_rmsnorm(gpu(P), gpu(gamma), 1e-5, Rd, residual_out=Rd)
    assert rout.data_ptr() == Rd.data_ptr()
    h, yref = oracle.reduce_partials_rmsnorm(f64(P), f64(R), f64(gamma), 1e-5)
    assert_close(from_gpu(Rd), h, "in-place residual", literal=True)
    assert_close(from_gpu(y), yref, "in-place y", literal=True)


@pytest.mark.parametrize("case", ["col_k_max", "col_k_max_nk", "col_n_max", "row_k_max"])
@pytest.mark.parametrize("kern", ["auto", "tiled"])
def test_maximum_row_pitches(ttl, gemm_force, case, kern):
    """The largest row pitches the ABI accepts: X rows of k = 2^21 elements (the row GEMM reading
    the upper half of each row), and W rows of n = 2^23 columns.  Every 32-bit byte offset inside a
    tile is then within a factor of two of its limit; sampled outputs match the oracle."""
    gemm_force.set(splits=0)
    if kern == "auto":
        gemm_force.set(kernel="auto")
    else:
        gemm_force.set(kernel=kern)
    if case == "col_n_max":
        b, k, n = 8, 64, 1 << 23
    else:
        b, k, n = 260, 1 << 21, 128
    X = wl.random_bf16((b, k), 300, device="cuda")
    W = wl.random_bf16((k, n), 301, std=0.02, device="cuda")
    rows = [0, 1, 127, 128, 255, 256, b - 1] if b > 256 else list(range(b))
    if case == "row_k_max":
        t, r = 2, 1
        P = ttl.shard_linear_row(X, W, t, r, False)
        ref = oracle.row_shard(from_gpu(X[rows]), from_gpu(W), t, r, x_is_parallel=False)
        assert_close(from_gpu(P[rows]), ref, f"row k=2^21 {kern}")
        return
    if case == "col_n_max":
        gen = np.random.default_rng(302)
        cols = np.r_[0:64, n - 64:n, np.sort(gen.choice(np.arange(64, n - 64), 64, replace=False))]
        Y = ttl.shard_linear_col(X, W, 1, 0)
        Wc = W[:, torch.as_tensor(cols, device="cuda")].contiguous()
        ref = oracle.col_shard(from_gpu(X), from_gpu(Wc), oracle.plain_split(len(cols), 1), 1, 0)
        assert_close(from_gpu(Y)[:, cols], ref, f"col n=2^23 {kern}")
        return
    if case == "col_k_max_nk":
        Y = ttl.shard_linear_col(X, W.t().contiguous(), 1, 0, w_layout=ttl.W_NK)
    else:
        Y = ttl.shard_linear_col(X, W, 1, 0)
    ref = oracle.col_shard(from_gpu(X[rows]), from_gpu(W), oracle.plain_split(n, 1), 1, 0)
    assert_close(from_gpu(Y[rows]), ref, f"{case} {kern}")


def test_empty_batch_is_a_shape_error(ttl):
    """Sizes must be at least 1: a batch of no tokens is TTL_ERR_SHAPE at every entry point, raised
    by the binding before anything is enqueued, and nothing is written."""
    k, I, H, t = 256, 688, 256, 2
    X = gpu(wl.random_bf16((0, k), 1))
    Wgu = gpu(wl.random_bf16((k, 2 * I), 2, std=0.05))
    Wd = gpu(wl.random_bf16((I, H), 3, std=0.05))
    gamma = gpu(wl.random_bf16((H,), 4))
    P = torch.empty((t, 0, H), dtype=torch.bfloat16, device="cuda")
    act = torch.empty((0, I // t), dtype=torch.bfloat16, device="cuda")
    calls = [
        lambda: ttl.shard_linear_col(X, Wgu, t, 1, ttl.merged_gate_up_split(I, t), ttl.EPI_SILU_MUL),
        lambda: ttl.shard_linear_col_gathered(X, Wgu, t, 1, ttl.merged_gate_up_split(I, t), ttl.EPI_SILU_MUL),
        lambda: ttl.shard_linear_row(act, Wd, t, 1, True),
        lambda: ttl.reduce_partials_rmsnorm(P, gamma, 1e-5, None),
        lambda: ttl.reduce_scatter_partials_rmsnorm(P, gamma, 1e-5, 0, None),
    ]
    for call in calls:
        with pytest.raises(ttl.TTLError) as err:
            call()
        assert err.value.status == ttl.ERR_SHAPE, err.value


@LAYOUTS
def test_identity_and_one_hot_are_exact(ttl, gemm_path, layout):
    # W = identity: every column of the output is one column of X, exactly.
    b, k, t = 40, 256, 2
    X = wl.random_bf16((b, k), 70)
    W, lay = _stored(ttl, torch.eye(k, dtype=torch.bfloat16), layout)
    Y0 = ttl.shard_linear_col(gpu(X), W, t, 1, w_layout=lay)
    assert torch.equal(Y0.cpu(), X[:, k // t:])
    # one-hot rows of X: each output row is a row of W, exactly (row split: of the rank's rows).
    n = 264
    Wr = wl.random_bf16((k, n), 71)
    Xo = torch.zeros((b, k), dtype=torch.bfloat16)
    idx = torch.arange(b) * 7 % k
    Xo[torch.arange(b), idx] = 1.0
    Wrd, lay = _stored(ttl, Wr, layout)
    P = ttl.shard_linear_row(gpu(Xo), Wrd, 1, 0, x_is_parallel=True, w_layout=lay)
    assert torch.equal(P.cpu(), Wr[idx])


def test_layouts_agree_bitwise(ttl, gemm_path):
    """Both weight storages feed the matrix cores the same products in the same k order."""
    b, k, I, t = 300, 512, 1024, 4
    X = gpu(wl.random_bf16((b, k), 90))
    W = wl.random_bf16((k, 2 * I), 91, std=0.05)
    sp = ttl.merged_gate_up_split(I, t)
    a = ttl.shard_linear_col(X, gpu(W), t, 2, sp, ttl.EPI_SILU_MUL, w_layout=ttl.W_KN)
    c = ttl.shard_linear_col(X, gpu(W.t().contiguous()), t, 2, sp, ttl.EPI_SILU_MUL, w_layout=ttl.W_NK)
    torch.cuda.synchronize()
    assert torch.equal(a, c)


@pytest.mark.parametrize("k", [64, 128, 192, 320, 576])
@LAYOUTS
def test_tiled_kernels_short_k(ttl, gemm_force, k, layout):
    """The four-wave kernel's 256 x 256 and 256 x 128 tiles over 1, 2, 3, 5 and 9 k-tiles (its
    prologue and the two peeled k-tiles), ragged in M and N, match the oracle and the eight-wave
    kernel bit for bit (all accumulate the same products in the same k order)."""
    gemm_force.set(splits=0)
    b, I, t = 300, 688, 2
    X = wl.random_bf16((b, k), 95 + k)
    W = wl.random_bf16((k, 2 * I), 96 + k, std=0.05)
    Wd_, lay = _stored(ttl, W, layout)
    sp = ttl.merged_gate_up_split(I, t)
    outs = {}
    for kern in ("tiled", "eightwave", "narrow"):
        gemm_force.set(kernel=kern)
        outs[kern] = ttl.shard_linear_col(gpu(X), Wd_, t, 1, sp, ttl.EPI_SILU_MUL, w_layout=lay)
        torch.cuda.synchronize()
    ref = oracle.silu_mul(oracle.col_shard(f64(X), f64(W), oracle.merged_gate_up_split(I, t), t, 1))
    assert_close(from_gpu(outs["tiled"]), ref, f"four-wave k={k} {layout}")
    assert torch.equal(outs["tiled"], outs["eightwave"])
    assert torch.equal(outs["tiled"], outs["narrow"])


@pytest.mark.parametrize("splits", [2, 3, 7])
@pytest.mark.parametrize("silu", [False, True])
@pytest.mark.parametrize("kern", ["tilesplit", "narrowsplit"])
@LAYOUTS
def test_tiles_cut_along_k(ttl, gemm_force, splits, silu, kern, layout):
    """256 x 256 (and 256 x 128) tiles of the four-wave kernel cut into k ranges (10 k-tiles of 64:
    ranges of 5+5, 4+4+2 and 2+2+2+2+2), ragged in M and N, against the oracle; SiLU·up runs as the
    gate columns then the up columns and is paired by the finalize kernel."""
    gemm_force.set(kernel=kern)
    gemm_force.set(splits=splits)
    b, k, t = 600, 640, 2
    X = wl.random_bf16((b, k), 99 + splits)
    if silu:
        I = 1040
        W = wl.random_bf16((k, 2 * I), 100 + splits, std=0.05)
        sp_c, sp_np, epi = ttl.merged_gate_up_split(I, t), oracle.merged_gate_up_split(I, t), ttl.EPI_SILU_MUL
    else:
        W = wl.random_bf16((k, 1072), 100 + splits, std=0.05)
        sp_c, sp_np, epi = None, oracle.plain_split(1072, t), 0
    Wd_, lay = _stored(ttl, W, layout)
    for r in range(t):
        Y = ttl.shard_linear_col(gpu(X), Wd_, t, r, sp_c, epi, w_layout=lay)
        ref = oracle.col_shard(f64(X), f64(W), sp_np, t, r)
        if silu:
            ref = oracle.silu_mul(ref)
        assert_close(from_gpu(Y), ref, f"tiles cut along k: splits={splits} silu={silu} r={r} {layout}")


@pytest.mark.parametrize("silu", [False, True])
@LAYOUTS
def test_short_last_round_split_by_rows(ttl, gemm_force, silu, layout):
    """2176 x 8192 outputs are 288 tiles of 256 x 256: one whole round on 256 CUs plus 32 tiles.
    By default the first 2048 rows run as tiles and the last 128 rows through the split-K kernel;
    sampled rows on both sides of the cut match the oracle, and the head rows match the forced
    tiled run bit for bit."""
    gemm_force.set(splits=0)
    b, k = 2176, 256
    n = 8192
    X = wl.random_bf16((b, k), 97)
    if silu:
        W = wl.random_bf16((k, 2 * n), 98, std=0.05)
        sp_c, sp_np, epi = ttl.merged_gate_up_split(n, 1), oracle.merged_gate_up_split(n, 1), ttl.EPI_SILU_MUL
    else:
        W = wl.random_bf16((k, n), 98, std=0.05)
        sp_c, sp_np, epi = None, oracle.plain_split(n, 1), 0
    Wd_, lay = _stored(ttl, W, layout)
    outs = {}
    for kern in ("auto", "tiled"):
        if kern == "auto":
            gemm_force.set(kernel="auto")
        else:
            gemm_force.set(kernel=kern)
        outs[kern] = ttl.shard_linear_col(gpu(X), Wd_, 1, 0, sp_c, epi, w_layout=lay)
        torch.cuda.synchronize()
    rows = np.r_[0:8, 2040:2056, 2100:2108, 2168:2176]
    ref = oracle.col_shard(f64(X)[rows], f64(W), sp_np, 1, 0)
    if silu:
        ref = oracle.silu_mul(ref)
    assert_close(from_gpu(outs["auto"])[rows], ref, f"row-cut rows silu={silu} {layout}")
    assert torch.equal(outs["auto"][:2048], outs["tiled"][:2048])


@pytest.mark.parametrize("case", ["narrow", "narrowsplit"])
def test_auto_choice_of_narrow_tiles(ttl, gemm_force, case):
    """Shapes whose 256 x 256 tiles fill too few CUs: 512 x 12288 outputs (96 wide tiles, 192
    narrow ones: narrow tiles, whole k) and 512 x 6144 outputs at k = 4096 (48 wide tiles x 4
    splits against 96 narrow tiles x 2 splits: narrow tile splits).  The shape-based choice matches
    the forced kernel bit for bit and sampled rows match the oracle."""
    gemm_force.set(splits=0)
    b, k, n = (512, 256, 12288) if case == "narrow" else (512, 4096, 6144)
    X = wl.random_bf16((b, k), 310)
    W = wl.random_bf16((k, n), 311, std=0.05)
    outs = {}
    for kern in ("auto", case):
        if kern == "auto":
            gemm_force.set(kernel="auto")
        else:
            gemm_force.set(kernel=kern)
            if kern == "narrowsplit":
                gemm_force.set(splits=2)
        outs[kern] = ttl.shard_linear_col(gpu(X), gpu(W), 1, 0)
        torch.cuda.synchronize()
    assert torch.equal(outs["auto"], outs[case])
    rows = np.r_[0:4, 254:258, 508:512]
    ref = oracle.col_shard(f64(X)[rows], f64(W), oracle.plain_split(n, 1), 1, 0)
    assert_close(from_gpu(outs["auto"])[rows], ref, f"auto {case}")


def _stored3(ttl, W, layout):
    """_stored, plus the blocked storage (packed on the device)."""
    if layout == "blk":
        return ttl.pack_weight_blocked(gpu(W)), ttl.W_BLOCKED
    return _stored(ttl, W, layout)


# (b, k, n, silu, cus): the cut the planner makes for `cus` compute units, in 256-column strips
# (128 act columns with SiLU·up):
MIXED_CASES = [
    # 7 SiLU·up strips: strips [0, 3) take 4 x 256 rows (the last ragged), [3, 7) 1 x 256 + 4 x 192
    # rows (the last ragged); 4 k-tiles
    (1000, 256, 896, True, 16),
    # 7 plain strips, the last one 128 columns wide; one k-tile
    (1000, 64, 1664, False, 16),
    # 28 plain strips: [0, 26) 9 x 256 rows (the last ragged), [26, 28) 3 x 256 + 8 x 192; 3 k-tiles
    (2176, 192, 7168, False, 16),
    # 7 SiLU·up strips, the last one 72 act columns wide (its gate and up columns ragged); 2 k-tiles
    (1000, 128, 840, True, 16),
]


@pytest.mark.parametrize("b,k,n,silu,cus", MIXED_CASES)
@pytest.mark.parametrize("layout", ["kn", "nk", "blk"])
def test_mixed_row_cut(ttl, gemm_force, capfd, b, k, n, silu, cus, layout):
    """A launch cut per column strip into 256-row tiles (whole rounds) and 192-row tiles below
    them (one more round), planned for a small CU count so that small shapes take the cut: the
    cut runs (the planner's trace line), its result equals the 256 x 256 tiles' and the 192 x 256
    tiles' bit for bit (same products, same k order), and every element matches the oracle."""
    gemm_force.set(splits=0)
    gemm_force.set(trace=True)
    gemm_force.set(plan_cus=cus)
    X = wl.random_bf16((b, k), 400 + b + k)
    if silu:
        W = wl.random_bf16((k, 2 * n), 401 + k, std=0.05)
        sp_c, sp_np, epi = ttl.merged_gate_up_split(n, 1), oracle.merged_gate_up_split(n, 1), ttl.EPI_SILU_MUL
    else:
        W = wl.random_bf16((k, n), 401 + k, std=0.05)
        sp_c, sp_np, epi = None, oracle.plain_split(n, 1), 0
    if layout == "blk" and W.shape[1] % 128 != 0:
        pytest.skip("blocked storage needs a weight whose column count is a multiple of 128")
    Wd_, lay = _stored3(ttl, W, layout)
    capfd.readouterr()
    outs = {}
    for kern in ("mixed", "tiled", "short"):
        gemm_force.set(kernel=kern)
        outs[kern] = ttl.shard_linear_col(gpu(X), Wd_, 1, 0, sp_c, epi, w_layout=lay)
        torch.cuda.synchronize()
    err = capfd.readouterr().err
    assert err.count("ttl gemm cut") == 1, err
    assert torch.equal(outs["mixed"], outs["tiled"])
    assert torch.equal(outs["short"], outs["tiled"])
    ref = oracle.col_shard(f64(X), f64(W), sp_np, 1, 0)
    if silu:
        ref = oracle.silu_mul(ref)
    assert_close(from_gpu(outs["mixed"]), ref, f"mixed cut b={b} k={k} n={n} silu={silu} {layout}")


# (b, k, n, t, x_is_parallel): row GEMMs with rows past the whole 256-row tiles, at most 16 per
# row-tile, appended to the tiles
APPENDED_ROW_CASES = [
    (528, 128, 512, 1, True),     # 2 row-tiles, 16 appended rows (row-tile 0's)
    (808, 640, 1152, 2, True),    # 3 row-tiles, 40 rows (16, 16, 8); ragged columns; 5 k-tiles
    (1044, 64, 768, 1, True),     # one k-tile; 20 rows (16, 4, none, none)
    (513, 384, 256, 2, False),    # one appended row; X not parallel (the rank's k slice of it)
]


@pytest.mark.parametrize("layout", ["kn", "nk", "blk"])
@pytest.mark.parametrize("b,k,n,t,x_is_parallel", APPENDED_ROW_CASES)
def test_appended_rows(ttl, gemm_force, capfd, b, k, n, t, x_is_parallel, layout):
    """The rows below the whole 256-row tiles appended to the tiles of the 16 x 16 x 32 kernel (16
    per row-tile, the last ones partly or wholly past M; one launch): each rank bit-equal to whole
    256 x 256 tiles of the same kernel (the same products in the same k order) and every element
    against the oracle, for every weight storage."""
    gemm_force.set(trace=True)
    w = k // t
    X = wl.random_bf16((b, k), 50 + b)
    W = wl.random_bf16((k, n), 51 + b, std=0.05)
    Xd = gpu(X)
    Wd, lay = _stored3(ttl, W, layout)
    Xo, Wo = f64(X), f64(W)
    capfd.readouterr()
    for r in range(t):
        xin = Xd[:, r * w:(r + 1) * w].contiguous() if x_is_parallel else Xd
        gemm_force.set(kernel="appended")
        P = ttl.shard_linear_row(xin, Wd, t, r, x_is_parallel, w_layout=lay)
        torch.cuda.synchronize()
        err = capfd.readouterr().err
        assert err.count("ttl gemm appended rows") == 1, err
        gemm_force.set(kernel="tiled16")
        Q = ttl.shard_linear_row(xin, Wd, t, r, x_is_parallel, w_layout=lay)
        torch.cuda.synchronize()
        assert torch.equal(P, Q), f"appended rows differ from whole tiles (rank {r})"
        ref = oracle.row_shard(Xo, Wo, t, r, x_is_parallel=False)
        assert_close(from_gpu(P), ref, f"appended rows b={b} k={k} n={n} t={t} r={r} {layout}")


@pytest.mark.parametrize("layout", ["kn", "nk"])
def test_appended_rows_qkv(ttl, gemm_force, capfd, layout):
    """Appended rows on a column GEMM through the three head-sliced segments (q, k, v) of a qkv
    weight: bit-equal to whole tiles, every element against the oracle."""
    gemm_force.set(trace=True)
    b, k, nq, nkv, hd, t = 530, 256, 32, 8, 64, 2
    X = wl.random_bf16((b, k), 60)
    sp_np, sp_c = oracle.qkv_split(nq, nkv, hd, t), ttl.qkv_split(nq, nkv, hd, t)
    W = wl.random_bf16((k, sum(sp_np[0])), 61, std=0.05)
    Wd, lay = _stored(ttl, W, layout)
    capfd.readouterr()
    for r in range(t):
        gemm_force.set(kernel="appended")
        Y = ttl.shard_linear_col(gpu(X), Wd, t, r, sp_c, 0, w_layout=lay)
        torch.cuda.synchronize()
        assert capfd.readouterr().err.count("ttl gemm appended rows") == 1
        gemm_force.set(kernel="tiled16")
        Z = ttl.shard_linear_col(gpu(X), Wd, t, r, sp_c, 0, w_layout=lay)
        torch.cuda.synchronize()
        assert torch.equal(Y, Z), f"appended rows differ from whole tiles (rank {r})"
        assert_close(from_gpu(Y), oracle.col_shard(f64(X), f64(W), sp_np, t, r), f"appended qkv r={r} {layout}")


@pytest.mark.parametrize("layout", ["kn", "nk", "blk"])
@pytest.mark.parametrize("silu", [False, True])
def test_auto_mixed_row_cut(ttl, gemm_force, capfd, silu, layout):
    """At 256 CUs the shape-based choice cuts 2500 x 10240 outputs (400 tiles of 256 x 256: one
    round plus 144 tiles) and 4096 x 3584 SiLU·up outputs (448 tiles: one round plus 192) into
    256-row and 192-row tiles of the 16 x 16 x 32 kernel, for every weight storage: bit-equal to the
    whole 256 x 256 tiles of either kernel; sampled rows (both sides of every strip class's cut row)
    against the oracle.  The row GEMM of 4096 x 8192 (512 tiles, two whole rounds) is not cut."""
    gemm_force.set(splits=0)
    gemm_force.set(plan_cus=0)
    gemm_force.set(trace=True)
    k = 128
    if silu:
        b, n = 4096, 3584
        W = wl.random_bf16((k, 2 * n), 411, std=0.05)
        sp_c, sp_np, epi = ttl.merged_gate_up_split(n, 1), oracle.merged_gate_up_split(n, 1), ttl.EPI_SILU_MUL
        rows = np.r_[0:2, 1022:1026, 1214:1218, 2558:2562, 2750:2754, 4094:4096]
    else:
        b, n = 2500, 10240
        W = wl.random_bf16((k, n), 411, std=0.05)
        sp_c, sp_np, epi = None, oracle.plain_split(n, 1), 0
        rows = np.r_[0:2, 254:258, 446:450, 1790:1794, 1982:1986, 2496:2500]
    Wd_, lay = _stored3(ttl, W, layout)
    X = wl.random_bf16((b, k), 410)
    capfd.readouterr()
    outs = {}
    for kern in ("auto", "tiled", "tiled16"):
        gemm_force.set(kernel=kern)
        outs[kern] = ttl.shard_linear_col(gpu(X), Wd_, 1, 0, sp_c, epi, w_layout=lay)
        torch.cuda.synchronize()
        if kern == "auto":
            assert capfd.readouterr().err.count("ttl gemm cut") == 1
    assert torch.equal(outs["auto"], outs["tiled"])
    assert torch.equal(outs["auto"], outs["tiled16"])
    ref = oracle.col_shard(f64(X)[rows], f64(W), sp_np, 1, 0)
    if silu:
        ref = oracle.silu_mul(ref)
    assert_close(from_gpu(outs["auto"])[rows], ref, f"auto cut silu={silu} {layout}")
    # two whole rounds: no cut
    gemm_force.set(kernel="auto")
    capfd.readouterr()
    Xr = gpu(wl.random_bf16((4096, 256), 412))
    ttl.shard_linear_row(Xr, gpu(wl.random_bf16((256, 8192), 413, std=0.05)), 1, 0, True)
    torch.cuda.synchronize()
    assert "ttl gemm cut" not in capfd.readouterr().err


def _blocked_reference(W):
    """The TTL_W_BLOCKED memory order of a [k, n] weight, by index arithmetic on the host."""
    k, n = W.shape
    return W.reshape(k // 64, 64, n // 128, 128).permute(2, 0, 1, 3).reshape(k, n).contiguous()


def test_pack_weight_blocked(ttl):
    W = wl.random_bf16((192, 384), 130)
    got = ttl.pack_weight_blocked(gpu(W))
    assert torch.equal(got.cpu(), _blocked_reference(W))


@pytest.mark.parametrize("b", [5, 300])
def test_blocked_weights_match_kn_bitwise(ttl, gemm_path, b):
    """Weights stored in 64 x 128 blocks give bit-identical results to [k][n] storage through every
    kernel (only the addresses differ), for SiLU·up, qkv and gathered column calls and the row
    call; one of each is also checked against the oracle."""
    k, I, t = 512, 1024, 4
    X = gpu(wl.random_bf16((b, k), 131))
    Wgu = wl.random_bf16((k, 2 * I), 132, std=0.05)
    sp = ttl.merged_gate_up_split(I, t)
    Wgu_kn, Wgu_blk = gpu(Wgu), ttl.pack_weight_blocked(gpu(Wgu))
    for r in (0, t - 1):
        a = ttl.shard_linear_col(X, Wgu_kn, t, r, sp, ttl.EPI_SILU_MUL, w_layout=ttl.W_KN)
        c = ttl.shard_linear_col(X, Wgu_blk, t, r, sp, ttl.EPI_SILU_MUL, w_layout=ttl.W_BLOCKED)
        torch.cuda.synchronize()
        assert torch.equal(a, c), f"SiLU·up rank {r}"
    ref = oracle.silu_mul(oracle.col_shard(f64(X.cpu()), f64(Wgu), oracle.merged_gate_up_split(I, t), t, t - 1))
    assert_close(from_gpu(c), ref, f"blocked SiLU·up b={b}")
    # qkv: 8 q heads, 4 kv heads of 64 (n = 1024)
    Wqkv = wl.random_bf16((k, 1024), 133, std=0.05)
    spq = ttl.qkv_split(8, 4, 64, t)
    a = ttl.shard_linear_col(X, gpu(Wqkv), t, 1, spq, w_layout=ttl.W_KN)
    c = ttl.shard_linear_col(X, ttl.pack_weight_blocked(gpu(Wqkv)), t, 1, spq, w_layout=ttl.W_BLOCKED)
    g = torch.full((b, t * 256), float("nan"), dtype=torch.bfloat16, device="cuda")
    ttl.shard_linear_col_gathered(X, ttl.pack_weight_blocked(gpu(Wqkv)), t, 1, spq, Y_all=g,
                                  w_layout=ttl.W_BLOCKED)
    torch.cuda.synchronize()
    assert torch.equal(a, c) and torch.equal(g[:, 256:512], a), "qkv"
    # row: k = 1024, rank rows of 256
    Wd = wl.random_bf16((1024, 768), 134, std=0.05)
    Xr = gpu(wl.random_bf16((b, 1024), 135))
    for r in range(t):
        a = ttl.shard_linear_row(Xr, gpu(Wd), t, r, False, w_layout=ttl.W_KN)
        c = ttl.shard_linear_row(Xr, ttl.pack_weight_blocked(gpu(Wd)), t, r, False, w_layout=ttl.W_BLOCKED)
        torch.cuda.synchronize()
        assert torch.equal(a, c), f"row rank {r}"
    assert_close(from_gpu(c), oracle.row_shard(f64(Xr.cpu()), f64(Wd), t, t - 1, x_is_parallel=False),
                 f"blocked row b={b}")


def test_bitwise_deterministic(ttl, gemm_path):
    b, k, I, t = 300, 512, 1024, 2
    X, Wgu = gpu(wl.random_bf16((b, k), 80)), gpu(wl.random_bf16((k, 2 * I), 81, std=0.05))
    Wd = gpu(wl.random_bf16((I, k), 82, std=0.05))
    sp = ttl.merged_gate_up_split(I, t)
    outs = []
    for _ in range(2):
        act = ttl.shard_linear_col(X, Wgu, t, 1, sp, ttl.EPI_SILU_MUL)
        P = torch.stack([ttl.shard_linear_row(act, Wd, t, 1) for _ in range(2)])
        r, y = ttl.reduce_partials_rmsnorm(P, gpu(torch.ones(k, dtype=torch.bfloat16)), 1e-5)
        torch.cuda.synchronize()
        outs.append((act.cpu(), P.cpu(), r.cpu(), y.cpu()))
    for a, c in zip(*outs):
        assert torch.equal(a, c)


@pytest.mark.parametrize("splits", [1, 2, 3, 7, 65])
@LAYOUTS
def test_splitk_split_counts(ttl, gemm_force, splits, layout):
    """Split-K with a given number of k ranges, k tail of 8 (4104 = 64 * 64 + 8), ragged M and N.

    65 splits puts one k-tile in each range, the last one holding only the 8-wide tail."""
    gemm_force.set(kernel="splitk")
    gemm_force.set(splits=splits)
    b, k = 37, 4104
    _col_case(ttl, b, k, oracle.merged_gate_up_split(200, 1), ttl.merged_gate_up_split(200, 1), 1,
              seed=100 + splits, epi=ttl.EPI_SILU_MUL, layout=layout)
    _col_case(ttl, 3, k, oracle.qkv_split(8, 2, 32, 2), ttl.qkv_split(8, 2, 32, 2), 2, seed=110 + splits,
              layout=layout)
    n, t = 392, 2
    X = wl.random_bf16((b, 2 * k), 120 + splits)
    W = wl.random_bf16((2 * k, n), 121 + splits, std=0.05)
    Wd, lay = _stored(ttl, W, layout)
    for r in range(t):
        P = ttl.shard_linear_row(gpu(X), Wd, t, r, x_is_parallel=False, w_layout=lay)
        assert_close(from_gpu(P), oracle.row_shard(f64(X), f64(W), t, r, x_is_parallel=False),
                     f"split-K row splits={splits} r={r} {layout}")


@pytest.mark.parametrize("b", [65, 200, 256, 400])
@pytest.mark.parametrize("splits", [0, 1, 3])
@LAYOUTS
def test_splitk_short_k_small_row_tiles(ttl, gemm_force, b, splits, layout):
    """With a short k (at most 2048) the split-K kernel runs 65..512-row batches in 32-row tiles
    (64-row above 256 rows): SiLU·up column and row GEMMs with a k tail, at the planned split count
    (0) and forced ones, against the oracle."""
    gemm_force.set(kernel="splitk")
    gemm_force.set(splits=splits)
    _col_case(ttl, b, 1032, oracle.merged_gate_up_split(272, 2), ttl.merged_gate_up_split(272, 2), 2,
              seed=130 + b + splits, epi=ttl.EPI_SILU_MUL, layout=layout)
    k, n, t = 2048, 520, 2
    X = wl.random_bf16((b, k), 140 + b + splits)
    W = wl.random_bf16((k, n), 141 + b + splits, std=0.05)
    Wd, lay = _stored(ttl, W, layout)
    for r in range(t):
        P = ttl.shard_linear_row(gpu(X), Wd, t, r, x_is_parallel=False, w_layout=lay)
        assert_close(from_gpu(P), oracle.row_shard(f64(X), f64(W), t, r, x_is_parallel=False),
                     f"short-k split-K row b={b} splits={splits} r={r} {layout}")


def test_splitk_repeated_launches_reuse_workspace(ttl, gemm_force):
    """Back-to-back split-K launches of different sizes share (and grow) the library's workspace;
    a repeated shape must reproduce its first result bit for bit."""
    gemm_force.set(kernel="splitk")
    gemm_force.set(splits=0)
    shapes = [(64, 8192, 1024), (1, 4096, 3584), (64, 8192, 1024), (200, 2048, 4096), (1, 4096, 3584)]
    outs = {}
    for i, (b, k, n) in enumerate(shapes):
        X = gpu(wl.random_bf16((b, k), 130 + b))
        W = gpu(wl.random_bf16((k, n), 131 + n, std=0.05))
        Y = ttl.shard_linear_col(X, W, 1, 0)
        key = (b, k, n)
        if key in outs:
            assert torch.equal(Y, outs[key]), f"launch {i} {key} differs from its first run"
        else:
            outs[key] = Y
            Xs, Ws = X.cpu(), W.cpu()
            rows = [0, b - 1]
            ref = oracle.col_shard(f64(Xs[rows]), f64(Ws), oracle.plain_split(n, 1), 1, 0)
            assert_close(from_gpu(Y[rows]), ref, f"repeated split-K {key}")


@pytest.mark.parametrize("layout", ["kn", "nk", "blk"])
@pytest.mark.parametrize("silu", [False, True])
def test_auto_narrow_splits(ttl, gemm_force, layout, silu):
    """One row-tile of 200 rows with k = 4096 (64 k-tiles): the shape-based choice cuts 256 x 128
    tiles of the 16 x 16 x 32 kernel into 8 k splits (8 k-tiles each).  Bit-equal to the forced launch
    of that plan, and every element against the oracle."""
    b, k = 200, 4096
    I = 896 if silu else 1792  # 14 tiles of 128 weight columns
    n = 2 * I if silu else I
    X = wl.random_bf16((b, k), 70 + int(silu))
    W = wl.random_bf16((k, n), 72 + int(silu), std=0.02)
    Wd_, lay = _stored3(ttl, W, layout)
    sp_c = ttl.merged_gate_up_split(I, 1) if silu else None
    sp_np = oracle.merged_gate_up_split(I, 1) if silu else oracle.plain_split(I, 1)
    epi = ttl.EPI_SILU_MUL if silu else 0
    Xd = gpu(X)
    gemm_force.set(kernel="auto", splits=0)
    auto = ttl.shard_linear_col(Xd, Wd_, 1, 0, sp_c, epi, w_layout=lay)
    gemm_force.set(kernel="narrowsplit", splits=8)
    forced = ttl.shard_linear_col(Xd, Wd_, 1, 0, sp_c, epi, w_layout=lay)
    torch.cuda.synchronize()
    assert torch.equal(auto, forced)
    ref = oracle.col_shard(f64(X), f64(W), sp_np, 1, 0)
    if silu:
        ref = oracle.silu_mul(ref)
    assert_close(from_gpu(auto), ref, f"auto narrow splits silu={silu} {layout}")


@pytest.mark.parametrize("layout", ["kn", "nk", "blk"])
@pytest.mark.parametrize("b,k,I,t,silu", [
    (300, 256, 344, 1, True),     # ragged rows and act columns, four k-tiles
    (513, 640, 1024, 2, False),   # ten k-tiles, three row-tiles
    (257, 128, 1152, 1, False),   # ragged rows, 9 narrow column tiles (4.5 wide ones)
    (64, 64, 256, 1, True),       # one k-tile
    (700, 192, 768, 2, True)])    # three k-tiles
def test_narrow_tiles_16x16(ttl, gemm_force, b, k, I, t, silu, layout):
    """256 x 128 tiles of 16 x 16 x 32 products (whole, and cut along k): bit-equal to 256 x 256
    tiles of the same kernel (whole) and to 256 x 256 tiles cut into the same k splits (each output
    sums the same products in the same k order; the splits cover the same k ranges and are summed in
    the same order), for every weight storage, and every element against the oracle."""
    if layout == "blk" and (2 * I if silu else I) % 128:
        pytest.skip("blocked storage needs a weight whose column count is a multiple of 128")
    X = wl.random_bf16((b, k), 17 + b)
    n = 2 * I if silu else I
    W = wl.random_bf16((k, n), 18 + k, std=0.05)
    Wd_, lay = _stored3(ttl, W, layout)
    sp_c = ttl.merged_gate_up_split(I, t) if silu else None
    sp_np = oracle.merged_gate_up_split(I, t) if silu else oracle.plain_split(I, t)
    epi = ttl.EPI_SILU_MUL if silu else 0
    Xd = gpu(X)
    for r in range(t):
        out = {}
        for kern, splits in (("narrow", 0), ("tiled16", 0), ("narrowsplit", 2), ("tilesplit", 2)):
            gemm_force.set(kernel=kern, splits=splits)
            out[kern] = ttl.shard_linear_col(Xd, Wd_, t, r, sp_c, epi, w_layout=lay)
        torch.cuda.synchronize()
        assert torch.equal(out["narrow"], out["tiled16"]), f"narrow tiles differ from 256 x 256 tiles (rank {r})"
        assert torch.equal(out["narrowsplit"], out["tilesplit"]), f"narrow k splits differ from 256 x 256 ones (rank {r})"
        ref = oracle.col_shard(f64(X), f64(W), sp_np, t, r)
        if silu:
            ref = oracle.silu_mul(ref)
        for kern in ("narrow", "narrowsplit"):
            assert_close(from_gpu(out[kern]), ref, f"{kern} b={b} k={k} I={I} t={t} r={r} silu={silu} {layout}")


@pytest.mark.parametrize("b,k,n,t,kind", [
    (1, 2048, 1024, 2, "silu"),     # one token row; the shortest k the kernel takes (16 k32 steps per wave)
    (17, 2080, 624, 2, "silu"),     # ragged rows, 312 act columns (19.5 workgroups); 65 k32 steps, uneven quarters
    (64, 4096, 1056, 4, "plain"),   # 64 rows (four row blocks); 264 columns, 8 in the last workgroup
    (33, 2048, 0, 2, "qkv"),        # three column segments (8 q + 2 kv heads of 32, t = 2)
    (64, 8192, 520, 4, "row"),      # row-parallel, X the rank's own k slice
    (40, 8192, 520, 4, "row_full"),  # row-parallel, X full width (the rank's slice read in place)
])
def test_stream_nk_split_free(ttl, gemm_force, b, k, n, t, kind):
    """The split-free kernel for [n][k] weights and up to 64 token rows (forced): every element of
    every rank against the oracle, and a second launch bit-equal to the first (its four waves' sums
    are added in a fixed order)."""
    X = wl.random_bf16((b, k), 500 + b)
    if kind == "qkv":
        sp_np, sp_c = oracle.qkv_split(8, 2, 32, t), ttl.qkv_split(8, 2, 32, t)
        n = sum(sp_np[0])
    elif kind == "silu":
        sp_np, sp_c = oracle.merged_gate_up_split(n, t), ttl.merged_gate_up_split(n, t)
        n = 2 * n
    else:
        sp_np, sp_c = oracle.plain_split(n, t), None
    W = wl.random_bf16((k, n), 501 + b, std=0.05)
    Xd, Wd = gpu(X), gpu(W.t().contiguous())
    Xo, Wo = f64(X), f64(W)
    gemm_force.set(kernel="streamnk", splits=0)
    for r in range(t):
        if kind.startswith("row"):
            w = k // t
            xin = Xd[:, r * w:(r + 1) * w].contiguous() if kind == "row" else Xd
            run = lambda: ttl.shard_linear_row(xin, Wd, t, r, kind == "row", w_layout=ttl.W_NK)
            ref = oracle.row_shard(Xo, Wo, t, r, x_is_parallel=False)
        else:
            epi = ttl.EPI_SILU_MUL if kind == "silu" else 0
            run = lambda: ttl.shard_linear_col(Xd, Wd, t, r, sp_c, epi, w_layout=ttl.W_NK)
            ref = oracle.col_shard(Xo, Wo, sp_np, t, r)
            if kind == "silu":
                ref = oracle.silu_mul(ref)
        first, second = run(), run()
        torch.cuda.synchronize()
        assert torch.equal(first, second), f"split-free kernel not reproducible (rank {r})"
        assert_close(from_gpu(first), ref, f"split-free [n][k] {kind} b={b} k={k} n={n} t={t} r={r}")


@pytest.mark.parametrize("silu", [False, True])
def test_auto_choice_of_stream_nk(ttl, gemm_force, silu):
    """Where its workgroups fill at least 3/4 of the CUs (6144 plain columns: 192 workgroups of 32;
    3072 act columns: 192 of 16), the shape-based choice for [n][k] weights and 8 rows is the
    split-free kernel (chosen by shape up to 16 rows): bit-equal to the forced launch, and every
    element against the oracle."""
    b, k = 8, 2048
    n_out = 3072 if silu else 6144
    n = 2 * n_out if silu else n_out
    X = wl.random_bf16((b, k), 520 + int(silu))
    W = wl.random_bf16((k, n), 521 + int(silu), std=0.05)
    Xd, Wd = gpu(X), gpu(W.t().contiguous())
    sp_c = ttl.merged_gate_up_split(n_out, 1) if silu else None
    sp_np = oracle.merged_gate_up_split(n_out, 1) if silu else oracle.plain_split(n, 1)
    epi = ttl.EPI_SILU_MUL if silu else 0
    gemm_force.set(kernel="auto", splits=0)
    auto = ttl.shard_linear_col(Xd, Wd, 1, 0, sp_c, epi, w_layout=ttl.W_NK)
    gemm_force.set(kernel="streamnk", splits=0)
    forced = ttl.shard_linear_col(Xd, Wd, 1, 0, sp_c, epi, w_layout=ttl.W_NK)
    torch.cuda.synchronize()
    assert torch.equal(auto, forced)
    ref = oracle.col_shard(f64(X), f64(W), sp_np, 1, 0)
    if silu:
        ref = oracle.silu_mul(ref)
    assert_close(from_gpu(auto), ref, f"auto split-free silu={silu}")


@pytest.mark.parametrize("b,k,I,t,silu", [
    (300, 256, 344, 1, True),     # ragged rows and act columns, four k-tiles
    (513, 1024, 2048, 4, True),   # several tiles per rank
    (257, 512, 1000, 1, False),   # ragged columns
    (1000, 640, 1536, 2, False),  # ten k-tiles
    (64, 64, 128, 1, False),      # one k-tile
    (600, 128, 2000, 1, False),   # two k-tiles
    (700, 192, 768, 2, True)])    # three k-tiles
def test_mfma16_tiles_equal_mfma32_tiles(ttl, gemm_force, b, k, I, t, silu):
    """[n][k] weights through 256 x 256 tiles of 16 x 16 x 32 products: every output equals the
    32 x 32 x 16 kernel's bit for bit (each output sums the same products in the same k order), and
    against the oracle."""
    X = wl.random_bf16((b, k), 7 + b)
    n = 2 * I if silu else I
    W = wl.random_bf16((k, n), 8 + k, std=0.05)
    Wd_, lay = _stored(ttl, W, "nk")
    sp_c = ttl.merged_gate_up_split(I, t) if silu else None
    sp_np = oracle.merged_gate_up_split(I, t) if silu else oracle.plain_split(I, t)
    epi = ttl.EPI_SILU_MUL if silu else 0
    Xd = gpu(X)
    for r in range(t):
        gemm_force.set(kernel="tiled")
        a = ttl.shard_linear_col(Xd, Wd_, t, r, sp_c, epi, w_layout=lay)
        gemm_force.set(kernel="tiled16")
        c = ttl.shard_linear_col(Xd, Wd_, t, r, sp_c, epi, w_layout=lay)
        torch.cuda.synchronize()
        assert torch.equal(a, c), f"16 x 16 x 32 tiles differ from 32 x 32 x 16 tiles (rank {r})"
    ref = oracle.col_shard(f64(X), f64(W), sp_np, t, t - 1)
    if silu:
        ref = oracle.silu_mul(ref)
    assert_close(from_gpu(c), ref, f"16x16x32 tiles b={b} k={k} I={I} t={t} silu={silu}")


@pytest.mark.parametrize("b,k,I,t,silu,cus", [
    (300, 256, 344, 1, True, 3),      # 6 tiles on 3 workgroups, two each
    (513, 192, 1024, 2, True, 6),     # three k-tiles (an odd count: the stages swap between tiles)
    (1000, 640, 1536, 1, False, 16),  # 24 tiles on 16 workgroups: 8 of them take a second tile
    (600, 128, 2000, 1, False, 12),   # two k-tiles, both fetched for the next tile
    (1024, 1024, 2048, 4, True, 10),  # 16 tiles per rank on 10 workgroups
    (700, 320, 768, 2, False, 3)])
@LAYOUTS
def test_persistent_tiles(ttl, gemm_force, capfd, b, k, I, t, silu, cus, layout):
    """256 x 256 tiles by a persistent grid (planned for a few CUs so that small shapes have more
    tiles than workgroups): a workgroup computes its first tile while fetching the first k-tiles of
    its second.  Bit for bit the whole-tile launch's results (same products, same k order), and
    every element against the oracle."""
    X = wl.random_bf16((b, k), 7 + b)
    n = 2 * I if silu else I
    W = wl.random_bf16((k, n), 8 + k, std=0.05)
    Wd_, lay = _stored(ttl, W, layout)
    sp_c = ttl.merged_gate_up_split(I, t) if silu else None
    sp_np = oracle.merged_gate_up_split(I, t) if silu else oracle.plain_split(I, t)
    epi = ttl.EPI_SILU_MUL if silu else 0
    Xd = gpu(X)
    capfd.readouterr()
    for r in range(t):
        gemm_force.set(kernel="tiled", plan_cus=0, trace=True)
        whole = ttl.shard_linear_col(Xd, Wd_, t, r, sp_c, epi, w_layout=lay)
        gemm_force.set(kernel="persist", plan_cus=cus)
        got = ttl.shard_linear_col(Xd, Wd_, t, r, sp_c, epi, w_layout=lay)
        torch.cuda.synchronize()
        assert torch.equal(got, whole), f"persistent tiles differ from whole tiles (rank {r})"
    assert capfd.readouterr().err.count(f"on {cus} workgroups") == t  # every rank ran persistent
    ref = oracle.col_shard(f64(X), f64(W), sp_np, t, t - 1)
    if silu:
        ref = oracle.silu_mul(ref)
    assert_close(from_gpu(got), ref, f"persistent tiles b={b} k={k} I={I} t={t} silu={silu} {layout}")


def test_persistent_row_gemm_two_rounds(ttl, gemm_force, capfd):
    """The row GEMM at 4096 x 8192 outputs (512 tiles: two whole rounds on 256 CUs): the planner's
    whole tiles (outputs staged through LDS) and the persistent grid (direct stores while the ring
    holds the next tile) are bit-equal; sampled rows against the oracle."""
    b, k, n, t = 4096, 3584, 8192, 8
    X = wl.random_bf16((b, k // t), 175, device="cuda")
    W = wl.random_bf16((k, n), 176, std=0.02, device="cuda")
    gemm_force.set(kernel="auto", trace=True)
    capfd.readouterr()
    whole = ttl.shard_linear_row(X, W, t, 5, True)
    torch.cuda.synchronize()
    assert "workgroups" not in capfd.readouterr().err  # whole tiles by shape
    gemm_force.set(kernel="persist", trace=True)
    got = ttl.shard_linear_row(X, W, t, 5, True)
    torch.cuda.synchronize()
    assert "512 tiles on 256 workgroups" in capfd.readouterr().err
    assert torch.equal(got, whole)
    rows = [0, 255, 256, 2047, 2048, 4095]
    ref = oracle.row_shard(f64(X[rows].cpu()), f64(W.cpu()), t, 5, x_is_parallel=True)
    assert_close(from_gpu(got[rows]), ref, "persistent row GEMM, two rounds")


@pytest.mark.parametrize("kern", ["splitk", "tilesplit"])
def test_splitk_on_two_streams_at_once(ttl, gemm_force, kern):
    """Split-K launches on two streams at once write their fp32 partials to separate workspaces (one
    per stream): every result equals the same call made alone on one stream, bit for bit.  The two
    shapes need different workspace sizes, and their launches are interleaved across the streams so
    that they overlap on the device."""
    gemm_force.set(kernel=kern, splits=8)
    cases = [((64, 8192), (8192, 2048)), ((128, 4096), (4096, 4096))] if kern == "splitk" else \
            [((512, 4096), (4096, 1024)), ((768, 2048), (2048, 2048))]
    ops = []
    for i, (xs, ws) in enumerate(cases):
        X = gpu(wl.random_bf16(xs, 170 + i))
        W = gpu(wl.random_bf16(ws, 172 + i, std=0.05))
        ops.append((X, W))
    main = torch.cuda.current_stream()
    alone = []
    for X, W in ops:
        alone.append(ttl.shard_linear_col(X, W, 1, 0, stream=main))
        torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for s in streams:
        s.wait_stream(main)
    reps = 6
    outs = [[torch.empty_like(alone[i]) for _ in range(reps)] for i in range(2)]
    for rep in range(reps):
        for i, (X, W) in enumerate(ops):
            ttl.shard_linear_col(X, W, 1, 0, Y=outs[i][rep], stream=streams[i])
    torch.cuda.synchronize()
    for i in range(2):
        for rep in range(reps):
            assert torch.equal(outs[i][rep], alone[i]), f"stream {i} launch {rep} differs from the lone call"
    rows = [0, ops[0][0].shape[0] - 1]
    ref = oracle.col_shard(f64(ops[0][0][rows].cpu()), f64(ops[0][1].cpu()),
                           oracle.plain_split(ops[0][1].shape[1], 1), 1, 0)
    assert_close(from_gpu(alone[0][rows]), ref, f"{kern} two-stream case")


def test_capture_needing_a_new_workspace_is_refused(ttl, gemm_force):
    """A split-K call captured on a stream that has no workspace yet fails with TTL_ERR_HIP before
    anything is enqueued (a buffer cannot be allocated during capture); after one eager call on
    that stream the same capture succeeds and its replay matches the eager result."""
    gemm_force.set(kernel="splitk", splits=4)
    X = gpu(wl.random_bf16((48, 2048), 180))
    W = gpu(wl.random_bf16((2048, 1024), 181, std=0.05))
    Y = torch.empty((48, 1024), dtype=torch.bfloat16, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with pytest.raises(ttl.TTLError) as e:
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                ttl.shard_linear_col(X, W, 1, 0, Y=Y)
    assert e.value.status == ttl.ERR_HIP
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        want = ttl.shard_linear_col(X, W, 1, 0).clone()
    torch.cuda.synchronize()
    g2 = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g2, stream=s):
            ttl.shard_linear_col(X, W, 1, 0, Y=Y)
    for _ in range(2):
        Y.zero_()
        g2.replay()
        torch.cuda.synchronize()
        assert torch.equal(Y, want)


def test_tiny_mlp_chain_all_ranks(ttl):
    """The tiny Llama-style MLP (hidden 256, intermediate 688, t = 2, 16 tokens) end to end."""
    w = wl.TINY_MLP_T2
    b = w.batches[0]
    inp = wl.mlp_inputs(w, b, seed=0)
    d = {k: gpu(v) for k, v in inp.items()}
    o = {k: f64(v) for k, v in inp.items()}
    sp = ttl.merged_gate_up_split(w.intermediate, w.t)
    P = torch.empty((w.t, b, w.hidden), dtype=torch.bfloat16, device="cuda")
    acts = []
    for r in range(w.t):
        act = ttl.shard_linear_col(d["X"], d["Wgu"], w.t, r, sp, ttl.EPI_SILU_MUL)
        ttl.shard_linear_row(act, d["Wd"], w.t, r, True, P=P[r])
        acts.append(act)
    rout, y = ttl.reduce_partials_rmsnorm(P, d["gamma"], w.eps, d["R"])
    ref_acts, ref_P, _, ref_P_stored = oracle.mlp_rank_chain(o["X"], o["Wgu"], o["Wd"], w.t, w.intermediate)
    h, yref = oracle.reduce_partials_rmsnorm(ref_P_stored, o["R"], o["gamma"], w.eps)
    for r in range(w.t):
        assert_close(from_gpu(acts[r]), ref_acts[r], f"tiny act r={r}")
        assert_close(from_gpu(P[r]), ref_P[r], f"tiny partial r={r}")
    assert_close(from_gpu(rout), h, "tiny residual_out", literal=True)
    assert_close(from_gpu(y), yref, "tiny y", literal=True)
    # the unrounded float64 chain (no bf16 storage between steps) is within tolerance too
    _, P64, _, _ = oracle.mlp_rank_chain(o["X"], o["Wgu"], o["Wd"], w.t, w.intermediate, store_bf16=False)
    h64, y64 = oracle.reduce_partials_rmsnorm(P64, o["R"], o["gamma"], w.eps)
    assert_close(from_gpu(y), y64, "tiny y vs unrounded chain")
    # the sum of the rank partials equals the unsharded gated MLP (row-split invariant)
    full = (oracle.silu(o["X"] @ o["Wgu"][:, :w.intermediate]) * (o["X"] @ o["Wgu"][:, w.intermediate:])) @ o["Wd"]
    psum = from_gpu(P).sum(0)
    assert_close(psum, full, "tiny sum of partials vs unsharded MLP")


# ---- gather_output=True and the sequence-parallel reduction ---------------------------------------

@pytest.mark.parametrize("case", ["plain", "silu", "qkv"])
@LAYOUTS
def test_col_gathered(ttl, gemm_path, case, layout):
    """Every simulated rank writes its block of the all-gathered output; together they equal the
    oracle's gathered result (for a plain split: X @ W)."""
    b, k, t = 70, 512, 4
    if case == "plain":
        n, sp_o, sp_c, epi = 1056, oracle.plain_split(1056, t), None, ttl.EPI_NONE
    elif case == "silu":
        I = 688 * 2
        n, sp_o, sp_c, epi = 2 * I, oracle.merged_gate_up_split(I, t), ttl.merged_gate_up_split(I, t), ttl.EPI_SILU_MUL
    else:
        sp_o, sp_c, epi = oracle.qkv_split(16, 2, 32, t), ttl.qkv_split(16, 2, 32, t), ttl.EPI_NONE
        n = sum(sp_o[0])
    X = wl.random_bf16((b, k), 140)
    W = wl.random_bf16((k, n), 141, std=0.05)
    Xd = gpu(X)
    Wd_, lay = _stored(ttl, W, layout)
    width = ttl.split_width(sp_c, n, t) // (2 if epi == ttl.EPI_SILU_MUL else 1)
    # sentinel fill: a rank's call must touch its own block only
    Y = torch.full((b, t * width), float("nan"), dtype=torch.bfloat16, device="cuda")
    for r in range(t):
        ttl.shard_linear_col_gathered(Xd, Wd_, t, r, sp_c, epi, Y_all=Y, w_layout=lay)
        torch.cuda.synchronize()
        done = Y[:, : (r + 1) * width]
        assert not torch.isnan(done).any(), f"rank {r} left part of its block unwritten"
        if r + 1 < t:
            assert torch.isnan(Y[:, (r + 1) * width:]).all(), f"rank {r} wrote outside its block"
        # the gathered block is the plain column output of the same rank, bit for bit
        single = ttl.shard_linear_col(Xd, Wd_, t, r, sp_c, epi, w_layout=lay)
        assert torch.equal(Y[:, r * width:(r + 1) * width], single)
    ref = oracle.col_gathered(f64(X), f64(W), sp_o, t, epi_silu_mul=(epi == ttl.EPI_SILU_MUL))
    assert_close(from_gpu(Y), ref, f"gathered {case} {layout} {gemm_path}")


@pytest.mark.parametrize("t,b,n,with_residual", [(2, 16, 256, True), (4, 2048, 4096, True),
                                                  (8, 64, 8192, True), (8, 8, 1024, False),
                                                  (3, 9, 4104, True)])
def test_reduce_scatter_rmsnorm(ttl, t, b, n, with_residual):
    """Each rank reduces and normalises its b/t rows; the chunks together are the full reduction."""
    P = wl.random_bf16((t, b, n), 150 + n)
    R = wl.random_bf16((b, n), 151 + n) if with_residual else None
    gamma = wl.random_bf16((n,), 152 + n, mean=1.0, std=0.1)
    Pd, gd = gpu(P), gpu(gamma)
    rows = b // t
    Ro = f64(R) if with_residual else None
    for r in range(t):
        Rs = gpu(R[r * rows:(r + 1) * rows].contiguous()) if with_residual else None
        rout, y = ttl.reduce_scatter_partials_rmsnorm(Pd, gd, 1e-5, r, Rs)
        assert rout.shape == (rows, n) and y.shape == (rows, n)
        Rr = Ro[r * rows:(r + 1) * rows] if with_residual else None
        h, yref = oracle.reduce_scatter_partials_rmsnorm(f64(P), Rr, f64(gamma), 1e-5, t, r)
        assert_close(from_gpu(rout), h, f"reduce-scatter residual_out t={t} b={b} n={n} r={r}", literal=True)
        assert_close(from_gpu(y), yref, f"reduce-scatter y t={t} b={b} n={n} r={r}", literal=True)


@pytest.mark.parametrize("t,b,n,with_residual", [(8, 4096, 8192, True), (8, 64, 8192, True),
                                                  (4, 2048, 4096, False), (3, 9, 4104, True),
                                                  (16, 32, 1024, True), (1, 5, 256, True)])
def test_reduce_over_peer_buffers(ttl, t, b, n, with_residual):
    """The partials in t separate buffers (one per rank, as peers' buffers would be mapped): over
    all rows (one-shot) bit-equal to reduce_partials_rmsnorm of the same partials as one [t, b, n]
    slab, over each rank's b/t rows (two-shot) bit-equal to reduce_scatter_partials_rmsnorm (the
    same row count, so the same launch shape and order of the mean square's reduction), and equal
    to the oracle."""
    P = wl.random_bf16((t, b, n), 160 + t, device="cuda")
    peers = [P[r].clone() for r in range(t)]  # separate allocations
    R = wl.random_bf16((b, n), 161, device="cuda") if with_residual else None
    gamma = wl.random_bf16((n,), 162, mean=1.0, std=0.1, device="cuda")
    rout, y = ttl.reduce_partials_rmsnorm_peers(peers, gamma, 1e-5, residual=R)
    rout_s, y_s = ttl.reduce_partials_rmsnorm(P, gamma, 1e-5, R)
    torch.cuda.synchronize()
    assert torch.equal(rout, rout_s) and torch.equal(y, y_s)
    sample = torch.as_tensor(np.unique(np.r_[0:2, b // 2, b - 1]), device="cuda")
    Ro = from_gpu(R[sample]) if with_residual else None
    h, yref = oracle.reduce_partials_rmsnorm(from_gpu(P[:, sample]), Ro, from_gpu(gamma), 1e-5)
    assert_close(from_gpu(rout[sample]), h, f"peers residual_out t={t} b={b} n={n}", literal=True)
    assert_close(from_gpu(y[sample]), yref, f"peers y t={t} b={b} n={n}", literal=True)
    if b % t == 0:
        rows = b // t
        for r in range(t):
            Rs = R[r * rows:(r + 1) * rows].contiguous() if with_residual else None
            ro, yo = ttl.reduce_partials_rmsnorm_peers(peers, gamma, 1e-5, row0=r * rows, rows=rows, residual=Rs)
            ro_s, yo_s = ttl.reduce_scatter_partials_rmsnorm(P, gamma, 1e-5, r, Rs)
            torch.cuda.synchronize()
            assert torch.equal(ro, ro_s) and torch.equal(yo, yo_s), f"two-shot chunk {r}"
            assert torch.equal(ro, rout_s[r * rows:(r + 1) * rows]), f"two-shot chunk {r}"  # h: per element


def test_reduce_scatter_rejects_ragged_rows(ttl):
    P = torch.zeros((4, 6, 8), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ttl.TTLError) as e:
        ttl.reduce_scatter_partials_rmsnorm(P, torch.ones(8, dtype=torch.bfloat16, device="cuda"), 1e-5, 0)
    assert e.value.status == ttl.ERR_NOT_DIVISIBLE


# ---- stream capture -------------------------------------------------------------------------------

@pytest.mark.parametrize("b", [64, 600, 1000])
def test_graph_replay_matches_eager(ttl, gemm_force, capfd, b):
    """The rank chain (gate_up + SiLU·up, down, reduce + RMSNorm over all ranks) captured into a HIP
    graph and replayed three times, with eager work between the replays (including a split-K call
    large enough to replace the library's workspace), reproduces the eager outputs bit for bit.
    b = 64 runs the split-K kernel with its workspace, b = 600 the 256 x 256 tiles, b = 1000 the
    256-row / 192-row cut (planned for 10 CUs: both GEMMs are 16 tiles of 256 x 256, one round
    plus 6 tiles, cut into 10 tiles of 256 rows and 10 of 192 rows)."""
    gemm_force.set(kernel="auto")
    gemm_force.set(splits=0)
    if b == 600:
        gemm_force.set(kernel="tiled")
    if b == 1000:
        gemm_force.set(kernel="mixed")
        gemm_force.set(plan_cus=10)
        gemm_force.set(trace=True)
    t, H, I = 4, 1024, 2048
    X = gpu(wl.random_bf16((b, H), 160))
    R = gpu(wl.random_bf16((b, H), 161))
    gamma = gpu(wl.random_bf16((H,), 162, mean=1.0, std=0.1))
    Wgu = gpu(wl.random_bf16((H, 2 * I), 163, std=0.05))
    Wd = gpu(wl.random_bf16((I, H), 164, std=0.05))
    sp = ttl.merged_gate_up_split(I, t)
    act = torch.empty((t, b, I // t), dtype=torch.bfloat16, device="cuda")
    P = torch.empty((t, b, H), dtype=torch.bfloat16, device="cuda")
    rout = torch.empty((b, H), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((b, H), dtype=torch.bfloat16, device="cuda")

    def chain():
        for r in range(t):
            ttl.shard_linear_col(X, Wgu, t, r, sp, ttl.EPI_SILU_MUL, Y=act[r])
            ttl.shard_linear_row(act[r], Wd, t, r, True, P=P[r])
        ttl.reduce_partials_rmsnorm(P, gamma, 1e-5, R, residual_out=rout, Y=y)

    capfd.readouterr()
    chain()  # eager, on the current stream
    torch.cuda.synchronize()
    if b == 1000:
        assert capfd.readouterr().err.count("ttl gemm cut") == 2 * t  # both GEMMs of every rank
    want = [v.clone() for v in (act, P, rout, y)]
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        chain()  # eager on the capturing stream: allocates its split-K workspace before capture
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            chain()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    Xbig = gpu(wl.random_bf16((32, 8192), 165))
    Wbig = gpu(wl.random_bf16((8192, 16384), 166, std=0.02))
    for rep in range(3):
        for v in (act, P, rout, y):
            v.zero_()
        g.replay()
        torch.cuda.synchronize()
        for got, exp in zip((act, P, rout, y), want):
            assert torch.equal(got, exp), f"replay {rep} differs from the eager run"
        # eager work between replays on the capturing stream: a split-K call whose workspace need
        # (64 splits of 32 x 16384 fp32 = 134 MB) exceeds every earlier one, so the library
        # replaces that stream's buffer (the captured graph keeps the one it recorded)
        saved = dict(gemm_force.state)
        gemm_force.set(kernel="splitk", splits=64 + rep)
        with torch.cuda.stream(s):
            Ybig = ttl.shard_linear_col(Xbig, Wbig, 1, 0)
        gemm_force.set(**saved)
        torch.cuda.synchronize()
        assert torch.isfinite(Ybig.float()).all()
