"""Pins of the CPU oracle against what the pages and mathematics fix (no GPU, no HIP library).

Every check here is independent of the oracle's own formulas: brute-force dot products summed with
math.fsum, sharding invariants (column shards concatenate to the unsharded product, row partials sum
to it), closed forms of SiLU and RMSNorm, the head arithmetic printed on the pages, and torch's
fp32->bf16 rounding as a library yardstick.  ``test_planted_mistakes_are_caught`` plants plausible
mistakes into the oracle and checks that at least one pin fails for each.
"""

import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle
import oracle.tp_linear as otl
from tensor_transformer_linear_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bf16(shape, seed, mean=0.0, std=1.0):
    """Seeded bf16 tensor -> (oracle float64 array, python nested lists decoded by torch)."""
    t = wl.random_bf16(shape, seed, mean, std)
    return oracle.bf16_bits_to_f64(wl.bf16_bits(t)), t.float().double().tolist()


def _fsum_dot(xrow, W, c, ks):
    return math.fsum(xrow[p] * W[p][c] for p in ks)


def _fp64_bound(xrow, W, c, ks):
    # float64 summation error bound: len(ks) * 2**-53 * sum |x*w|
    return len(ks) * 2.0 ** -53 * math.fsum(abs(xrow[p] * W[p][c]) for p in ks) + 1e-300


# ---------------------------------------------------------------------------------------------
# Pins (each raises AssertionError on a mismatch)
# ---------------------------------------------------------------------------------------------

def pin_decode():
    bits = np.array([0x3F80, 0xC000, 0x7F80, 0x0001, 0x3F81, 0x8000, 0x4049], dtype=np.uint16)
    got = oracle.bf16_bits_to_f64(bits)
    want = [1.0, -2.0, math.inf, 2.0 ** -133, 1.0 + 2.0 ** -7, -0.0, 3.140625]
    assert got.tolist() == want
    assert math.copysign(1.0, got[5]) == -1.0


def pin_rounding_vs_torch():
    # For values that are exactly float32, rounding float64 -> bf16 directly must equal torch's
    # float32 -> bf16 round-to-nearest-even.
    g = torch.Generator().manual_seed(7)
    x = torch.cat([torch.randn(20000, generator=g) * 10.0 ** torch.randint(-30, 30, (20000,), generator=g),
                   torch.tensor([0.0, -0.0, 1e-40, -3e-39, 3.389e38, -3.4e38, 65504.0, 1.0 + 2 ** -8])])
    want = x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.f64_to_bf16_bits(x.double().numpy())
    assert np.array_equal(got, want)


def pin_rounding_ties():
    # halfway cases go to the even neighbour
    xs = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8), 2.0 ** -133 * 1.5, 2.0 ** -133 * 2.5])
    want = [1.0, 1 + 2.0 ** -6, -1.0, 2.0 ** -132, 2.0 ** -132]
    assert oracle.round_bf16(xs).tolist() == want
    # just above halfway rounds up
    assert oracle.round_bf16(np.array([1 + 2.0 ** -8 + 2.0 ** -30]))[0] == 1 + 2.0 ** -7


def _tiny_cases():
    # (b, k, split-builder, t) with non-square, odd-ish shapes
    return [
        (3, 40, lambda t: oracle.plain_split(48, t), 4),
        (5, 24, lambda t: oracle.plain_split(16, t), 1),
        (4, 32, lambda t: oracle.merged_gate_up_split(24, t), 2),
        (2, 16, lambda t: oracle.merged_gate_up_split(32, t), 8),
        (3, 16, lambda t: oracle.qkv_split(8, 4, 4, t), 4),   # t <= n_kv
        (3, 16, lambda t: oracle.qkv_split(8, 2, 4, t), 4),   # t > n_kv: kv heads replicated
    ]


def pin_col_brute_force():
    seed = 100
    for b, k, mk, t in _tiny_cases():
        split = mk(t)
        n = sum(split[0])
        X, Xl = _bf16((b, k), seed)
        W, Wl = _bf16((k, n), seed + 1, std=0.5)
        seed += 2
        ks = range(k)
        for r in range(t):
            Y = oracle.col_shard(X, W, split, t, r)
            cols = oracle.rank_columns(split, t, r)
            # independent restatement of which columns rank r owns
            want_cols = []
            off = 0
            for n_i, p_i in zip(*split):
                w = n_i // p_i
                q = r * p_i // t
                want_cols += list(range(off + q * w, off + (q + 1) * w))
                off += n_i
            assert list(cols) == want_cols
            assert Y.shape == (b, len(want_cols))
            for a in range(b):
                for j, c in enumerate(want_cols):
                    ref = _fsum_dot(Xl[a], Wl, c, ks)
                    assert abs(Y[a, j] - ref) <= _fp64_bound(Xl[a], Wl, c, ks)


def pin_col_concat_invariant():
    b, k, I, t = 6, 48, 40, 4
    X, _ = _bf16((b, k), 11)
    # plain column split: concatenation over ranks == unsharded X @ W
    W, _ = _bf16((k, 80), 12, std=0.1)
    full = X @ W
    cat = np.concatenate([oracle.col_shard(X, W, oracle.plain_split(80, t), t, r) for r in range(t)], 1)
    np.testing.assert_allclose(cat, full, rtol=0, atol=1e-12)
    # merged gate|up: gate halves over ranks give X @ Wg, up halves give X @ Wu
    Wgu, _ = _bf16((k, 2 * I), 13, std=0.1)
    outs = [oracle.col_shard(X, Wgu, oracle.merged_gate_up_split(I, t), t, r) for r in range(t)]
    h = I // t
    np.testing.assert_allclose(np.concatenate([o[:, :h] for o in outs], 1), X @ Wgu[:, :I], atol=1e-12, rtol=0)
    np.testing.assert_allclose(np.concatenate([o[:, h:] for o in outs], 1), X @ Wgu[:, I:], atol=1e-12, rtol=0)
    # qkv by head, t <= n_kv: q, k, v parts each concatenate to the full projection
    nq, nkv, hd = 8, 4, 4
    Wqkv, _ = _bf16((k, (nq + 2 * nkv) * hd), 14, std=0.1)
    outs = [oracle.col_shard(X, Wqkv, oracle.qkv_split(nq, nkv, hd, t), t, r) for r in range(t)]
    qw, kw = nq * hd // t, nkv * hd // t
    Q = np.concatenate([o[:, :qw] for o in outs], 1)
    K = np.concatenate([o[:, qw:qw + kw] for o in outs], 1)
    V = np.concatenate([o[:, qw + kw:] for o in outs], 1)
    np.testing.assert_allclose(Q, X @ Wqkv[:, :nq * hd], atol=1e-12, rtol=0)
    np.testing.assert_allclose(K, X @ Wqkv[:, nq * hd:(nq + nkv) * hd], atol=1e-12, rtol=0)
    np.testing.assert_allclose(V, X @ Wqkv[:, (nq + nkv) * hd:], atol=1e-12, rtol=0)
    # t > n_kv: rank r holds kv head floor(r * n_kv / t); ranks sharing it hold identical k/v
    nkv2, t2 = 2, 8
    Wq2, _ = _bf16((k, (nq + 2 * nkv2) * hd), 15, std=0.1)
    sp = oracle.qkv_split(nq, nkv2, hd, t2)
    for r in range(t2):
        o = oracle.col_shard(X, Wq2, sp, t2, r)
        head = r * nkv2 // t2
        kcols = slice(nq * hd + head * hd, nq * hd + (head + 1) * hd)
        np.testing.assert_allclose(o[:, nq * hd // t2: nq * hd // t2 + hd], X @ Wq2[:, kcols], atol=1e-12, rtol=0)


def pin_row_brute_force():
    seed = 300
    for b, k, n, t in [(3, 48, 20, 4), (2, 16, 8, 1), (4, 64, 12, 8), (5, 24, 16, 2)]:
        X, Xl = _bf16((b, k), seed)
        W, Wl = _bf16((k, n), seed + 1, std=0.5)
        seed += 2
        w = k // t
        for r in range(t):
            ks = range(r * w, (r + 1) * w)
            P_full_input = oracle.row_shard(X, W, t, r, x_is_parallel=False)
            P_par_input = oracle.row_shard(X[:, r * w:(r + 1) * w], W, t, r, x_is_parallel=True)
            assert P_full_input.shape == (b, n)
            assert np.array_equal(P_full_input, P_par_input)
            for a in range(b):
                for c in range(n):
                    ref = _fsum_dot(Xl[a], Wl, c, ks)
                    assert abs(P_full_input[a, c] - ref) <= _fp64_bound(Xl[a], Wl, c, ks)


def pin_row_sum_invariant():
    b, k, n = 5, 96, 36
    X, _ = _bf16((b, k), 21)
    W, _ = _bf16((k, n), 22, std=0.1)
    full = X @ W
    for t in (1, 2, 4, 8):
        s = sum(oracle.row_shard(X, W, t, r, False) for r in range(t))
        np.testing.assert_allclose(s, full, rtol=0, atol=1e-12)
        if t == 1:
            np.testing.assert_allclose(oracle.row_shard(X, W, 1, 0, False), full, rtol=0, atol=1e-12)


def pin_silu_closed_forms():
    xs = np.linspace(-30, 30, 601)
    s = oracle.silu(xs)
    assert oracle.silu(np.array([0.0]))[0] == 0.0
    # silu(x) - silu(-x) = x, since sigmoid(x) + sigmoid(-x) = 1
    np.testing.assert_allclose(s - oracle.silu(-xs), xs, rtol=0, atol=1e-12)
    # slope 1/2 at the origin
    assert abs(oracle.silu(np.array([1e-9]))[0] / 1e-9 - 0.5) < 1e-8
    # asymptotes: silu(x) -> x for large x, -> 0 for very negative x
    assert abs(oracle.silu(np.array([40.0]))[0] - 40.0) < 1e-12
    assert abs(oracle.silu(np.array([-40.0]))[0]) < 1e-15
    # the minimum: at x* = -(1 + W(1/e)) (Lambert W), silu(x*) = x* + 1 = -W(1/e)
    w = float(scipy.special.lambertw(math.exp(-1)).real)
    xstar = -(1.0 + w)
    v = oracle.silu(np.array([xstar, xstar - 1e-4, xstar + 1e-4]))
    assert abs(v[0] + w) < 1e-14
    assert v[1] > v[0] and v[2] > v[0]


def pin_silu_mul():
    g = np.array([[0.0, 1.5, -2.0, 40.0]])
    u = np.array([[3.0, 1.0, 0.0, 0.5]])
    y = oracle.silu_mul(np.concatenate([g, u], 1))
    assert y.shape == (1, 4)
    # u = 1 passes silu(g) through; u = 0 zeroes; large g gives g * u; g = 0 gives 0
    assert y[0, 0] == 0.0 and y[0, 2] == 0.0
    np.testing.assert_allclose(y[0, 1], oracle.silu(np.array([1.5]))[0], rtol=0, atol=0)
    np.testing.assert_allclose(y[0, 3], 20.0, rtol=0, atol=1e-12)


def pin_rmsnorm_closed_forms():
    n, eps = 64, 1e-5
    gamma, _ = _bf16((n,), 31, mean=1.0, std=0.1)
    # constant row h = c: y = c / sqrt(c^2 + eps) * gamma
    for c in (3.0, -0.5, 1e-3):
        P = np.full((1, 1, n), c)
        h, y = oracle.reduce_partials_rmsnorm(P, None, gamma, eps)
        np.testing.assert_allclose(y[0], c / math.sqrt(c * c + eps) * gamma, rtol=1e-15, atol=0)
        assert np.array_equal(h[0], np.full(n, c))
    # zero row stays zero
    _, y0 = oracle.reduce_partials_rmsnorm(np.zeros((2, 1, n)), np.zeros((1, n)), gamma, eps)
    assert np.all(y0 == 0.0)
    # mean((y/gamma)^2) = ms / (ms + eps) for any row (catches eps outside the root, sum vs mean)
    Pr, _ = _bf16((3, 4, n), 32)
    R, _ = _bf16((4, n), 33)
    h, y = oracle.reduce_partials_rmsnorm(Pr, R, gamma, eps)
    ms = np.mean(h * h, axis=1)
    np.testing.assert_allclose(np.mean((y / gamma) ** 2, axis=1), ms / (ms + eps), rtol=1e-13)
    # with eps = 0 the output is scale invariant (positive scale)
    _, ya = oracle.reduce_partials_rmsnorm(Pr, R, gamma, 0.0)
    _, yb = oracle.reduce_partials_rmsnorm(Pr * 4.0, R * 4.0, gamma, 0.0)
    np.testing.assert_allclose(ya, yb, rtol=1e-14, atol=0)


def pin_reduce_residual():
    t, b, n = 4, 3, 16
    P, Pl = _bf16((t, b, n), 41)
    R, Rl = _bf16((b, n), 42)
    gamma, gl = _bf16((n,), 43, mean=1.0, std=0.1)
    h, y = oracle.reduce_partials_rmsnorm(P, R, gamma, 1e-5)
    # brute force per element: h = sum_r P[r] + R, y = h / sqrt(mean h^2 + eps) * gamma
    for a in range(b):
        hr = [math.fsum([Pl[r][a][j] for r in range(t)] + [Rl[a][j]]) for j in range(n)]
        ms = math.fsum(v * v for v in hr) / n
        for j in range(n):
            assert abs(h[a, j] - hr[j]) <= 1e-14 * (1 + abs(hr[j]))
            want = hr[j] / math.sqrt(ms + 1e-5) * gl[j]
            assert abs(y[a, j] - want) <= 1e-13 * (1 + abs(want))
    # residual absent == zero residual; partials zero -> h is the residual
    h1, y1 = oracle.reduce_partials_rmsnorm(P, None, gamma, 1e-5)
    h2, y2 = oracle.reduce_partials_rmsnorm(P, np.zeros((b, n)), gamma, 1e-5)
    assert np.array_equal(h1, h2) and np.array_equal(y1, y2)
    h3, _ = oracle.reduce_partials_rmsnorm(np.zeros((t, b, n)), R, gamma, 1e-5)
    assert np.array_equal(h3, R)


def pin_head_arithmetic_golden():
    with open(os.path.join(GOLDEN, "qkv_heads_per_rank.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        q, kv, rep = oracle.qkv_local_heads(c["q_heads"], c["kv_heads"], c["t"])
        assert (q, kv, rep) == (c["q_per_rank"], c["kv_per_rank"], c["kv_replicas"]), c
        if "cols_per_rank" in c:
            sp = oracle.qkv_split(c["q_heads"], c["kv_heads"], c["head_dim"], c["t"])
            for r in range(c["t"]):
                assert len(oracle.rank_columns(sp, c["t"], r)) == c["cols_per_rank"]


def pin_divisibility():
    with pytest.raises(ValueError):
        oracle.divide(10, 4)
    with pytest.raises(ValueError):
        oracle.rank_columns(oracle.plain_split(30, 4), 4, 0)
    with pytest.raises(ValueError):
        oracle.row_shard(np.zeros((1, 30)), np.zeros((30, 2)), 4, 0, False)
    with pytest.raises(ValueError):
        oracle.qkv_local_heads(32, 8, 3)
    assert oracle.divide(28672, 8) == 3584


def pin_chain_composition():
    # mlp_rank_chain == hand composition; rows are independent (row subset == subset of rows)
    b, hdim, I, t = 5, 32, 24, 4
    X, _ = _bf16((b, hdim), 51)
    Wgu, _ = _bf16((hdim, 2 * I), 52, std=0.2)
    Wd, _ = _bf16((I, hdim), 53, std=0.2)
    acts, P, acts_s, P_s = oracle.mlp_rank_chain(X, Wgu, Wd, t, I, store_bf16=False)
    assert all(np.array_equal(a, b) for a, b in zip(acts, acts_s)) and np.array_equal(P, P_s)
    # unsharded gated MLP: silu(X Wg) * (X Wu) @ Wd == sum of rank partials
    full = (oracle.silu(X @ Wgu[:, :I]) * (X @ Wgu[:, I:])) @ Wd
    np.testing.assert_allclose(P.sum(0), full, rtol=0, atol=1e-12)
    acts2, P2, acts2_s, P2_s = oracle.mlp_rank_chain(X[[0, 3]], Wgu, Wd, t, I, store_bf16=True)
    _, P3, _, P3_s = oracle.mlp_rank_chain(X, Wgu, Wd, t, I, store_bf16=True)
    assert np.array_equal(P2, P3[:, [0, 3]]) and np.array_equal(P2_s, P3_s[:, [0, 3]])
    # bf16 storage: every stored value is the representable rounding of the exact one, and the
    # down projection reads the stored act
    assert np.array_equal(oracle.round_bf16(P2), P2_s)
    assert all(np.array_equal(oracle.round_bf16(a), b) for a, b in zip(acts2, acts2_s))
    np.testing.assert_allclose(P2[1], oracle.row_shard(acts2_s[1], Wd, t, 1, True), rtol=0, atol=0)


def pin_gathered_columns():
    # gather_output=True: the rank outputs concatenated in rank order.  Plain split: equals the
    # unsharded X @ W, checked element by element against fsum dot products; SiLU·up: equals the
    # full silu(X Wg) * (X Wu) by its closed form.
    b, k, n, t = 3, 24, 32, 4
    X, Xl = _bf16((b, k), 61)
    W, Wl = _bf16((k, n), 62, std=0.5)
    G = oracle.col_gathered(X, W, oracle.plain_split(n, t), t)
    assert G.shape == (b, n)
    for a in range(b):
        for c in range(n):
            ref = _fsum_dot(Xl[a], Wl, c, range(k))
            assert abs(G[a, c] - ref) <= _fp64_bound(Xl[a], Wl, c, range(k))
    I = 16
    Wgu, Wgul = _bf16((k, 2 * I), 63, std=0.3)
    A = oracle.col_gathered(X, Wgu, oracle.merged_gate_up_split(I, t), t, epi_silu_mul=True)
    assert A.shape == (b, I)
    for a in range(b):
        for j in range(I):
            g = _fsum_dot(Xl[a], Wgul, j, range(k))
            u = _fsum_dot(Xl[a], Wgul, I + j, range(k))
            want = g / (1.0 + math.exp(-g)) * u
            assert abs(A[a, j] - want) <= 1e-12 * (1 + abs(want))
    # rank order matters: block r is rank r's own output
    sp = oracle.plain_split(n, t)
    for r in range(t):
        np.testing.assert_array_equal(G[:, r * n // t:(r + 1) * n // t], oracle.col_shard(X, W, sp, t, r))


def pin_reduce_scatter_chunks():
    # The t reduce-scatter calls produce the full reduction's rows, chunk by chunk; each chunk is
    # also checked by brute force (fsum over ranks, residual shard, closed-form RMSNorm).
    t, b, n = 4, 8, 16
    P, Pl = _bf16((t, b, n), 71)
    R, Rl = _bf16((b, n), 72)
    gamma, gl = _bf16((n,), 73, mean=1.0, std=0.1)
    h_full, y_full = oracle.reduce_partials_rmsnorm(P, R, gamma, 1e-5)
    rows = b // t
    for r in range(t):
        h, y = oracle.reduce_scatter_partials_rmsnorm(P, R[r * rows:(r + 1) * rows], gamma, 1e-5, t, r)
        assert h.shape == (rows, n)
        np.testing.assert_array_equal(h, h_full[r * rows:(r + 1) * rows])
        np.testing.assert_array_equal(y, y_full[r * rows:(r + 1) * rows])
        for i in range(rows):
            a = r * rows + i
            hr = [math.fsum([Pl[q][a][j] for q in range(t)] + [Rl[a][j]]) for j in range(n)]
            ms = math.fsum(v * v for v in hr) / n
            for j in range(n):
                assert abs(h[i, j] - hr[j]) <= 1e-14 * (1 + abs(hr[j]))
                want = hr[j] / math.sqrt(ms + 1e-5) * gl[j]
                assert abs(y[i, j] - want) <= 1e-13 * (1 + abs(want))
    with pytest.raises(ValueError):
        oracle.reduce_scatter_partials_rmsnorm(np.zeros((4, 6, 8)), None, np.ones(8), 1e-5, 4, 0)


PINS = [pin_decode, pin_rounding_vs_torch, pin_rounding_ties, pin_col_brute_force,
        pin_col_concat_invariant, pin_row_brute_force, pin_row_sum_invariant, pin_silu_closed_forms,
        pin_silu_mul, pin_rmsnorm_closed_forms, pin_reduce_residual, pin_head_arithmetic_golden,
        pin_divisibility, pin_chain_composition, pin_gathered_columns, pin_reduce_scatter_chunks]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin()


# ---------------------------------------------------------------------------------------------
# Planted mistakes: each mutant of the oracle must make at least one pin fail
# ---------------------------------------------------------------------------------------------

def _mut_rank_offset(orig):
    def f(split, t, rank):
        return orig(split, t, (rank + 1) % t)  # wrong slice index
    return f


def _mut_gate_up_contiguous(orig):
    def f(intermediate, t):
        return oracle.column_split((2 * intermediate,), (t,))  # naive contiguous n/t slice of [g|u]
    return f


def _mut_silu_sign(orig):
    def f(x):
        x = np.asarray(x, dtype=np.float64)
        return x / (1.0 + np.exp(x))
    return f


def _mut_silu_mul_swap(orig):
    def f(Y):
        h = Y.shape[1] // 2
        return orig(np.concatenate([Y[:, h:], Y[:, :h]], 1))  # gate/up swapped
    return f


def _mut_row_transposed_slice(orig):
    def f(X, W, t, rank, x_is_parallel):
        X = np.asarray(X, dtype=np.float64)
        W = np.asarray(W, dtype=np.float64)
        w = W.shape[0] // t
        Xr = X if x_is_parallel else X[:, :w]  # always slice 0 of the input
        return Xr @ W[rank * w:(rank + 1) * w, :]
    return f


def _mut_eps_outside(orig):
    def f(P, residual, gamma, eps):
        P = np.asarray(P, dtype=np.float64)
        h = P.sum(0) + (0 if residual is None else np.asarray(residual))
        y = h / (np.sqrt(np.mean(h * h, -1, keepdims=True)) + eps) * gamma
        return h, y
    return f


def _mut_sum_not_mean(orig):
    def f(P, residual, gamma, eps):
        P = np.asarray(P, dtype=np.float64)
        h = P.sum(0) + (0 if residual is None else np.asarray(residual))
        y = h / np.sqrt(np.sum(h * h, -1, keepdims=True) + eps) * gamma
        return h, y
    return f


def _mut_drop_last_partial(orig):
    def f(P, residual, gamma, eps):
        return orig(np.asarray(P)[:-1], residual, gamma, eps)
    return f


def _mut_drop_residual(orig):
    def f(P, residual, gamma, eps):
        return orig(P, None, gamma, eps)
    return f


def _mut_round_truncate(orig):
    def f(x):
        x = np.asarray(x, dtype=np.float64)
        bits = x.astype(np.float32).view(np.uint32) & np.uint32(0xFFFF0000)
        return bits.view(np.float32).astype(np.float64)
    return f


def _mut_kv_replica(orig):
    def f(nq, nkv, hd, t):
        return oracle.column_split((nq * hd, nkv * hd, nkv * hd), (t, t, t))
    return f


def _mut_decode_shift(orig):
    def f(bits):
        b = np.asarray(bits, dtype=np.uint16)
        return (b.astype(np.uint32) << np.uint32(15)).view(np.float32).astype(np.float64)
    return f


def _mut_gather_reversed(orig):
    def bad(X, W, split, t, epi_silu_mul=False):
        y = orig(X, W, split, t, epi_silu_mul)
        w = y.shape[-1] // t
        return np.concatenate([y[:, r * w:(r + 1) * w] for r in reversed(range(t))], axis=-1)
    return bad


def _mut_scatter_wrong_chunk(orig):
    def bad(P, residual_shard, gamma, eps, t, rank):
        return orig(P, residual_shard, gamma, eps, t, (rank + 1) % t)
    return bad


MUTANTS = [
    ("rank_columns", _mut_rank_offset),
    ("merged_gate_up_split", _mut_gate_up_contiguous),
    ("silu", _mut_silu_sign),
    ("silu_mul", _mut_silu_mul_swap),
    ("row_shard", _mut_row_transposed_slice),
    ("reduce_partials_rmsnorm", _mut_eps_outside),
    ("reduce_partials_rmsnorm", _mut_sum_not_mean),
    ("reduce_partials_rmsnorm", _mut_drop_last_partial),
    ("reduce_partials_rmsnorm", _mut_drop_residual),
    ("round_bf16", _mut_round_truncate),
    ("qkv_split", _mut_kv_replica),
    ("bf16_bits_to_f64", _mut_decode_shift),
    ("col_gathered", _mut_gather_reversed),
    ("reduce_scatter_partials_rmsnorm", _mut_scatter_wrong_chunk),
]


@pytest.mark.parametrize("name,mut", MUTANTS, ids=[f"{n}:{m.__name__}" for n, m in MUTANTS])
def test_planted_mistakes_are_caught(monkeypatch, name, mut):
    orig = getattr(otl, name)
    bad = mut(orig)
    monkeypatch.setattr(otl, name, bad)
    monkeypatch.setattr(oracle, name, bad)
    failed = []
    for pin in PINS:
        try:
            pin()
        except (Exception, pytest.fail.Exception) as e:  # any pin tripping counts
            failed.append((pin.__name__, type(e).__name__))
    assert failed, f"no pin caught the planted mistake in {name}"
