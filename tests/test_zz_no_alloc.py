"""shard_linear_col_noalloc, whose split-K partials live in the library's static device scratch
instead of an allocated workspace, against the allocating entry points through the C ABI: bit for
bit the same outputs on consecutive calls (the second with a smaller input), sampled rows against
the oracle, and a HIP-graph capture on a stream that never ran an eager call (nothing to
allocate), replayed with eager work in between."""

import numpy as np
import pytest
import torch

import oracle
from tensor_transformer_linear_amd import workloads as wl
from tests.util import assert_close, f64, from_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ttl():
    from tensor_transformer_linear_amd import ttl as lib
    assert torch.cuda.is_available()
    return lib


def _rand(shape, seed, std=1.0):
    return wl.random_bf16(shape, seed, std=std, device="cuda")


def test_noalloc_equals_allocating_calls(ttl, gemm_force):
    gemm_force.reset()
    # Call 1: the Llama-3-70B layer's qkv at 2176 tokens, t = 8 (8 q + 1 kv heads of 128 per rank):
    # 45 tiles of 256 x 256 in 5 k-splits, 55.7 MB of fp32 partials in the scratch.
    t, b1, H = 8, 2176, 8192
    X1 = _rand((b1, H), 190)
    W1 = _rand((H, 10240), 191, std=0.02)
    sp1 = ttl.qkv_split(64, 8, 128, t)
    outs1 = {}
    for rank in (0, 7):
        want = ttl.shard_linear_col(X1, W1, t, rank, sp1)
        got = ttl.shard_linear_col_noalloc(X1, W1, t, rank, sp1, Y=torch.empty_like(want))
        torch.cuda.synchronize()
        assert torch.equal(got, want), f"qkv rank {rank}: the static-scratch call differs"
        outs1[rank] = got
    rows = [0, 1, 1023, 2047, 2048, 2175]
    ref = oracle.col_shard(f64(X1[rows].cpu()), f64(W1.cpu()), oracle.qkv_split(64, 8, 128, t), t, 7)
    assert_close(from_gpu(outs1[7][rows]), ref, "noalloc qkv rank 7")

    # Call 2, smaller: a 64-token Llama-3-70B gate_up with SiLU·up, W stored [n][k]: the split-K
    # kernel, 56 tiles in 4 k-splits (7.3 MB of partials), over the scratch the first call left.
    b2, I = 64, 28672
    X2 = _rand((b2, H), 192)
    W2 = _rand((H, 2 * I), 193, std=0.02)
    W2t = W2.t().contiguous()
    sp2 = ttl.merged_gate_up_split(I, t)
    want2 = ttl.shard_linear_col(X2, W2t, t, 3, sp2, ttl.EPI_SILU_MUL, w_layout=ttl.W_NK)
    got2 = ttl.shard_linear_col_noalloc(X2, W2t, t, 3, sp2, ttl.EPI_SILU_MUL, Y=torch.empty_like(want2),
                                        w_layout=ttl.W_NK)
    torch.cuda.synchronize()
    assert torch.equal(got2, want2), "decode gate_up: the static-scratch call differs"
    ref2 = oracle.silu_mul(oracle.col_shard(f64(X2.cpu()), f64(W2.cpu()), oracle.merged_gate_up_split(I, t), t, 3))
    assert_close(from_gpu(got2), ref2, "noalloc decode gate_up rank 3")

    # The first shape once more: unaffected by what the smaller call left in the scratch.
    again = ttl.shard_linear_col_noalloc(X1, W1, t, 7, sp1)
    torch.cuda.synchronize()
    assert torch.equal(again, outs1[7])


def test_noalloc_captures_without_an_eager_call(ttl, gemm_force):
    """Captured on a fresh stream with no eager call before it (the allocating entry point would
    need one there), replayed three times with eager split-K calls in between: every replay equals
    the allocating entry point's result."""
    gemm_force.reset()
    t, b, H, I = 8, 32, 4096, 14336
    X = _rand((b, H), 194)
    W = _rand((H, 2 * I), 195, std=0.02)
    sp = ttl.merged_gate_up_split(I, t)
    want = ttl.shard_linear_col(X, W, t, 5, sp, ttl.EPI_SILU_MUL)
    ttl.shard_linear_col_noalloc(X, W, t, 5, sp, ttl.EPI_SILU_MUL)  # looks up the scratch address
    torch.cuda.synchronize()
    Y = torch.empty_like(want)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            ttl.shard_linear_col_noalloc(X, W, t, 5, sp, ttl.EPI_SILU_MUL, Y=Y)
    torch.cuda.synchronize()
    X2 = _rand((48, 8192), 196)
    W2 = _rand((8192, 4096), 197, std=0.02)
    for rep in range(3):
        Y.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(Y, want), f"replay {rep} differs"
        ttl.shard_linear_col_noalloc(X2, W2, 1, 0)  # other partials through the same scratch
        torch.cuda.synchronize()
