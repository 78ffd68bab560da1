"""Shapes and seeded synthetic inputs for the sharded linear path.

This module only *draws* inputs; it holds none of the path's arithmetic.  Both the HIP path and the
CPU oracle receive the tensors it returns.

Shapes follow Llama-style decoders as used on the vLLM tensor-parallel walkthrough (pinghaoyang.com.cn,
"vLLM 源码完全拆解（十一）", sections "MergedColumnParallelLinear / QkvParallelLinear" and
"一个典型 block 的列行交替拼装") and the Llama-3-70B shape on the worker-orchestration page
(mlinterviewnotes.com, "Worker orchestration and multi-node serving", opening section:
80 layers, hidden 8192, 64 query heads, 8 kv heads).

Value recipe (no dataset is involved; these stand in for real activations and weights):
  activations X, attention-output stand-in A and residual R ~ N(0, 1);
  weights ~ N(0, 0.02) (second parameter is the standard deviation);
  RMSNorm gain gamma ~ N(1, 0.1);
  each value drawn in fp32 from one ``torch.Generator`` seeded per workload, then rounded to bf16
  (round to nearest even).  Draw order: X, R, gamma(s), then full unsharded weights in layer order
  (Wqkv, A, Wo, Wgate_up, Wdown).  Per-rank shards are views/offsets of these full tensors.
"""

from __future__ import annotations

import dataclasses
from typing import Dict, Tuple

import torch

EPS = 1e-5


@dataclasses.dataclass(frozen=True)
class MlpShard:
    """Gated MLP of one TP group: gate_up column-parallel, down row-parallel."""
    name: str
    hidden: int
    intermediate: int
    t: int
    batches: Tuple[int, ...]
    eps: float = EPS


@dataclasses.dataclass(frozen=True)
class AttnShard:
    """Attention projections of one TP group: qkv column-parallel by head, o_proj row-parallel."""
    name: str
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    t: int
    batches: Tuple[int, ...]
    eps: float = EPS


@dataclasses.dataclass(frozen=True)
class LayerShard:
    """Whole decoder layer, linear path only: qkv/o_proj then gate_up/down, two reduce+norm steps."""
    name: str
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    intermediate: int
    t: int
    batches: Tuple[int, ...]
    eps: float = EPS


TINY_MLP_T2 = MlpShard("tiny_mlp_h256_i688_t2", hidden=256, intermediate=688, t=2, batches=(16,))
LLAMA3_8B_MLP_TP8 = MlpShard("llama3_8b_mlp_tp8", hidden=4096, intermediate=14336, t=8,
                             batches=(1, 32, 256))
LLAMA3_8B_ATTN_TP4 = AttnShard("llama3_8b_attn_tp4", hidden=4096, n_q_heads=32, n_kv_heads=8,
                               head_dim=128, t=4, batches=(2048,))
LLAMA3_70B_MLP_TP8 = MlpShard("llama3_70b_mlp_tp8", hidden=8192, intermediate=28672, t=8,
                              batches=(4096, 64))
# 2048-token chunked-prefill segment plus 128 decode rows, stacked as one M = 2176 batch.
LLAMA3_70B_LAYER_TP8 = LayerShard("llama3_70b_layer_tp8", hidden=8192, n_q_heads=64, n_kv_heads=8,
                                  head_dim=128, intermediate=28672, t=8, batches=(2048 + 128,))

WORKLOADS = (TINY_MLP_T2, LLAMA3_8B_MLP_TP8, LLAMA3_8B_ATTN_TP4, LLAMA3_70B_MLP_TP8,
             LLAMA3_70B_LAYER_TP8)


def _draw(gen: torch.Generator, shape, mean: float, std: float, device) -> torch.Tensor:
    z = torch.randn(shape, generator=gen, dtype=torch.float32, device=device)
    if std != 1.0:
        z.mul_(std)
    if mean != 0.0:
        z.add_(mean)
    return z.to(torch.bfloat16)


def make_generator(seed: int = 0, device="cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def mlp_inputs(w: MlpShard, b: int, seed: int = 0, device="cpu") -> Dict[str, torch.Tensor]:
    """Full (unsharded) bf16 tensors for one MLP workload at batch b.

    Wgu is [hidden, 2*intermediate] with the gate block first, then the up block.
    """
    g = make_generator(seed, device)
    out = {}
    out["X"] = _draw(g, (b, w.hidden), 0.0, 1.0, device)
    out["R"] = _draw(g, (b, w.hidden), 0.0, 1.0, device)
    out["gamma"] = _draw(g, (w.hidden,), 1.0, 0.1, device)
    out["Wgu"] = _draw(g, (w.hidden, 2 * w.intermediate), 0.0, 0.02, device)
    out["Wd"] = _draw(g, (w.intermediate, w.hidden), 0.0, 0.02, device)
    return out


def attn_inputs(w: AttnShard, b: int, seed: int = 0, device="cpu") -> Dict[str, torch.Tensor]:
    """Full bf16 tensors for one attention-projection workload.

    Wqkv is [hidden, (nq + 2*nkv)*head_dim] laid out q | k | v.  A is the attention-core output
    stand-in [b, nq*head_dim] (the attention core itself is not on the linear path).
    """
    g = make_generator(seed, device)
    nq, nkv, hd = w.n_q_heads, w.n_kv_heads, w.head_dim
    out = {}
    out["X"] = _draw(g, (b, w.hidden), 0.0, 1.0, device)
    out["R"] = _draw(g, (b, w.hidden), 0.0, 1.0, device)
    out["gamma"] = _draw(g, (w.hidden,), 1.0, 0.1, device)
    out["Wqkv"] = _draw(g, (w.hidden, (nq + 2 * nkv) * hd), 0.0, 0.02, device)
    out["A"] = _draw(g, (b, nq * hd), 0.0, 1.0, device)
    out["Wo"] = _draw(g, (nq * hd, w.hidden), 0.0, 0.02, device)
    return out


def layer_inputs(w: LayerShard, b: int, seed: int = 0, device="cpu") -> Dict[str, torch.Tensor]:
    g = make_generator(seed, device)
    nq, nkv, hd = w.n_q_heads, w.n_kv_heads, w.head_dim
    out = {}
    out["X"] = _draw(g, (b, w.hidden), 0.0, 1.0, device)
    out["R"] = _draw(g, (b, w.hidden), 0.0, 1.0, device)
    out["gamma_attn"] = _draw(g, (w.hidden,), 1.0, 0.1, device)
    out["gamma_mlp"] = _draw(g, (w.hidden,), 1.0, 0.1, device)
    out["Wqkv"] = _draw(g, (w.hidden, (nq + 2 * nkv) * hd), 0.0, 0.02, device)
    out["A"] = _draw(g, (b, nq * hd), 0.0, 1.0, device)
    out["Wo"] = _draw(g, (nq * hd, w.hidden), 0.0, 0.02, device)
    out["Wgu"] = _draw(g, (w.hidden, 2 * w.intermediate), 0.0, 0.02, device)
    out["Wd"] = _draw(g, (w.intermediate, w.hidden), 0.0, 0.02, device)
    return out


def random_bf16(shape, seed: int, mean: float = 0.0, std: float = 1.0, device="cpu") -> torch.Tensor:
    """A single seeded bf16 tensor (used for stage-wise inputs such as partials or activations)."""
    return _draw(make_generator(seed, device), shape, mean, std, device)


def bf16_bits(x: torch.Tensor):
    """Raw bf16 bit patterns of a CPU tensor as a numpy uint16 array (no arithmetic)."""
    return x.detach().cpu().contiguous().view(torch.int16).numpy().view("uint16")
