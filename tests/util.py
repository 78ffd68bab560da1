"""Helpers shared by the GPU parity tests: moving seeded inputs to both sides and comparing."""

from __future__ import annotations

import numpy as np
import torch

import oracle
from tensor_transformer_linear_amd import workloads as wl

TOL = 2e-2  # per output tensor: error beyond the bf16 rounding of the output <= TOL * rms(ref)


def f64(x: torch.Tensor) -> np.ndarray:
    """The oracle's view of a bf16 tensor: its own decoding of the raw bits."""
    return oracle.bf16_bits_to_f64(wl.bf16_bits(x))


def gpu(x: torch.Tensor) -> torch.Tensor:
    return x.to("cuda", non_blocking=False)


def from_gpu(y: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return f64(y.cpu())


def rms(ref: np.ndarray) -> float:
    return float(np.sqrt(np.mean(np.square(ref)))) if ref.size else 0.0


def bf16_half_ulp(v: np.ndarray) -> np.ndarray:
    """Half the spacing of bf16 values around |v| (the largest error of rounding v to bf16)."""
    a = np.abs(v)
    _, e = np.frexp(np.where(a > 0, a, 1.0))
    half = np.ldexp(1.0, np.maximum(e, -125) - 9)  # spacing 2**(e-8) for |v| in [2**(e-1), 2**e)
    return np.where(a > 0, half, 2.0 ** -134)


def assert_close(got: np.ndarray, ref: np.ndarray, what: str, tol: float = TOL, literal: bool = False):
    """The parity bar for one output tensor.

    literal=True (the normalised outputs y and the residual stream): max |got - ref| <= tol * rms(ref),
    the bound as stated.  literal=False (the SiLU·up activations and the GEMM outputs and partials):
    max over elements of (|got - ref| - rounding of the output to bf16) <= tol * rms(ref).  `got` is a
    bf16 output and `ref` the oracle's unrounded float64 value.  Storing a value in bf16 alone moves
    it by up to half a bf16 spacing (2**-9 to 2**-8 of its magnitude), which for the heavy-tailed
    SiLU·up products, and for GEMM outputs whose largest elements sit beyond about five times their
    rms, exceeds 2e-2 * rms at those elements for any bf16 result, however computed; there that
    storage rounding is discounted element by element and the bound applies to the computation's
    error beyond it.  Both figures are printed on one line tagged "parity".
    """
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    if ref.size == 0:
        return 0.0
    diff = np.abs(got - ref)
    excess = np.maximum(diff - bf16_half_ulp(np.maximum(np.abs(ref), np.abs(got))), 0.0)
    err = float(np.max(excess))
    raw = float(np.max(diff))
    bound = tol * rms(ref)
    print(f"  parity {what}: raw max|err| = {raw:.3e}, beyond bf16 rounding = {err:.3e}, "
          f"bound = {bound:.3e} (rms(ref) = {rms(ref):.3e}), asserted on "
          f"{'raw' if literal else 'beyond-rounding'}", flush=True)
    if literal:
        assert raw <= bound, f"{what}: max|err| {raw:.4e} > {tol} * rms(ref) = {bound:.4e}"
        return raw / max(rms(ref), 1e-300)
    assert err <= bound, f"{what}: error {err:.4e} beyond bf16 rounding > {tol} * rms(ref) = {bound:.4e}"
    return err / max(rms(ref), 1e-300)


def parity_rows(b: int, extra=()) -> list:
    """Token rows compared with the oracle at full size.  Every row when b <= 256.  Otherwise at
    least 256 rows: the first and the last row of every 64-row block (every tile the GEMMs launch,
    256 rows, 192 rows of the 256-row / 192-row cut, or 32..128 rows of the split-K kernel, starts
    at a multiple of 64, so each of them contributes at least its first row), plus seeded picks
    among the others and any `extra` rows.  Rows are independent through every step, so each
    sampled row is compared exactly."""
    if b <= 256:
        return list(range(b))
    rows = {0, b - 1}
    for r0 in range(0, b, 64):
        rows.add(r0)
        rows.add(min(r0 + 63, b - 1))
    rows.update(int(r) for r in extra if 0 <= r < b)
    rng = np.random.default_rng(1234 + b)
    rest = np.array([r for r in range(b) if r not in rows])
    need = max(0, 256 + 32 - len(rows))
    rows.update(int(r) for r in rng.choice(rest, size=min(need, rest.size), replace=False))
    return sorted(rows)
