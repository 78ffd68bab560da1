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


def assert_close(got: np.ndarray, ref: np.ndarray, what: str, tol: float = TOL):
    """max over elements of (|got - ref| - rounding of the output to bf16) <= tol * rms(ref).

    `got` is a bf16 output and `ref` the oracle's unrounded float64 value.  Storing a value in bf16
    alone moves it by up to half a bf16 spacing (2**-9 to 2**-8 of its magnitude), which for the
    heavy-tailed SiLU*up products exceeds 2e-2 * rms at their largest elements for any bf16 result,
    however computed; that storage rounding is therefore discounted element by element and the bound
    applies to the computation's error beyond it.  The raw max |got - ref| is printed as well.
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
    print(f"  {what}: max excess over bf16 rounding = {err:.3e}, raw max|err| = {raw:.3e}, "
          f"bound = {bound:.3e} (rms(ref) = {rms(ref):.3e})", flush=True)
    assert err <= bound, f"{what}: error {err:.4e} beyond bf16 rounding > {tol} * rms(ref) = {bound:.4e}"
    return err / max(rms(ref), 1e-300)


def sample_rows(b: int, extra=()) -> list:
    """Rows checked one by one at full size: both ends, tile boundaries and a few seeded picks."""
    rows = {0, b - 1}
    # tile edges, and the 256-row / 192-row cut of 4096-row SiLU·up launches (1024 + 192 * j,
    # 2560 + 192 * j)
    for edge in (31, 32, 127, 128, 255, 256, 511, 512, 1023, 1024, 1215, 1216, 2047, 2048, 2559,
                 2560, 2751, 2752, 4095):
        if edge < b:
            rows.add(edge)
    rng = np.random.default_rng(1234 + b)
    rows.update(int(r) for r in rng.integers(0, b, size=min(6, b)))
    rows.update(int(r) for r in extra if 0 <= r < b)
    return sorted(rows)
