"""Helpers shared by the GPU parity tests: tensor <-> bit conversions and the
comparison rules.

Comparison rules (fixed for this method):
* combined output: |gpu - oracle| <= 8e-3 * M + 1e-6 for bf16 and
  <= 1e-3 * M + 1e-6 for fp16, where M is the largest finite |value| of the
  inputs being combined; NaN and infinite positions must match;
* global LSE: |gpu - oracle| <= 1e-5 absolute; non-finite values must match
  exactly (-inf with -inf);
* pack / unpack: bitwise equal.
"""
import numpy as np
import torch

TOL = {"bf16": 8e-3, "f16": 1e-3}
TORCH_DT = {"bf16": torch.bfloat16, "f16": torch.float16}


def to_dev(bits: np.ndarray, dtype: str, dev) -> torch.Tensor:
    """uint16 bit patterns -> bf16 / fp16 tensor on ``dev`` (bit-exact)."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(TORCH_DT[dtype]).to(dev)


def f32_to_dev(a: np.ndarray, dev) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)


def bits_of(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def f32_bits_of(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int32).cpu().numpy().view(np.uint32)


def max_abs_input(bits: np.ndarray, dtype: str) -> float:
    x = (bits.astype(np.uint32) << 16).view(np.float32) if dtype == "bf16" else bits.view(np.float16)
    x = np.abs(x.astype(np.float64))
    x = x[np.isfinite(x)]
    return float(x.max()) if x.size else 0.0


def assert_output_close(y_gpu: torch.Tensor, y_ref: np.ndarray, dtype: str, M: float,
                        what: str = "") -> float:
    y = y_gpu.float().cpu().numpy().astype(np.float64)
    assert y.shape == y_ref.shape, (what, y.shape, y_ref.shape)
    assert np.array_equal(np.isnan(y), np.isnan(y_ref)), f"{what}: NaN positions differ"
    inf_r = np.isinf(y_ref)
    assert np.array_equal(y[inf_r], y_ref[inf_r]), f"{what}: infinities differ"
    fin = np.isfinite(y_ref)
    if not fin.any():
        return 0.0
    err = float(np.max(np.abs(y[fin] - y_ref[fin])))
    tol = TOL[dtype] * M + 1e-6
    assert err <= tol, f"{what}: max |gpu - oracle| = {err:.3g} > {tol:.3g}"
    return err


def assert_lse_close(L_gpu: torch.Tensor, L_ref: np.ndarray, what: str = "") -> float:
    L = L_gpu.cpu().numpy().astype(np.float64)
    assert L.shape == L_ref.shape
    fin = np.isfinite(L_ref)
    assert np.array_equal(L[~fin], L_ref[~fin]), f"{what}: non-finite LSEs differ"
    if not fin.any():
        return 0.0
    assert np.all(np.isfinite(L[fin])), f"{what}: GPU LSE non-finite where oracle is finite"
    err = float(np.max(np.abs(L[fin] - L_ref[fin])))
    assert err <= 1e-5, f"{what}: max |LSE gpu - oracle| = {err:.3g} > 1e-5"
    return err
