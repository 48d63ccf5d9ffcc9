"""Helpers shared by the GPU parity tests: tensor <-> bit conversions and the
comparison rules.

Comparison rules (fixed for this method):
* combined output: |gpu - oracle| <= tol * M + 1e-6, where M is the largest
  finite |value| of the inputs being combined and tol depends on the dtype of
  the RESULT: 8e-3 for bf16, 1e-3 for fp16 (the final rounding, 2^-9 and
  2^-12 relative, plus fp32 weights and accumulation), and 2e-5 for fp32
  results (from fp32 or 16-bit inputs). The fp32 figure: a weight 2^(x s)
  computed in fp32 is off by at most (2 |x s| + 2) 2^-24 relative, and only
  weights above 2^-24 matter, so |x s| < 24 and that is < 50 * 2^-24; the
  clamped sum, its reciprocal and the product add (N + 2) 2^-24; the N fused
  multiply-adds add N 2^-24 of M. For N <= 32 the sum is below 1.2e-5 * M.
  NaN and infinite positions must match;
* global LSE: |gpu - oracle| <= 1e-5 absolute; non-finite values must match
  exactly (-inf with -inf);
* pack / unpack: bitwise equal.
"""
import numpy as np
import torch

TOL = {"bf16": 8e-3, "f16": 1e-3, "f32": 2e-5}
TORCH_DT = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}


def to_dev(bits: np.ndarray, dtype: str, dev) -> torch.Tensor:
    """Element patterns -> tensor on ``dev`` (bit-exact): uint16 patterns for
    bf16 / fp16, float32 values or uint32 patterns for f32."""
    a = np.ascontiguousarray(bits)
    if dtype == "f32":
        return torch.from_numpy(a.view(np.float32).copy()).to(dev)
    return torch.from_numpy(a.view(np.int16)).view(TORCH_DT[dtype]).to(dev)


def f32_to_dev(a: np.ndarray, dev) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)


def bits_of(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def f32_bits_of(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int32).cpu().numpy().view(np.uint32)


def elem_bits_of(t: torch.Tensor, dtype: str) -> np.ndarray:
    """Element patterns of a tensor: uint16 for bf16 / fp16, uint32 for f32."""
    return f32_bits_of(t) if dtype == "f32" else bits_of(t)


def max_abs_input(bits: np.ndarray, dtype: str) -> float:
    bits = np.ascontiguousarray(bits)
    if dtype == "f32":
        x = bits.view(np.float32)
    elif dtype == "bf16":
        x = (bits.astype(np.uint32) << 16).view(np.float32)
    else:
        x = bits.view(np.float16)
    with np.errstate(invalid="ignore"):  # signalling-NaN patterns widen to NaN
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


def host_threads() -> int:
    """Threads for host-side oracle work: the CPUs this process may use, at
    most 16 (one GPU's share of a host's CPUs)."""
    import os
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def assert_combine_close_in_chunks(y_gpu: torch.Tensor, L_gpu, o: np.ndarray, l: np.ndarray,
                                   dtype: str, base2: bool, M: float, chunk_tokens: int = 1024,
                                   what: str = "") -> None:
    """Every row of a combine [B, H, D] (and its global LSE [B, H], if given)
    against the oracle, element by element. The oracle runs over token ranges
    of o [N, B, H, D] / l [N, B, H] on host threads (rows are independent, so a
    token range of the inputs gives exactly those rows' results), which bounds
    host memory at full size."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle

    B = o.shape[1]
    ranges = [(s, min(s + chunk_tokens, B)) for s in range(0, B, chunk_tokens)]

    def ref(r):
        s, e = r
        return oracle.lse_combine(np.ascontiguousarray(o[:, s:e]), np.ascontiguousarray(l[:, s:e]),
                                  dtype, base2=base2)

    with ThreadPoolExecutor(max_workers=host_threads()) as ex:
        for (s, e), (y_ref, L_ref) in zip(ranges, ex.map(ref, ranges)):
            assert_output_close(y_gpu[s:e], y_ref, dtype, M, f"{what} tokens {s}:{e}")
            if L_gpu is not None:
                assert_lse_close(L_gpu[s:e], L_ref, f"{what} tokens {s}:{e}")
