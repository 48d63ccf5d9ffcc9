"""Seeded random sweep of every computing entry point against the oracle.

Shapes, dtypes, bases and result dtypes are drawn from a fixed-seed numpy
generator (the same cases on every run): N from 1 to 20, ragged token and head
counts, D from 1 to 640 (so every kernel family and its tails are hit), bf16 /
fp16 / fp32 partials, base e and 2, results in the input dtype or fp32. Each
case is small enough for the oracle to check every element.
"""
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import (assert_lse_close, assert_output_close, elem_bits_of, f32_bits_of,
                         f32_to_dev, max_abs_input, to_dev)

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
TDT = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}
SPECIALS = ((0.03, float("nan")), (0.03, float("inf")), (0.05, float("-inf")))


@pytest.fixture(scope="module")
def lsec():
    import lse_weighted_merge_combine_amd as m
    if not os.path.exists(m.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    m.load_library()
    return m


def _cases(kind, count, seed):
    rng = np.random.default_rng(seed)
    Ds = [1, 3, 8, 12, 24, 64, 100, 128, 136, 256, 512, 640]
    Ns = [1, 2, 3, 4, 5, 8, 16, 20]
    out = []
    for i in range(count):
        N = int(rng.choice(Ns))
        D = int(rng.choice(Ds))
        B = int(rng.integers(1, 70))
        H = int(rng.integers(1, 9))
        dtype = str(rng.choice(["bf16", "f16", "f32"]))
        base2 = bool(rng.integers(0, 2))
        out_f32 = dtype != "f32" and bool(rng.integers(0, 2))
        out.append((i, N, B, H, D, dtype, base2, out_f32))
    return out


def _result_dtype(dtype, out_f32):
    return "f32" if out_f32 or dtype == "f32" else dtype


@pytest.mark.parametrize("case", _cases("combine", 80, 2024), ids=lambda c: f"c{c[0]}")
def test_sweep_combine(lsec, case):
    i, N, B, H, D, dtype, base2, out_f32 = case
    print(f"[case] combine {case}", flush=True)
    o, l = synth.custom_inputs(N, B, H, D, dtype=dtype, seed=1000 + i, special=SPECIALS)
    y, L = lsec.lsec_combine(to_dev(o, dtype, DEV), f32_to_dev(l, DEV), base_e=not base2,
                             return_lse=True, out_dtype=torch.float32 if out_f32 else None)
    torch.cuda.synchronize()
    y_ref, L_ref = oracle.lse_combine(o, l, dtype, base2)
    assert_output_close(y, y_ref, _result_dtype(dtype, out_f32), max_abs_input(o, dtype))
    assert_lse_close(L, L_ref)


@pytest.mark.parametrize("case", _cases("merge", 32, 77), ids=lambda c: f"m{c[0]}")
def test_sweep_merge_and_planes(lsec, case):
    i, N, A, C, D, dtype, base2, out_f32 = case
    print(f"[case] merge/planes {case}", flush=True)
    o, l = synth.custom_inputs(N, A, C, D, dtype=dtype, seed=2000 + i, special=SPECIALS)
    odt = torch.float32 if out_f32 else None
    rdt = _result_dtype(dtype, out_f32)
    M = max_abs_input(o, dtype)
    token_dim = 1 + (i % 2)
    y, L = lsec.lsec_merge(to_dev(o, dtype, DEV), f32_to_dev(l, DEV), token_dim,
                           base_e=not base2, return_lse=True, out_dtype=odt)
    torch.cuda.synchronize()
    y_ref, L_ref = oracle.merge(o, l, dtype, token_dim, base2)
    assert_output_close(y, y_ref, rdt, M, "merge")
    assert_lse_close(L, L_ref, "merge")
    # the first T of A tokens of each plane, read in place from longer planes
    T = max(0, A - 1 - (i % 3))
    buf = torch.full((N, A + 3, C, D), float("nan"), dtype=TDT[dtype], device=DEV)
    lbuf = torch.full((N, A + 3, C), float("nan"), device=DEV)
    buf[:, :A] = to_dev(o, dtype, DEV)
    lbuf[:, :A] = f32_to_dev(l, DEV)
    y2, L2 = lsec.lsec_combine_planes(buf, lbuf, T, base_e=not base2, return_lse=True,
                                      out_dtype=odt)
    torch.cuda.synchronize()
    if T:
        y2_ref, L2_ref = oracle.lse_combine(np.ascontiguousarray(o[:, :T]),
                                            np.ascontiguousarray(l[:, :T]), dtype, base2)
        assert_output_close(y2, y2_ref, rdt, M, "planes")
        assert_lse_close(L2, L2_ref, "planes")
    # the same planes with the valid count in device memory (capacity A)
    Tv = (7 * i) % (A + 2) - 1  # -1 .. A
    qsl = np.array([0, max(Tv, 0) // 2, Tv], dtype=np.int32)
    y3 = torch.full((A, C, D), -3.0, dtype=TDT[rdt], device=DEV)
    L3 = torch.full((A, C), -3.0, device=DEV)
    lsec.lsec_combine_planes(buf, lbuf, A, base_e=not base2, return_lse=True, out=y3,
                             out_lse=L3, out_dtype=odt, query_start_loc=torch.from_numpy(qsl).to(DEV))
    torch.cuda.synchronize()
    y3_ref, L3_ref, tv = oracle.lse_combine_valid(o, l, qsl, dtype, base2)
    if tv:
        assert_output_close(y3[:tv], y3_ref, rdt, M, "planes_valid")
        assert_lse_close(L3[:tv], L3_ref, "planes_valid")
    assert bool(torch.all(y3[tv:] == -3.0)) and bool(torch.all(L3[tv:] == -3.0)), "padding written"


@pytest.mark.parametrize("case", _cases("packed", 40, 555), ids=lambda c: f"p{c[0]}")
def test_sweep_pack_exchange_unpack(lsec, case):
    i, N, B, Hl, D, dtype, base2, out_f32 = case
    H = N * Hl
    print(f"[case] pack/unpack {case}", flush=True)
    outs, lses = [], []
    for r in range(N):
        a, b = synth.custom_inputs(1, B, H, D, dtype=dtype, seed=3000 + 50 * i + r,
                                   special=SPECIALS)
        outs.append(a[0])
        lses.append(b[0])
    p = i % N
    # GPU pack of every rank, bit-exact with the oracle; rank p's receive buffer
    sends = []
    for r in range(N):
        s = lsec.lsec_pack_send(to_dev(outs[r], dtype, DEV), f32_to_dev(lses[r], DEV), N)
        torch.cuda.synchronize()
        assert np.array_equal(elem_bits_of(s, dtype), oracle.pack_send(outs[r], lses[r], N, dtype))
        sends.append(s)
    recv_h = oracle.exchange([oracle.pack_send(outs[r], lses[r], N, dtype) for r in range(N)])[p]
    recv = torch.stack([sends[r][p] for r in range(N)]).contiguous()
    assert np.array_equal(elem_bits_of(recv, dtype), recv_h)
    uo, ul = lsec.lsec_unpack(recv)
    y, L = lsec.lsec_unpack_combine(recv, base_e=not base2, return_lse=True,
                                    out_dtype=torch.float32 if out_f32 else None)
    torch.cuda.synchronize()
    oo, ol = oracle.unpack(recv_h, D, dtype)
    assert np.array_equal(elem_bits_of(uo, dtype), oo)
    assert np.array_equal(f32_bits_of(ul), ol.view(np.uint32))
    y_ref, L_ref = oracle.unpack_combine(recv_h, D, dtype, base2)
    assert_output_close(y, y_ref, _result_dtype(dtype, out_f32), max_abs_input(oo, dtype))
    assert_lse_close(L, L_ref)


@pytest.mark.parametrize("case", _cases("correct", 32, 99), ids=lambda c: f"r{c[0]}")
def test_sweep_correct_partial(lsec, case):
    i, N, B, H, D, dtype, base2, out_f32 = case
    print(f"[case] correct_partial {case}", flush=True)
    o, l = synth.custom_inputs(N, B, H, D, dtype=dtype, seed=4000 + i, special=SPECIALS)
    r = (7 * i) % N
    y, L = lsec.lsec_correct_partial(f32_to_dev(l, DEV), r, to_dev(o[r], dtype, DEV),
                                     base_e=not base2, return_lse=True,
                                     out_dtype=torch.float32 if out_f32 else None)
    torch.cuda.synchronize()
    y_ref, L_ref = oracle.correct_partial(l, r, o[r], dtype, base2)
    assert_output_close(y, y_ref, _result_dtype(dtype, out_f32), max_abs_input(o[r], dtype))
    assert_lse_close(L, L_ref)
