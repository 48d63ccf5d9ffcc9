"""GPU parity for fp32 elements and fp32 results, against the CPU oracle.

fp32 partial outputs travel in a packed row of D + 1 fp32 elements (the LSE
is the tail element); 16-bit partial outputs can be combined into an fp32
result (``out_dtype=torch.float32``), the dtype the page's CPU function
`_lse_weighted_combine` promotes bf16 / fp16 products with fp32 weights to.
Tolerances are those of gpu_helpers, chosen by the dtype of the result.
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
F32 = torch.float32
SPECIALS = ((0.04, float("nan")), (0.04, float("inf")), (0.04, float("-inf")))


@pytest.fixture(scope="module")
def lsec():
    import lse_weighted_merge_combine_amd as m
    if not os.path.exists(m.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    m.load_library()
    return m


def _announce(msg):
    print(f"[case] {msg}", flush=True)


def _inputs(N, B, H, D, dtype, seed):
    return synth.custom_inputs(N, B, H, D, dtype=dtype, seed=seed, special=SPECIALS)


# ---------------------------------------------------------------- fp32 partial outputs

F32_SHAPES = [
    # N, B, H, D, base2          (path)
    (16, 37, 5, 128, False),     # tiled S=1, 32 lanes per row
    (8, 29, 3, 512, True),       # tiled S=1, a row spans two waves
    (4, 23, 6, 256, True),       # tiled S=1, one wave per row
    (2, 31, 7, 64, False),       # row kernel, 16 lanes per row
    (1, 50, 3, 512, False),      # row kernel, N = 1
    (3, 11, 7, 128, True),       # tiled S=1, N at run time
    (9, 20, 2, 12, True),        # row kernel, 3 lanes per row
    (32, 6, 4, 128, False),      # row kernel, runtime N > 16
    (2, 3, 3, 1024, False),      # row kernel, 256 lanes per row
    (4, 10, 3, 1000, False),     # row kernel, 250 lanes per row
    (3, 5, 2, 3, True),          # element kernel: D % 4 != 0
    (2, 2, 2, 2048, True),       # element kernel: D / 4 > 256
]


@pytest.mark.parametrize("N,B,H,D,base2", F32_SHAPES)
def test_combine_f32_shapes(lsec, N, B, H, D, base2):
    _announce(f"combine f32 N={N} B={B} H={H} D={D} base2={base2}")
    o, l = _inputs(N, B, H, D, "f32", N * 1000 + D + 1)
    assert o.dtype == np.float32
    y, L = lsec.lsec_combine(to_dev(o, "f32", DEV), f32_to_dev(l, DEV), base_e=not base2,
                             return_lse=True)
    torch.cuda.synchronize()
    assert y.dtype == F32
    y_ref, L_ref = oracle.lse_combine(o, l, "f32", base2)
    assert_output_close(y, y_ref, "f32", max_abs_input(o, "f32"))
    assert_lse_close(L, L_ref)


TILED_F32 = [
    # N, B, H, D, base2, slots     (rows)
    (2, 8197, 32, 128, False, 16),  # 262304 rows
    (2, 2081, 32, 512, True, 16),   # 66592 rows, a row spans two waves
    (4, 3001, 33, 256, False, 8),   # 99033 rows, one wave per row
    (2, 2051, 17, 512, False, 8),   # 34867 rows
    (8, 3125, 31, 128, True, 4),    # 96875 rows
    (8, 1250, 31, 128, False, 2),   # 38750 rows
    (2, 1000, 3, 128, True, 1),     # 3000 rows
    (12, 3000, 16, 256, False, 4),  # 48000 rows, N at run time
    (5, 2051, 17, 512, True, 8),    # 34867 rows, N at run time, a row spans two waves
]


@pytest.mark.parametrize("N,B,H,D,base2,slots", TILED_F32)
def test_tiled_f32_slots_ragged(lsec, N, B, H, D, base2, slots):
    _announce(f"tiled combine f32 N={N} B={B} H={H} D={D} base2={base2} S={slots}")
    assert lsec.lsec_combine_path(N, B, H, D, dtype=F32) == f"combine_tiled_kernel S={slots}"
    o, l = _inputs(N, B, H, D, "f32", B + D + 3)
    y, L = lsec.lsec_combine(to_dev(o, "f32", DEV), f32_to_dev(l, DEV), base_e=not base2,
                             return_lse=True)
    torch.cuda.synchronize()
    y_ref, L_ref = oracle.lse_combine(o, l, "f32", base2)
    assert_output_close(y, y_ref, "f32", max_abs_input(o, "f32"))
    assert_lse_close(L, L_ref)


# ---------------------------------------------------------------- fp32 results from 16-bit inputs

OUT_F32 = [
    # N, B, H, D, dtype, base2, path
    (2, 16389, 32, 128, "bf16", False, "combine_tiled_kernel S=16"),
    (2, 2081, 63, 512, "bf16", True, "combine_tiled_kernel S=16"),
    (4, 4099, 32, 128, "f16", False, "combine_tiled_kernel S=4"),
    (8, 1250, 31, 128, "bf16", True, "combine_tiled_kernel S=1"),
    (3, 11, 7, 128, "f16", True, "combine_tiled_kernel S=1"),   # N at run time
    (20, 11, 7, 128, "f16", True, "combine_rows_kernel"),       # N > 16
    (9, 20, 2, 24, "bf16", False, "combine_rows_kernel"),
    (1, 37, 5, 128, "bf16", False, "combine_rows_kernel"),      # N = 1
    (5, 19, 3, 64, "f16", True, "combine_rows_kernel"),         # N at run time, D = 64
    (16, 9, 4, 1024, "bf16", False, "combine_rows_kernel"),     # 128 lanes per row
    (2, 5, 3, 2048, "bf16", True, "combine_rows_kernel"),       # 256 lanes per row
    (4, 10, 3, 1004, "bf16", True, "combine_elems_kernel"),
]


@pytest.mark.parametrize("N,B,H,D,dtype,base2,path", OUT_F32)
def test_combine_fp32_result_from_16bit(lsec, N, B, H, D, dtype, base2, path):
    _announce(f"combine {dtype} -> f32 N={N} B={B} H={H} D={D} base2={base2}")
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float16
    assert lsec.lsec_combine_path(N, B, H, D, dtype=tdt, out_dtype=F32) == path
    o, l = _inputs(N, B, H, D, dtype, B * 3 + D)
    y, L = lsec.lsec_combine(to_dev(o, dtype, DEV), f32_to_dev(l, DEV), base_e=not base2,
                             return_lse=True, out_dtype=F32)
    torch.cuda.synchronize()
    assert y.dtype == F32
    y_ref, L_ref = oracle.lse_combine(o, l, dtype, base2)
    assert_output_close(y, y_ref, "f32", max_abs_input(o, dtype))
    assert_lse_close(L, L_ref)


def test_fp32_result_is_the_unrounded_16bit_result(lsec):
    """The 16-bit result is the fp32 result rounded to nearest even, bit for bit
    (same kernel, same accumulation order; only the final store differs)."""
    N, B, H, D = 8, 64, 16, 128
    _announce("bf16 result == round(f32 result)")
    o, l = _inputs(N, B, H, D, "bf16", 21)
    og, lg = to_dev(o, "bf16", DEV), f32_to_dev(l, DEV)
    y16 = lsec.lsec_combine(og, lg)
    y32 = lsec.lsec_combine(og, lg, out_dtype=F32)
    torch.cuda.synchronize()
    assert torch.equal(y32.to(torch.bfloat16).view(torch.int16), y16.view(torch.int16))


@pytest.mark.parametrize("N,D", [(20, 128), (1, 64), (3, 24)])
def test_row_kernel_fp32_result_rounds_to_its_16bit_result(lsec, N, D):
    """The row kernel's fp32 result (split loads: a lane owns two quarter-rows)
    rounded to bf16 equals its bf16 result bit for bit: each element is
    accumulated over the planes in the same order either way."""
    B, H = 33, 6
    _announce(f"row kernel bf16 == round(f32) N={N} D={D}")
    assert lsec.lsec_combine_path(N, B, H, D, out_dtype=F32) == "combine_rows_kernel"
    o, l = _inputs(N, B, H, D, "bf16", 31 + N + D)
    og, lg = to_dev(o, "bf16", DEV), f32_to_dev(l, DEV)
    y16 = lsec.lsec_combine(og, lg)
    y32 = lsec.lsec_combine(og, lg, out_dtype=F32)
    torch.cuda.synchronize()
    assert torch.equal(y32.to(torch.bfloat16).view(torch.int16), y16.view(torch.int16))


@pytest.mark.parametrize("N,B,H,D", [(20, 9, 40, 128), (4, 7, 8, 64)])
def test_row_kernel_unpack_combine_fp32_result(lsec, N, B, H, D):
    """Packed rows (4-byte aligned) through the row kernel with an fp32 result."""
    _announce(f"row kernel unpack_combine bf16 -> f32 N={N} B={B} H={H} D={D}")
    assert lsec.lsec_combine_path(N, B, H // N, D, packed=True, out_dtype=F32) == \
        "combine_rows_kernel"
    outs, lses = [], []
    for r in range(N):
        a, b = _inputs(1, B, H, D, "bf16", 950 + r)
        outs.append(a[0])
        lses.append(b[0])
    recv_h = oracle.exchange([oracle.pack_send(outs[r], lses[r], N) for r in range(N)])[0]
    y, L = lsec.lsec_unpack_combine(to_dev(recv_h, "bf16", DEV), return_lse=True, out_dtype=F32)
    torch.cuda.synchronize()
    y_ref, L_ref = oracle.unpack_combine(recv_h, D, "bf16")
    oo, _ = oracle.unpack(recv_h, D)
    assert_output_close(y, y_ref, "f32", max_abs_input(oo, "bf16"))
    assert_lse_close(L, L_ref)


def test_page_alias_returns_promoted_fp32(lsec):
    o, l = synth.custom_inputs(3, 4, 4, 64, seed=13)
    y, L = lsec.lse_weighted_combine(to_dev(o, "bf16", DEV), f32_to_dev(l, DEV), return_lse=True,
                                     is_lse_base_on_e=False)
    torch.cuda.synchronize()
    assert y.dtype == F32
    y_ref, L_ref = oracle.lse_combine(o, l, "bf16", base2=True)
    assert_output_close(y, y_ref, "f32", max_abs_input(o, "bf16"))
    assert_lse_close(L, L_ref)


# ---------------------------------------------------------------- packed fp32 rows (P = 1)

@pytest.mark.parametrize("N,B,H,D", [
    (4, 9, 8, 128), (2, 7, 6, 64), (8, 3, 16, 512),
    (4, 5, 8, 6),     # general path: D % 4 != 0
    (2, 5, 4, 5),     # odd D
    (3, 4, 9, 132),   # fast path, 33 lanes per row
])
def test_pack_unpack_f32(lsec, N, B, H, D):
    _announce(f"pack/unpack f32 N={N} B={B} H={H} D={D}")
    o, l = _inputs(1, B, H, D, "f32", 77 + D)
    o, l = o[0], l[0]
    l.view(np.uint32)[0, 0] = 0x7FC0BEEF  # NaN payload must survive
    o.view(np.uint32)[0, 0, 0] = 0x7FA00001  # signalling-NaN pattern in the data, too
    send = lsec.lsec_pack_send(to_dev(o, "f32", DEV), f32_to_dev(l, DEV), N)
    torch.cuda.synchronize()
    assert tuple(send.shape) == (N, B, H // N, D + 1)
    ref = oracle.pack_send(o, l, N, dtype="f32")
    assert np.array_equal(elem_bits_of(send, "f32"), ref)
    uo, ul = lsec.lsec_unpack(to_dev(ref, "f32", DEV))
    torch.cuda.synchronize()
    oo, ol = oracle.unpack(ref, D, dtype="f32")
    assert np.array_equal(elem_bits_of(uo, "f32"), oo)
    assert np.array_equal(f32_bits_of(ul), ol.view(np.uint32))
    y, L = lsec.lsec_unpack_combine(to_dev(ref, "f32", DEV), base_e=True, return_lse=True)
    torch.cuda.synchronize()
    y_ref, L_ref = oracle.unpack_combine(ref, D, "f32", False)
    assert_output_close(y, y_ref, "f32", max_abs_input(oo, "f32"))
    assert_lse_close(L, L_ref)


@pytest.mark.parametrize("N,B,H,D,slots", [
    (4, 8193, 16, 128, 2),    # 32772 rows of the packed layout, ragged
    (2, 4097, 32, 512, 16),   # 65552 rows, a row spans two waves
    (8, 4099, 64, 256, 4),    # 32792 rows, one wave per row
])
def test_tiled_unpack_combine_f32(lsec, N, B, H, D, slots):
    _announce(f"tiled unpack_combine f32 N={N} B={B} H={H} D={D} S={slots}")
    assert lsec.lsec_combine_path(N, B, H // N, D, packed=True, dtype=F32) == \
        f"combine_tiled_kernel S={slots}"
    outs, lses = [], []
    for r in range(N):
        a, b = _inputs(1, B, H, D, "f32", 600 + r)
        outs.append(a[0])
        lses.append(b[0])
    recv_h = oracle.exchange([oracle.pack_send(outs[r], lses[r], N, dtype="f32")
                              for r in range(N)])[1]
    y, L = lsec.lsec_unpack_combine(to_dev(recv_h, "f32", DEV), base_e=False, return_lse=True)
    torch.cuda.synchronize()
    y_ref, L_ref = oracle.unpack_combine(recv_h, D, "f32", True)
    oo, _ = oracle.unpack(recv_h, D, dtype="f32")
    assert_output_close(y, y_ref, "f32", max_abs_input(oo, "f32"))
    assert_lse_close(L, L_ref)


@pytest.mark.parametrize("N,B,Hl,base2,return_lse", [
    (2, 6, 2, False, True),       # 12 rows: three spans, one partial block
    (4, 1027, 4, True, True),     # 4108 rows: 1027 spans, the last block partial
    (8, 2048, 8, False, True),    # the packed_f32 workload's receive side
    (8, 4101, 4, False, False),   # 16404 rows, no global LSE
    (16, 257, 4, True, True),     # N = 16
])
def test_span32_unpack_combine(lsec, N, B, Hl, base2, return_lse):
    """Packed rows of 128 fp32 values in whole spans of four: the fp32 span
    kernel (aligned chunk loads, the LSEs taken from them, realigned stores)."""
    D, H = 128, N * Hl
    _announce(f"span32 unpack_combine N={N} B={B} Hl={Hl} base2={base2}")
    assert lsec.lsec_combine_path(N, B, Hl, D, packed=True, dtype=F32) == "combine_span32_kernel"
    outs, lses = [], []
    for r in range(N):
        a, b = synth.custom_inputs(1, B, H, D, dtype="f32", seed=1900 + 31 * N + r,
                                   special=SPECIALS)
        outs.append(a[0])
        lses.append(b[0])
    recv_h = oracle.exchange([oracle.pack_send(outs[r], lses[r], N, dtype="f32")
                              for r in range(N)])[N - 1]
    res = lsec.lsec_unpack_combine(to_dev(recv_h, "f32", DEV), base_e=not base2,
                                   return_lse=return_lse)
    torch.cuda.synchronize()
    y, L = res if return_lse else (res, None)
    y_ref, L_ref = oracle.unpack_combine(recv_h, D, "f32", base2)
    oo, _ = oracle.unpack(recv_h, D, dtype="f32")
    assert_output_close(y, y_ref, "f32", max_abs_input(oo, "f32"))
    if return_lse:
        assert_lse_close(L, L_ref)


@pytest.mark.parametrize("N,B,H", [(8, 64, 16), (16, 37, 64), (2, 1030, 4)])
def test_span32_matches_the_tiled_kernel_bit_for_bit(lsec, N, B, H):
    """The same fp32 receive buffer 4 bytes past a 16-byte boundary takes the
    tiled kernel, the aligned one the span kernel; both weight and sum the
    planes in the same order, so the results agree bit for bit."""
    D = 128
    _announce(f"span32 vs tiled N={N} B={B} H={H}")
    assert lsec.lsec_combine_path(N, B, H // N, D, packed=True, dtype=F32) == \
        "combine_span32_kernel"
    outs, lses = [], []
    for r in range(N):
        a, b = synth.custom_inputs(1, B, H, D, dtype="f32", seed=1760 + r, special=SPECIALS)
        outs.append(a[0])
        lses.append(b[0])
    recv_h = oracle.exchange([oracle.pack_send(outs[r], lses[r], N, dtype="f32")
                              for r in range(N)])[1]
    flat = torch.empty(recv_h.size + 4, dtype=F32, device=DEV)
    shifted = flat[1:1 + recv_h.size].view(recv_h.shape)
    shifted.copy_(to_dev(recv_h, "f32", DEV))
    assert shifted.data_ptr() % 16 == 4
    y1, L1 = lsec.lsec_unpack_combine(shifted, return_lse=True)
    y2, L2 = lsec.lsec_unpack_combine(to_dev(recv_h, "f32", DEV), return_lse=True)
    torch.cuda.synchronize()
    y_ref, L_ref = oracle.unpack_combine(recv_h, D, "f32")
    oo, _ = oracle.unpack(recv_h, D, dtype="f32")
    for y, L in ((y1, L1), (y2, L2)):
        assert_output_close(y, y_ref, "f32", max_abs_input(oo, "f32"))
        assert_lse_close(L, L_ref)
    assert torch.equal(y1.view(torch.int32), y2.view(torch.int32))
    assert torch.equal(L1.view(torch.int32), L2.view(torch.int32))


def test_f32_exchange_on_the_gpu(lsec):
    """4 ranks pack fp32 outputs on the GPU, the all-to-all is a host-side
    placement, and each receiver's unpack_combine matches the oracle's
    combine of its head slice."""
    N, B, H, D = 4, 33, 16, 128
    _announce("f32 pack -> exchange -> unpack_combine")
    outs, lses = [], []
    for r in range(N):
        a, b = _inputs(1, B, H, D, "f32", 700 + r)
        outs.append(a[0])
        lses.append(b[0])
    sends = [lsec.lsec_pack_send(to_dev(outs[r], "f32", DEV), f32_to_dev(lses[r], DEV), N)
             for r in range(N)]
    Hl = H // N
    so, sl = np.stack(outs), np.stack(lses)
    for p in range(N):
        recv = torch.stack([sends[r][p] for r in range(N)]).contiguous()
        y, L = lsec.lsec_unpack_combine(recv, return_lse=True)
        torch.cuda.synchronize()
        sh = slice(p * Hl, (p + 1) * Hl)
        y_ref, L_ref = oracle.lse_combine(so[:, :, sh], sl[:, :, sh], "f32")
        assert_output_close(y, y_ref, "f32", max_abs_input(so, "f32"), f"rank {p}")
        assert_lse_close(L, L_ref, f"rank {p}")


def test_unpack_combine_fp32_result_from_bf16(lsec):
    N, B, H, D = 8, 2051, 64, 128
    _announce("unpack_combine bf16 -> f32")
    outs, lses = [], []
    for r in range(N):
        a, b = _inputs(1, B, H, D, "bf16", 800 + r)
        outs.append(a[0])
        lses.append(b[0])
    recv_h = oracle.exchange([oracle.pack_send(outs[r], lses[r], N) for r in range(N)])[2]
    y, L = lsec.lsec_unpack_combine(to_dev(recv_h, "bf16", DEV), return_lse=True, out_dtype=F32)
    torch.cuda.synchronize()
    assert y.dtype == F32
    y_ref, L_ref = oracle.unpack_combine(recv_h, D, "bf16")
    oo, _ = oracle.unpack(recv_h, D)
    assert_output_close(y, y_ref, "f32", max_abs_input(oo, "bf16"))
    assert_lse_close(L, L_ref)


# ---------------------------------------------------------------- merge and corrected partials

@pytest.mark.parametrize("N,A,C,D,dtype,token_dim,out_f32", [
    (8, 8, 2048, 128, "f32", 2, True),     # tiled, transposed store
    (4, 64, 33, 256, "f32", 1, True),
    (16, 4, 1031, 128, "bf16", 2, True),   # fp32 result from bf16
    (3, 5, 77, 64, "f16", 2, True),        # row kernel
    (2, 7, 13, 10, "f32", 2, True),        # element kernel
])
def test_merge_f32(lsec, N, A, C, D, dtype, token_dim, out_f32):
    _announce(f"merge {dtype} -> f32 N={N} A={A} C={C} D={D} token_dim={token_dim}")
    o, l = _inputs(N, A, C, D, dtype, A * 17 + C)
    y, L = lsec.lsec_merge(to_dev(o, dtype, DEV), f32_to_dev(l, DEV), token_dim,
                           return_lse=True, out_dtype=F32 if out_f32 else None)
    torch.cuda.synchronize()
    assert y.dtype == F32
    y_ref, L_ref = oracle.merge(o, l, dtype, token_dim)
    assert tuple(y.shape) == y_ref.shape
    assert_output_close(y, y_ref, "f32", max_abs_input(o, dtype))
    assert_lse_close(L, L_ref)


@pytest.mark.parametrize("N,B,H,D,dtype,base2", [
    (8, 2048, 16, 512, "f32", True),    # tiled, a row spans two waves
    (16, 500, 32, 128, "f32", False),   # tiled
    (4, 1000, 8, 256, "bf16", True),    # fp32 result from bf16, tiled
    (4, 33, 3, 64, "f32", False),       # element kernel
    (20, 9, 4, 128, "f16", True),       # element kernel (N > 16), fp32 result
])
def test_correct_partial_f32(lsec, N, B, H, D, dtype, base2):
    _announce(f"correct_partial {dtype} -> f32 N={N} B={B} H={H} D={D}")
    o, l = _inputs(N, B, H, D, dtype, N * 5 + D)
    lg = f32_to_dev(l, DEV)
    M = max_abs_input(o, dtype)
    total = torch.zeros((B, H, D), dtype=torch.float64, device=DEV)
    for r in range(N):
        y, L = lsec.lsec_correct_partial(lg, r, to_dev(o[r], dtype, DEV), base_e=not base2,
                                         return_lse=True, out_dtype=F32)
        assert y.dtype == F32
        total += y.double()
        if r in (0, N - 1):
            torch.cuda.synchronize()
            y_ref, L_ref = oracle.correct_partial(l, r, o[r], dtype, base2)
            assert_output_close(y, y_ref, "f32", max_abs_input(o[r], dtype), f"rank {r}")
            assert_lse_close(L, L_ref, f"rank {r}")
    torch.cuda.synchronize()
    # summed in fp64 over ranks, the fp32 corrected partials give the combine
    y_all, _ = oracle.lse_combine(o, l, dtype, base2)
    fin = np.isfinite(y_all)
    err = float(np.abs(total.cpu().numpy() - y_all)[fin].max())
    assert err <= 2 * 2e-5 * M + 1e-6


# ---------------------------------------------------------------- degenerate cases

@pytest.mark.parametrize("base_e", [True, False])
def test_single_shard_f32_identity(lsec, base_e):
    o, l = synth.custom_inputs(1, 33, 7, 128, dtype="f32", seed=8)
    y, L = lsec.lsec_combine(to_dev(o, "f32", DEV), f32_to_dev(l, DEV), base_e=base_e,
                             return_lse=True)
    torch.cuda.synchronize()
    assert np.array_equal(f32_bits_of(y), o[0].view(np.uint32))
    assert np.array_equal(f32_bits_of(L), l[0].view(np.uint32))
    # 16-bit input with an fp32 result: the exact widening of the input
    ob, lb = synth.custom_inputs(1, 9, 5, 64, dtype="bf16", seed=9)
    y2 = lsec.lsec_combine(to_dev(ob, "bf16", DEV), f32_to_dev(lb, DEV), out_dtype=F32)
    torch.cuda.synchronize()
    assert np.array_equal(y2.cpu().numpy().astype(np.float64), oracle.bits_to_f64(ob[0], "bf16"))


def test_all_shards_non_finite_f32(lsec):
    N, B, H, D = 4, 5, 3, 128
    o, _ = synth.custom_inputs(N, B, H, D, dtype="f32", seed=9)
    l = np.empty((N, B, H), dtype=np.float32)
    l[0], l[1], l[2], l[3] = np.nan, np.inf, -np.inf, np.nan
    for D_ in (128, 10):  # fast and general paths
        oo = np.ascontiguousarray(o[..., :D_])
        y, L = lsec.lsec_combine(to_dev(oo, "f32", DEV), f32_to_dev(l, DEV), return_lse=True)
        torch.cuda.synchronize()
        assert torch.all(y == 0)
        assert torch.all(torch.isneginf(L))


def test_misaligned_f32_views(lsec):
    """fp32 views that start 4 bytes into an allocation (element-aligned only)."""
    N, B, H, D = 4, 6, 5, 128
    _announce("misaligned f32 views")
    o, l = _inputs(N, B, H, D, "f32", 5)
    flat = torch.empty(o.size + 1, dtype=F32, device=DEV)
    og = flat[1:].view(N, B, H, D)
    og.copy_(to_dev(o, "f32", DEV))
    outflat = torch.empty(B * H * D + 1, dtype=F32, device=DEV)
    out = outflat[1:].view(B, H, D)
    y = lsec.lsec_combine(og, f32_to_dev(l, DEV), out=out)
    torch.cuda.synchronize()
    y_ref, _ = oracle.lse_combine(o, l, "f32")
    assert_output_close(y, y_ref, "f32", max_abs_input(o, "f32"))
    # bf16 inputs, fp32 result into a view 4 bytes in
    ob, lb = _inputs(N, B, H, D, "bf16", 6)
    y2 = lsec.lsec_combine(to_dev(ob, "bf16", DEV), f32_to_dev(lb, DEV), out=out, out_dtype=F32)
    torch.cuda.synchronize()
    y2_ref, _ = oracle.lse_combine(ob, lb, "bf16")
    assert_output_close(y2, y2_ref, "f32", max_abs_input(ob, "bf16"))


def test_f32_errors(lsec):
    with pytest.raises(ValueError):  # fp32 result cannot be requested as fp16
        lsec.lsec_combine(torch.zeros(2, 1, 1, 8, dtype=F32, device=DEV),
                          torch.zeros(2, 1, 1, device=DEV), out_dtype=torch.float16)
    with pytest.raises(ValueError):  # an fp32 output buffer needs out_dtype
        lsec.lsec_combine(torch.zeros(2, 1, 1, 8, dtype=torch.bfloat16, device=DEV),
                          torch.zeros(2, 1, 1, device=DEV),
                          out=torch.zeros(1, 1, 8, dtype=F32, device=DEV))
