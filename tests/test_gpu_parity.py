"""GPU parity: the HIP kernels (through the C ABI) against the CPU oracle.

Inputs come from the seeded generator; expected values come from the oracle
only. Combined outputs are compared within the tolerances in gpu_helpers;
pack / unpack are compared bit for bit.
"""
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import (assert_combine_close_in_chunks, assert_lse_close, assert_output_close,
                         bits_of, elem_bits_of, f32_bits_of, f32_to_dev, max_abs_input, to_dev)

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
TDT = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}


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


def test_native_library_loaded(lsec):
    maps = open("/proc/self/maps").read()
    assert "liblsec.so" in maps
    assert torch.cuda.is_available()


# ---------------------------------------------------------------- workloads at full size

@pytest.mark.parametrize("name", ["small", "fp16_base2", "mla_decode"])
@pytest.mark.parametrize("return_lse", [False, True])
def test_workload_full(lsec, name, return_lse):
    w = synth.WORKLOADS[name]
    _announce(f"{name} full N={w.N} B={w.B} H={w.H} D={w.D} return_lse={return_lse}")
    o, l = synth.combine_inputs(w)
    res = lsec.lsec_combine(to_dev(o, w.dtype, DEV), f32_to_dev(l, DEV), base_e=not w.base2,
                            return_lse=return_lse)
    torch.cuda.synchronize()
    y_ref, L_ref = oracle.lse_combine(o, l, w.dtype, base2=w.base2)
    M = max_abs_input(o, w.dtype)
    if return_lse:
        y, L = res
        assert_lse_close(L, L_ref, name)
    else:
        y = res
    assert_output_close(y, y_ref, w.dtype, M, name)
    if name == "small":  # the all -inf row gives 0 and -inf
        b, h = w.allneg_row
        assert torch.all(y[b, h] == 0)
        if return_lse:
            assert L[b, h].item() == float("-inf")


def test_large_batch_full_size(lsec):
    """N=16 B=16384 H=32 D=128 bf16, the launch the benchmark times (the tiled
    kernel with 16 slots): all 524,288 rows against the oracle, element by
    element, with the global LSE."""
    w = synth.WORKLOADS["large_batch"]
    _announce("large_batch full size, every row")
    assert lsec.lsec_combine_path(w.N, w.B, w.H, w.D) == "combine_tiled_kernel S=16"
    o, l = synth.combine_inputs(w)
    M = max_abs_input(o, w.dtype)
    y, L = lsec.lsec_combine(to_dev(o, w.dtype, DEV), f32_to_dev(l, DEV), base_e=True,
                             return_lse=True)
    torch.cuda.synchronize()
    assert_combine_close_in_chunks(y, L, o, l, w.dtype, False, M, what="large_batch")


def _packed_ranks(w, b_lo=0, b_hi=None):
    outs, lses = [], []
    for r in range(w.N):
        a, b = synth.rank_inputs(w, r, b_lo=b_lo, b_hi=b_hi)
        outs.append(a)
        lses.append(b)
    return outs, lses


def test_packed_workload_full(lsec):
    """8 ranks x [2048,64,128] bf16: GPU pack on every rank (bit-exact with the
    oracle), all-to-all stand-in, GPU unpack+combine on every receiving rank."""
    w = synth.WORKLOADS["packed"]
    _announce("packed full: 8 ranks pack, exchange, unpack_combine")
    outs, lses = _packed_ranks(w)
    Hl = w.H // w.N
    sends = []
    for r in range(w.N):
        s = lsec.lsec_pack_send(to_dev(outs[r], w.dtype, DEV), f32_to_dev(lses[r], DEV), w.N)
        torch.cuda.synchronize()
        assert np.array_equal(bits_of(s), oracle.pack_send(outs[r], lses[r], w.N)), f"rank {r}"
        sends.append(s)
    so, sl = np.stack(outs), np.stack(lses)
    M = max_abs_input(so, w.dtype)
    for p in range(w.N):
        recv = torch.stack([sends[r][p] for r in range(w.N)]).contiguous()
        y, L = lsec.lsec_unpack_combine(recv, base_e=True, return_lse=True)
        uo, ul = lsec.lsec_unpack(recv)
        torch.cuda.synchronize()
        sl_h = slice(p * Hl, (p + 1) * Hl)
        y_ref, L_ref = oracle.lse_combine(so[:, :, sl_h], sl[:, :, sl_h], w.dtype, base2=False)
        assert_output_close(y, y_ref, w.dtype, M, f"recv rank {p}")
        assert_lse_close(L, L_ref, f"recv rank {p}")
        assert np.array_equal(bits_of(uo), np.ascontiguousarray(so[:, :, sl_h]))
        assert np.array_equal(f32_bits_of(ul), np.ascontiguousarray(sl[:, :, sl_h]).view(np.uint32))


@pytest.mark.parametrize("dtype,base2", [("bf16", False), ("f16", True)])
def test_receive_side_on_oracle_packed_buffer(lsec, dtype, base2):
    """The receive kernels on a buffer the oracle packed and exchanged on the host."""
    N, B, H, D = 4, 37, 12, 128
    _announce(f"receive side on oracle buffer {dtype} N={N} B={B} H={H} D={D}")
    outs, lses = [], []
    for r in range(N):
        a, b = synth.custom_inputs(1, B, H, D, dtype=dtype, seed=300 + r,
                                   special=((0.05, float("nan")), (0.05, float("inf")),
                                            (0.05, float("-inf"))))
        outs.append(a[0])
        lses.append(b[0])
    recvs = oracle.exchange([oracle.pack_send(outs[r], lses[r], N) for r in range(N)])
    for p in (0, 3):
        recv_h = recvs[p]
        recv = to_dev(recv_h, dtype, DEV)
        y, L = lsec.lsec_unpack_combine(recv, base_e=not base2, return_lse=True)
        uo, ul = lsec.lsec_unpack(recv)
        torch.cuda.synchronize()
        y_ref, L_ref = oracle.unpack_combine(recv_h, D, dtype, base2)
        oo, ol = oracle.unpack(recv_h, D)
        assert_output_close(y, y_ref, dtype, max_abs_input(oo, dtype), f"rank {p}")
        assert_lse_close(L, L_ref, f"rank {p}")
        assert np.array_equal(bits_of(uo), oo)
        assert np.array_equal(f32_bits_of(ul), ol.view(np.uint32))


# ---------------------------------------------------------------- shapes and code paths

SPECIALS = ((0.04, float("nan")), (0.04, float("inf")), (0.04, float("-inf")))

SHAPES = [
    # N, B, H, D, dtype, base2      (path exercised)
    (16, 37, 5, 128, "bf16", False),  # templated N, ragged last block
    (8, 29, 3, 512, "bf16", True),    # one wave per row
    (4, 23, 6, 256, "f16", True),
    (2, 31, 7, 64, "bf16", False),
    (1, 50, 3, 512, "bf16", False),
    (3, 11, 7, 128, "f16", True),     # tiled, N at run time
    (5, 9, 4, 64, "bf16", True),
    (7, 13, 3, 256, "bf16", False),   # tiled, N at run time
    (32, 6, 4, 128, "bf16", False),
    (100, 5, 3, 128, "f16", True),    # row kernel, N far above 16
    (257, 2, 2, 64, "bf16", False),   # row kernel, N = 257
    (9, 20, 2, 24, "bf16", True),     # 3 lanes per row, rows straddle waves
    (2, 3, 3, 2048, "f16", False),    # 256 lanes per row
    (4, 10, 3, 1000, "bf16", False),  # row kernel, 125 lanes per row
    (3, 5, 2, 3, "f16", True),        # general path: tiny D
    (2, 2, 2, 4096, "bf16", True),    # general path: D > 2048
]


@pytest.mark.parametrize("N,B,H,D,dtype,base2", SHAPES)
def test_combine_shapes(lsec, N, B, H, D, dtype, base2):
    _announce(f"combine N={N} B={B} H={H} D={D} {dtype} base2={base2}")
    o, l = synth.custom_inputs(N, B, H, D, dtype=dtype, seed=N * 1000 + D, special=SPECIALS)
    y, L = lsec.lsec_combine(to_dev(o, dtype, DEV), f32_to_dev(l, DEV), base_e=not base2,
                             return_lse=True)
    torch.cuda.synchronize()
    y_ref, L_ref = oracle.lse_combine(o, l, dtype, base2)
    assert_output_close(y, y_ref, dtype, max_abs_input(o, dtype))
    assert_lse_close(L, L_ref)


# Large enough for the tiled kernel to pick 16, 8, 4, 2 and 1 row slots per
# lane (the largest count that still gives 2048 blocks), each with a ragged
# last block (rows not a multiple of the block's rows).
TILED = [
    # N, B, H, D, dtype, base2, slots   (rows)
    (2, 16389, 32, 128, "bf16", False, 16),  # 524448 rows
    (2, 8197, 32, 256, "f16", True, 16),     # 262304 rows, two rows per wave
    (2, 2081, 63, 512, "bf16", True, 16),    # 131103 rows, one wave per row
    (2, 9001, 33, 128, "bf16", True, 8),     # 297033 rows
    (2, 8193, 17, 256, "bf16", False, 8),    # 139281 rows
    (4, 4099, 32, 128, "bf16", False, 4),    # 131168 rows
    (2, 2051, 17, 512, "f16", False, 4),     # 34867 rows
    (8, 3125, 31, 128, "bf16", False, 2),    # 96875 rows
    (8, 1250, 31, 128, "f16", True, 1),      # 38750 rows
    (2, 1000, 3, 128, "bf16", True, 1),      # 3000 rows
    # N at run time (2 < N < 16, not a power of two): the plane groups of N = 16
    # with the planes past N skipped
    (3, 16389, 32, 128, "bf16", False, 16),  # 524448 rows
    (6, 4099, 16, 512, "bf16", True, 8),     # 65584 rows, one wave per row
    (12, 8193, 16, 256, "f16", False, 8),    # 131088 rows, two rows per wave
    (7, 3125, 31, 128, "bf16", False, 2),    # 96875 rows, groups of 4 planes: 4 + 3
    (15, 1250, 31, 128, "bf16", True, 1),    # 38750 rows, groups of 8 planes: 8 + 7
    (5, 1000, 3, 128, "bf16", True, 1),      # 3000 rows
]


@pytest.mark.parametrize("N,B,H,D,dtype,base2,slots", TILED)
def test_tiled_slots_ragged(lsec, N, B, H, D, dtype, base2, slots):
    _announce(f"tiled combine N={N} B={B} H={H} D={D} {dtype} base2={base2} S={slots}")
    assert lsec.lsec_combine_path(N, B, H, D) == f"combine_tiled_kernel S={slots}"
    o, l = synth.custom_inputs(N, B, H, D, dtype=dtype, seed=B + D, special=SPECIALS)
    y, L = lsec.lsec_combine(to_dev(o, dtype, DEV), f32_to_dev(l, DEV), base_e=not base2,
                             return_lse=True)
    torch.cuda.synchronize()
    y_ref, L_ref = oracle.lse_combine(o, l, dtype, base2)
    assert_output_close(y, y_ref, dtype, max_abs_input(o, dtype))
    assert_lse_close(L, L_ref)


def test_tiled_n16_relaxed_block_count(lsec):
    """N=16 takes 16 slots down to 1024 blocks: 67551 rows of D=512 (1056
    blocks, ragged last block); every row against the oracle."""
    N, B, H, D = 16, 2047, 33, 512
    _announce(f"tiled combine N={N} B={B} H={H} D={D} bf16, every row")
    assert lsec.lsec_combine_path(N, B, H, D) == "combine_tiled_kernel S=16"
    w = synth.Workload("n16_d512", 90, "combine", N, B, H, D, "bf16", ("normal", 0.0, 1.0),
                       ("uniform", -10.0, 30.0), special=SPECIALS, base2=True)
    o, l = synth.combine_inputs(w)
    M = max_abs_input(o, "bf16")
    y, L = lsec.lsec_combine(to_dev(o, "bf16", DEV), f32_to_dev(l, DEV), base_e=False,
                             return_lse=True)
    torch.cuda.synchronize()
    assert_combine_close_in_chunks(y, L, o, l, "bf16", True, M, chunk_tokens=128,
                                   what="n16_d512")


@pytest.mark.parametrize("N,B,H,D,dtype,slots", [
    (4, 8193, 4, 128, "bf16", 1),    # 8193 rows of the packed layout, ragged (not whole spans)
    (8, 4099, 8, 128, "bf16", 1),    # 4099 rows
    (2, 4097, 32, 512, "f16", 8),    # 65552 rows
    (2, 16389, 64, 128, "bf16", 16),  # 524448 rows
    (5, 8193, 15, 128, "bf16", 1),    # 24579 rows, N at run time
    (6, 16389, 12, 512, "f16", 4),    # 32778 rows, N at run time
])
def test_tiled_unpack_combine_ragged(lsec, N, B, H, D, dtype, slots):
    _announce(f"tiled unpack_combine N={N} B={B} H={H} D={D} {dtype} S={slots}")
    assert lsec.lsec_combine_path(N, B, H // N, D, packed=True) == f"combine_tiled_kernel S={slots}"
    outs, lses = [], []
    for r in range(N):
        a, b = synth.custom_inputs(1, B, H, D, dtype=dtype, seed=500 + r, special=SPECIALS)
        outs.append(a[0])
        lses.append(b[0])
    recv_h = oracle.exchange([oracle.pack_send(outs[r], lses[r], N) for r in range(N)])[1]
    y, L = lsec.lsec_unpack_combine(to_dev(recv_h, dtype, DEV), base_e=True, return_lse=True)
    torch.cuda.synchronize()
    y_ref, L_ref = oracle.unpack_combine(recv_h, D, dtype, False)
    oo, _ = oracle.unpack(recv_h, D)
    assert_output_close(y, y_ref, dtype, max_abs_input(oo, dtype))
    assert_lse_close(L, L_ref)


@pytest.mark.parametrize("N,B,Hl,dtype,base2,return_lse", [
    (2, 6, 2, "bf16", False, True),      # 12 rows: three spans, one partial block
    (4, 1027, 4, "f16", True, True),     # 4108 rows: 1027 spans, the last block partial
    (8, 2048, 8, "bf16", False, True),   # the packed workload's receive side
    (8, 4101, 4, "f16", False, False),   # 16404 rows, no global LSE
    (16, 257, 4, "bf16", True, True),    # N = 16
])
def test_span_unpack_combine(lsec, N, B, Hl, dtype, base2, return_lse):
    """Packed rows of 128 16-bit values in whole spans of four: the span kernel
    (aligned chunk loads, the LSE tails taken from them, realigned stores)."""
    D, H = 128, N * Hl
    _announce(f"span unpack_combine N={N} B={B} Hl={Hl} {dtype} base2={base2}")
    assert lsec.lsec_combine_path(N, B, Hl, D, packed=True, dtype=TDT[dtype]) == \
        "combine_span_kernel"
    outs, lses = [], []
    for r in range(N):
        a, b = synth.custom_inputs(1, B, H, D, dtype=dtype, seed=900 + 31 * N + r,
                                   special=SPECIALS)
        outs.append(a[0])
        lses.append(b[0])
    recv_h = oracle.exchange([oracle.pack_send(outs[r], lses[r], N, dtype) for r in range(N)])[N - 1]
    res = lsec.lsec_unpack_combine(to_dev(recv_h, dtype, DEV), base_e=not base2,
                                   return_lse=return_lse)
    torch.cuda.synchronize()
    y, L = res if return_lse else (res, None)
    y_ref, L_ref = oracle.unpack_combine(recv_h, D, dtype, base2)
    oo, _ = oracle.unpack(recv_h, D, dtype)
    assert_output_close(y, y_ref, dtype, max_abs_input(oo, dtype))
    if return_lse:
        assert_lse_close(L, L_ref)


@pytest.mark.parametrize("N,base2", [(4, False), (8, True), (2, False)])
def test_dcp_a2a_lse_reduce_simulated_ranks(lsec, N, base2):
    """N ranks on one GPU: each rank's reduce packs its [B,H,D] partial, the
    exchange copies plane `rank` of every rank's send buffer into its receive
    buffer (the all-to-all's chunk order), and the combine returns the rank's
    H/N heads; each rank matches the oracle's pack, exchange and combine."""
    B, H, D = 33, 16, 128
    _announce(f"dcp_a2a_lse_reduce N={N} base2={base2}")
    outs, lses = [], []
    for r in range(N):
        a, b = synth.custom_inputs(1, B, H, D, seed=800 + 10 * N + r, special=SPECIALS)
        outs.append(a[0])
        lses.append(b[0])
    dev_o = [to_dev(o, "bf16", DEV) for o in outs]
    dev_l = [f32_to_dev(l, DEV) for l in lses]
    sends = [lsec.lsec_pack_send(dev_o[r], dev_l[r], N) for r in range(N)]
    recvs_h = oracle.exchange([oracle.pack_send(outs[r], lses[r], N) for r in range(N)])
    for rank in range(N):
        def exchange(send, recv, rank=rank):
            assert torch.equal(send.view(torch.int16), sends[rank].view(torch.int16))
            for n in range(N):
                recv[n].copy_(sends[n][rank])

        y, L = lsec.dcp_a2a_lse_reduce(dev_o[rank], dev_l[rank], N, exchange, return_lse=True,
                                       is_lse_base_on_e=not base2)
        torch.cuda.synchronize()
        assert tuple(y.shape) == (B, H // N, D)
        y_ref, L_ref = oracle.unpack_combine(recvs_h[rank], D, "bf16", base2)
        oo, _ = oracle.unpack(recvs_h[rank], D)
        assert_output_close(y, y_ref, "bf16", max_abs_input(oo, "bf16"), f"rank {rank}")
        assert_lse_close(L, L_ref, f"rank {rank}")


def test_dcp_a2a_lse_reduce_on_kept_buffers(lsec):
    """The same reduce through the kept send / receive buffers of
    dcp_a2a_send_recv_buffers, twice in a row: bit for bit the result of
    freshly allocated buffers, and the buffers are the same memory both times."""
    N, B, H, D = 4, 21, 16, 128
    _announce(f"dcp_a2a_lse_reduce kept buffers N={N}")
    a, b = synth.custom_inputs(1, B, H, D, seed=871, special=SPECIALS)
    o, l = to_dev(a[0], "bf16", DEV), f32_to_dev(b[0], DEV)

    def exchange(send, recv):  # every rank sends what this rank sent (a stand-in)
        for n in range(N):
            recv[n].copy_(send[n])

    y0, L0 = lsec.dcp_a2a_lse_reduce(o, l, N, exchange, return_lse=True)
    shape = (N, B, H // N, D + lsec.lsec_pack_dim(torch.bfloat16))
    ptrs = None
    for _ in range(2):
        send, recv = lsec.dcp_a2a_send_recv_buffers(shape, DEV, torch.bfloat16)
        y, L = lsec.dcp_a2a_lse_reduce(o, l, N, exchange, return_lse=True, send=send, recv=recv)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), y0.view(torch.int16))
        assert torch.equal(L.view(torch.int32), L0.view(torch.int32))
        if ptrs is not None:
            assert (send.data_ptr(), recv.data_ptr()) == ptrs
        ptrs = (send.data_ptr(), recv.data_ptr())


@pytest.mark.parametrize("N,B,H,dtype", [(8, 64, 16, "bf16"), (16, 37, 64, "f16"), (2, 1030, 4, "bf16")])
def test_unpack_combine_receive_buffer_off_16_byte_alignment(lsec, N, B, H, dtype):
    """The same receive buffer 4 bytes past a 16-byte boundary (packed rows are
    only 4-byte aligned anyway) gives the same results as an aligned one. The
    aligned buffer takes the span kernel, the shifted one the tiled kernel;
    both sum the planes in the same order, so the results agree bit for bit."""
    D = 128
    _announce(f"unpack_combine N={N} B={B} H={H} {dtype}, receive buffer 4 bytes off 16-byte alignment")
    assert lsec.lsec_combine_path(N, B, H // N, D, packed=True, dtype=TDT[dtype]) == \
        "combine_span_kernel"
    outs, lses = [], []
    for r in range(N):
        a, b = synth.custom_inputs(1, B, H, D, dtype=dtype, seed=760 + r, special=SPECIALS)
        outs.append(a[0])
        lses.append(b[0])
    recv_h = oracle.exchange([oracle.pack_send(outs[r], lses[r], N, dtype) for r in range(N)])[1]
    flat = torch.empty(recv_h.size + 8, dtype=TDT[dtype], device=DEV)
    shifted = flat[2:2 + recv_h.size].view(recv_h.shape)
    shifted.copy_(to_dev(recv_h, dtype, DEV))
    assert shifted.data_ptr() % 16 == 4
    y1, L1 = lsec.lsec_unpack_combine(shifted, return_lse=True)
    y2, L2 = lsec.lsec_unpack_combine(to_dev(recv_h, dtype, DEV), return_lse=True)
    torch.cuda.synchronize()
    y_ref, L_ref = oracle.unpack_combine(recv_h, D, dtype)
    oo, _ = oracle.unpack(recv_h, D, dtype)
    for y, L in ((y1, L1), (y2, L2)):
        assert_output_close(y, y_ref, dtype, max_abs_input(oo, dtype))
        assert_lse_close(L, L_ref)
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    assert torch.equal(L1.view(torch.int32), L2.view(torch.int32))


@pytest.mark.parametrize("N,B,H,D,dtype", [
    (4, 9, 8, 128, "bf16"), (2, 7, 6, 64, "f16"), (8, 3, 16, 512, "bf16"),
    (4, 5, 8, 6, "bf16"),    # general path: D % 8 != 0
    (2, 5, 4, 5, "f16"),     # odd D: packed rows only 2-byte aligned
    (3, 4, 9, 130, "bf16"),  # general path
])
def test_pack_unpack_shapes(lsec, N, B, H, D, dtype):
    _announce(f"pack/unpack N={N} B={B} H={H} D={D} {dtype}")
    o, l = synth.custom_inputs(1, B, H, D, dtype=dtype, seed=77 + D, special=SPECIALS)
    o, l = o[0], l[0]
    lb = l.view(np.uint32)
    lb[0, 0] = 0x7FC0BEEF  # NaN payload must survive
    send = lsec.lsec_pack_send(to_dev(o, dtype, DEV), f32_to_dev(l, DEV), N)
    torch.cuda.synchronize()
    ref = oracle.pack_send(o, l, N)
    assert np.array_equal(bits_of(send), ref)
    uo, ul = lsec.lsec_unpack(to_dev(ref, dtype, DEV))
    torch.cuda.synchronize()
    oo, ol = oracle.unpack(ref, D)
    assert np.array_equal(bits_of(uo), oo)
    assert np.array_equal(f32_bits_of(ul), ol.view(np.uint32))
    y, L = lsec.lsec_unpack_combine(to_dev(ref, dtype, DEV), base_e=True, return_lse=True)
    torch.cuda.synchronize()
    y_ref, L_ref = oracle.unpack_combine(ref, D, dtype, False)
    assert_output_close(y, y_ref, dtype, max_abs_input(oo, dtype))
    assert_lse_close(L, L_ref)


@pytest.mark.parametrize("N,B,H,dtype,offset", [
    (1, 3, 4, "bf16", 0),      # N = 1
    (2, 7, 8, "f16", 0),       # Hl = 4, ragged B
    (4, 5, 48, "bf16", 0),     # Hl = 12
    (16, 33, 256, "f16", 0),   # Hl = 16
    (3, 129, 12, "bf16", 0),   # N = 3
    (4, 1001, 16, "bf16", 0),  # 16016 rows: 251 tiles, the last one partly filled
    (4, 4099, 16, "bf16", 0),  # 65584 rows: 1025 tiles of 64 rows on 1024 blocks
    (8, 5000, 64, "f16", 0),   # 320000 rows: 5000 tiles, four or five per block
    (4, 37, 16, "f16", 16),    # buffers 16 bytes into their allocations
])
def test_pack_pipe_shapes(lsec, N, B, H, dtype, offset):
    """The pipelined LDS pack over several heads per rank, ragged token
    counts, more tiles than its grid has blocks (blocks that walk two tiles,
    the last one partly filled) and buffers 16 bytes into their allocations:
    the send buffer must equal the oracle's bit for bit, the LSE tails
    included (NaN payloads, infinities, -0 and subnormals)."""
    D = 128
    _announce(f"pack_pipe N={N} B={B} H={H} {dtype} offset={offset}")
    assert lsec.lsec_pack_path(N, B, H, D, TDT[dtype]) == "pack_pipe_kernel"
    o, l = synth.custom_inputs(1, B, H, D, dtype=dtype, seed=91 + N + B, special=SPECIALS)
    o, l = o[0], l[0]
    lb = l.view(np.uint32)
    lb[0, 0] = 0x7FC0BEEF            # NaN payload
    lb[-1, -1] = 0x80000000          # -0
    lb[B // 2, H // 2] = 0x00000003  # subnormal
    lb[B - 1, 0] = 0xFF800000        # -inf
    e = offset // 2                  # elements of the offset
    oflat = torch.empty(o.size + e, dtype=TDT[dtype], device=DEV)
    og = oflat[e:].view(B, H, D)
    og.copy_(to_dev(o, dtype, DEV))
    lflat = torch.empty(l.size + offset // 4, dtype=torch.float32, device=DEV)
    lg = lflat[offset // 4:].view(B, H)
    lg.copy_(f32_to_dev(l, DEV))
    sflat = torch.empty(B * H * (D + 2) + e, dtype=TDT[dtype], device=DEV)
    send = sflat[e:].view(N, B, H // N, D + 2)
    lsec.lsec_pack_send(og, lg, N, send=send)
    torch.cuda.synchronize()
    assert np.array_equal(bits_of(send), oracle.pack_send(o, l, N))


@pytest.mark.parametrize("N,B,H,D,dtype", [
    (2, 2049, 16, 256, "bf16"),   # 32 rows per tile: 1025 tiles, the last 16 rows
    (4, 1025, 16, 512, "bf16"),   # 16 rows per tile: 1025 tiles, the last 16 rows
    (2, 21761, 16, 24, "f16"),    # 3 lanes per row, 340 rows per tile: 1025 tiles
    (2, 2049, 16, 128, "f32"),    # fp32 rows, 32 per tile: 1025 tiles
    (2, 257, 16, 1024, "f32"),    # 256 lanes per row, 4 rows per tile: 1028 tiles
])
def test_pack_pipe_tile_walk(lsec, N, B, H, D, dtype):
    """Row widths whose tiles outnumber the pipelined pack's blocks, so blocks
    walk several tiles through both LDS stages and the last tile is ragged:
    bit for bit the oracle's send buffer."""
    _announce(f"pack_pipe walk N={N} B={B} H={H} D={D} {dtype}")
    assert lsec.lsec_pack_path(N, B, H, D, TDT[dtype]) == "pack_pipe_kernel"
    o, l = synth.custom_inputs(1, B, H, D, dtype=dtype, seed=7 * D + B, special=SPECIALS)
    o, l = o[0], l[0]
    send = lsec.lsec_pack_send(to_dev(o, dtype, DEV), f32_to_dev(l, DEV), N)
    torch.cuda.synchronize()
    assert np.array_equal(elem_bits_of(send, dtype), oracle.pack_send(o, l, N, dtype=dtype))


def test_misaligned_buffers_take_general_path(lsec):
    """Views that start 2 bytes into an allocation (only element-aligned)."""
    N, B, H, D = 4, 6, 5, 128
    _announce("misaligned views")
    o, l = synth.custom_inputs(N, B, H, D, seed=5, special=SPECIALS)
    flat = torch.empty(o.size + 1, dtype=torch.bfloat16, device=DEV)
    og = flat[1:].view(N, B, H, D)
    og.copy_(to_dev(o, "bf16", DEV))
    outflat = torch.empty(B * H * D + 1, dtype=torch.bfloat16, device=DEV)
    out = outflat[1:].view(B, H, D)
    y = lsec.lsec_combine(og, f32_to_dev(l, DEV), out=out)
    torch.cuda.synchronize()
    y_ref, _ = oracle.lse_combine(o, l, "bf16")
    assert_output_close(y, y_ref, "bf16", max_abs_input(o, "bf16"))
    # packed: send buffer starting one element in (rows 2-byte aligned only)
    a, b = synth.custom_inputs(1, 5, 8, 16, seed=6)
    sflat = torch.empty(2 * 5 * 4 * 18 + 1, dtype=torch.bfloat16, device=DEV)
    send = sflat[1:].view(2, 5, 4, 18)
    lsec.lsec_pack_send(to_dev(a[0], "bf16", DEV), f32_to_dev(b[0], DEV), 2, send=send)
    torch.cuda.synchronize()
    assert np.array_equal(bits_of(send), oracle.pack_send(a[0], b[0], 2))
    y2, L2 = lsec.lsec_unpack_combine(send, return_lse=True)
    torch.cuda.synchronize()
    y2r, L2r = oracle.unpack_combine(bits_of(send), 16, "bf16")
    assert_output_close(y2, y2r, "bf16", max_abs_input(a[0], "bf16"))
    assert_lse_close(L2, L2r)


@pytest.mark.parametrize("dtype,shift", [("bf16", 2), ("f16", 6), ("f32", 1)])
def test_pack_into_4byte_aligned_send(lsec, dtype, shift):
    """A send buffer 4 bytes (or 12) past a 16-byte boundary: the pack stores
    the packed rows directly instead of staging whole 16-byte chunks in LDS."""
    N, B, H, D = 4, 37, 8, 128
    _announce(f"pack into a 4-byte aligned send buffer {dtype}")
    o, l = synth.custom_inputs(1, B, H, D, dtype=dtype, seed=41, special=SPECIALS)
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[dtype]
    P = lsec.lsec_pack_dim(tdt)
    flat = torch.empty(N * B * (H // N) * (D + P) + shift, dtype=tdt, device=DEV)
    send = flat[shift:].view(N, B, H // N, D + P)
    assert send.data_ptr() % 16 != 0 and send.data_ptr() % 4 == 0
    lsec.lsec_pack_send(to_dev(o[0], dtype, DEV), f32_to_dev(l[0], DEV), N, send=send)
    torch.cuda.synchronize()
    ref = oracle.pack_send(o[0], l[0], N, dtype=dtype)
    got = f32_bits_of(send) if dtype == "f32" else bits_of(send)
    assert np.array_equal(got, ref)


# ---------------------------------------------------------------- token-major merge

MERGE = [
    # N, A, C, D, dtype, token_dim, base2
    (8, 8, 2048, 128, "bf16", 2, False),   # head-scattered exchange [N, Hl, T, D] -> [T, Hl, D]
    (4, 512, 64, 128, "bf16", 1, False),   # token-scattered [N, T/N, H, D] -> [T/N, H, D]
    (16, 4, 8197, 128, "bf16", 2, True),   # tiled 8 slots, ragged, transposed store
    (4, 16, 1031, 512, "f16", 2, False),   # one wave per row
    (3, 5, 77, 64, "bf16", 2, True),       # row kernel (D = 64)
    (6, 4, 1031, 128, "bf16", 2, False),   # tiled, N at run time, transposed store
    (2, 7, 13, 12, "f16", 2, False),       # element kernel (D % 8 != 0)
]


@pytest.mark.parametrize("N,A,C,D,dtype,token_dim,base2", MERGE)
def test_merge_token_major(lsec, N, A, C, D, dtype, token_dim, base2):
    _announce(f"merge N={N} A={A} C={C} D={D} {dtype} token_dim={token_dim} base2={base2}")
    o, l = synth.custom_inputs(N, A, C, D, dtype=dtype, seed=A * 31 + C, special=SPECIALS)
    y, L = lsec.lsec_merge(to_dev(o, dtype, DEV), f32_to_dev(l, DEV), token_dim,
                           base_e=not base2, return_lse=True)
    torch.cuda.synchronize()
    y_ref, L_ref = oracle.merge(o, l, dtype, token_dim, base2)
    assert tuple(y.shape) == y_ref.shape
    assert_output_close(y, y_ref, dtype, max_abs_input(o, dtype))
    assert_lse_close(L, L_ref)


def test_merge_heads_workload_full(lsec):
    """The merge_heads workload the benchmark times: [8, 8, 2048, 128] bf16 planes
    merged token-major into [2048, 8, 128] (head-scattered exchange)."""
    w = synth.WORKLOADS["merge_heads"]
    _announce("merge_heads full")
    o, l = synth.combine_inputs(w)
    y = lsec.lsec_merge(to_dev(o, w.dtype, DEV), f32_to_dev(l, DEV), 2, base_e=True)
    torch.cuda.synchronize()
    y_ref, _ = oracle.merge(o, l, w.dtype, 2, False)
    assert tuple(y.shape) == (w.H, w.B, w.D)
    assert_output_close(y, y_ref, w.dtype, max_abs_input(o, w.dtype))


def test_merge_page_alias(lsec):
    o, l = synth.custom_inputs(4, 4, 33, 128, seed=14, special=SPECIALS)
    y = lsec.merge_dcp_outputs(to_dev(o, "bf16", DEV), f32_to_dev(l, DEV), 2)
    torch.cuda.synchronize()
    y_ref, _ = oracle.merge(o, l, "bf16", 2)
    assert_output_close(y, y_ref, "bf16", max_abs_input(o, "bf16"))


# ---------------------------------------------------------------- receive planes of the direct exchange

PLANES = [
    # W, T, T_max, H, D, dtype, base2   (path)
    (8, 3000, 4096, 16, 128, "bf16", False),  # tiled
    (4, 777, 1024, 8, 512, "f16", True),      # tiled, one wave per row
    (8, 2051, 2304, 8, 128, "f32", False),    # tiled fp32
    (3, 50, 64, 4, 128, "bf16", True),        # row kernel (N = 3)
    (2, 9, 16, 4, 12, "bf16", False),         # element kernel (D % 8 != 0)
    (4, 0, 16, 4, 128, "bf16", False),        # no valid tokens
    (4, 16, 16, 4, 128, "bf16", False),       # T = T_max: the dense combine
]


@pytest.mark.parametrize("W,T,T_max,H,D,dtype,base2", PLANES)
def test_combine_planes_of_a_ubatch_slot(lsec, W, T, T_max, H, D, dtype, base2):
    """A [U=2, 2, W, T_max, H, D] receive buffer whose tokens past T hold NaN
    (stale data of an earlier step): the combine of ubatch 1, slot 0 reads
    only the first T tokens of each plane."""
    _announce(f"combine_planes W={W} T={T} T_max={T_max} H={H} D={D} {dtype}")
    o, l = synth.custom_inputs(W, T_max, H, D, dtype=dtype, seed=T_max + D, special=SPECIALS)
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[dtype]
    buf = torch.full((2, 2, W, T_max, H, D), float("nan"), dtype=tdt, device=DEV)
    lbuf = torch.full((2, 2, W, T_max, H), float("nan"), device=DEV)
    buf[1, 0, :, :T] = to_dev(o, dtype, DEV)[:, :T]
    lbuf[1, 0, :, :T] = f32_to_dev(l, DEV)[:, :T]
    y, L = lsec.lsec_combine_planes(buf[1, 0], lbuf[1, 0], T, base_e=not base2, return_lse=True)
    torch.cuda.synchronize()
    assert tuple(y.shape) == (T, H, D)
    if T == 0:
        return
    oT = np.ascontiguousarray(o[:, :T])
    y_ref, L_ref = oracle.lse_combine(oT, np.ascontiguousarray(l[:, :T]), dtype, base2)
    assert_output_close(y, y_ref, dtype, max_abs_input(oT, dtype))
    assert_lse_close(L, L_ref)


def test_combine_planes_padded_stride(lsec):
    """Planes 4 elements apart beyond their size (stride not a multiple of 16
    bytes: the general kernel) and the same data as a leading-token view."""
    W, T, H, D = 4, 37, 8, 128
    _announce("combine_planes padded stride")
    o, l = synth.custom_inputs(W, T, H, D, seed=88, special=SPECIALS)
    pad = T * H * D + 4
    flat = torch.full((W * pad,), float("nan"), dtype=torch.bfloat16, device=DEV)
    view = flat.as_strided((W, T, H, D), (pad, H * D, D, 1))
    view.copy_(to_dev(o, "bf16", DEV))
    lflat = torch.full((W * (T * H + 3),), float("nan"), device=DEV)
    lview = lflat.as_strided((W, T, H), (T * H + 3, H, 1))
    lview.copy_(f32_to_dev(l, DEV))
    y, L = lsec.lsec_combine_planes(view, lview, T, return_lse=True)
    torch.cuda.synchronize()
    y_ref, L_ref = oracle.lse_combine(o, l, "bf16")
    assert_output_close(y, y_ref, "bf16", max_abs_input(o, "bf16"))
    assert_lse_close(L, L_ref)
    with pytest.raises(ValueError):  # overlapping planes
        lsec.lsec_combine_planes(flat.as_strided((W, T, H, D), (T * H * D - 8, H * D, D, 1)),
                                 lview, T)


# ---------------------------------------------------------------- valid-token count in device memory

PLANES_VALID = [
    # W, T (capacity), Tv (query_start_loc[-1]), H, D, dtype, base2, out_f32, path
    (8, 16384, 10001, 32, 128, "bf16", False, False, "combine_tiled_kernel S=16"),  # 16 slots
    (8, 4096, 2500, 16, 512, "bf16", True, False, "combine_tiled_kernel S=8"),     # a wave per row
    (8, 4096, 3001, 16, 128, "bf16", False, False, "combine_tiled_kernel S=2"),    # mid-block
    (8, 4096, 4096, 16, 128, "bf16", False, False, "combine_tiled_kernel S=2"),    # all valid
    (8, 4096, 5000, 16, 128, "bf16", False, False, "combine_tiled_kernel S=2"),    # clamped to T
    (8, 4096, 0, 16, 128, "bf16", False, False, "combine_tiled_kernel S=2"),       # all padding
    (8, 4096, -3, 16, 128, "bf16", False, False, "combine_tiled_kernel S=2"),      # negative: none
    (4, 777, 500, 8, 512, "f16", True, False, "combine_tiled_kernel S=1"),
    (8, 2051, 1, 8, 128, "f32", False, False, "combine_tiled_kernel S=1"),         # one token
    (8, 1024, 700, 8, 128, "bf16", False, True, "combine_tiled_kernel S=1"),       # fp32 result
    (5, 300, 171, 4, 256, "bf16", True, False, "combine_tiled_kernel S=1"),        # N at run time
    (1, 64, 40, 4, 128, "bf16", False, False, "combine_rows_kernel"),              # N = 1
    (20, 40, 23, 4, 128, "bf16", True, False, "combine_rows_kernel"),              # N > 16
    (2, 16, 9, 4, 12, "bf16", False, False, "combine_elems_kernel"),               # D % 8 != 0
]


def _offsets(tv: int, seed: int) -> np.ndarray:
    """Cumulative token offsets of a few requests whose last entry is tv."""
    rng = np.random.default_rng(seed)
    if tv <= 0:
        return np.array([0, tv], dtype=np.int32)
    cuts = np.sort(rng.integers(0, tv + 1, size=min(tv, 6)))
    return np.concatenate([[0], cuts, [tv]]).astype(np.int32)


@pytest.mark.parametrize("W,T,Tv,H,D,dtype,base2,out_f32,path", PLANES_VALID)
def test_combine_planes_valid_count_on_device(lsec, W, T, Tv, H, D, dtype, base2, out_f32, path):
    """The count of valid tokens comes from query_start_loc[num_reqs] in
    device memory: the first Tv tokens match the oracle, and the rows of the
    padding tokens past Tv keep what the output held before (bit for bit)."""
    _announce(f"combine_planes_valid W={W} T={T} Tv={Tv} H={H} D={D} {dtype} out_f32={out_f32}")
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[dtype]
    assert lsec.lsec_combine_path(W, T, H, D, dtype=tdt) == path
    o, l = synth.custom_inputs(W, T, H, D, dtype=dtype, seed=3 * T + D + W, special=SPECIALS)
    rdt = torch.float32 if out_f32 else tdt
    planes, lplanes = to_dev(o, dtype, DEV), f32_to_dev(l, DEV)
    qsl = _offsets(Tv, seed=T + Tv)
    out = torch.full((T, H, D), -7.0, dtype=rdt, device=DEV)
    out_lse = torch.full((T, H), -7.0, device=DEV)
    lsec.lsec_combine_planes(planes, lplanes, T, base_e=not base2, return_lse=True, out=out,
                             out_lse=out_lse, out_dtype=rdt,
                             query_start_loc=torch.from_numpy(qsl).to(DEV))
    torch.cuda.synchronize()
    y_ref, L_ref, tv = oracle.lse_combine_valid(o, l, qsl, dtype, base2)
    assert tv == min(max(Tv, 0), T)
    if tv:
        oT = o[:, :tv]
        assert_output_close(out[:tv], y_ref, "f32" if out_f32 else dtype, max_abs_input(oT, dtype))
        assert_lse_close(out_lse[:tv], L_ref)
    assert bool(torch.all(out[tv:] == -7.0)), "a padding token's output row was written"
    assert bool(torch.all(out_lse[tv:] == -7.0)), "a padding token's LSE was written"


def test_combine_planes_valid_rejects_bad_offsets(lsec):
    o = torch.zeros((2, 4, 2, 128), dtype=torch.bfloat16, device=DEV)
    l = torch.zeros((2, 4, 2), device=DEV)
    for bad in (torch.tensor([0, 4], dtype=torch.int64, device=DEV),    # int64
                torch.tensor([[0, 4]], dtype=torch.int32, device=DEV),  # 2-D
                torch.zeros(0, dtype=torch.int32, device=DEV),          # empty
                torch.arange(6, dtype=torch.int32, device=DEV)[::2],    # strided
                torch.tensor([0, 4], dtype=torch.int32)):               # host memory
        with pytest.raises(ValueError):
            lsec.lsec_combine_planes(o, l, 4, query_start_loc=bad)


# ---------------------------------------------------------------- all-gather + reduce-scatter local step

CORRECT = [
    # N, B, H, D, dtype, base2      (path)
    (8, 4096, 16, 512, "bf16", True),   # tiled, one wave per row, 8 slots
    (16, 1000, 32, 128, "bf16", False),  # tiled, ragged
    (2, 777, 5, 256, "f16", True),      # tiled, two rows per wave
    (4, 33, 3, 64, "bf16", False),      # element kernel (D outside {128, 256, 512})
    (20, 9, 4, 128, "bf16", True),      # element kernel (N > 16)
]


@pytest.mark.parametrize("N,B,H,D,dtype,base2", CORRECT)
def test_correct_partial(lsec, N, B, H, D, dtype, base2):
    _announce(f"correct_partial N={N} B={B} H={H} D={D} {dtype} base2={base2}")
    o, l = synth.custom_inputs(N, B, H, D, dtype=dtype, seed=N * 7 + D, special=SPECIALS)
    lg = f32_to_dev(l, DEV)
    M = max_abs_input(o, dtype)
    total = torch.zeros((B, H, D), dtype=torch.float64, device=DEV)
    for r in sorted({0, N // 2, N - 1}):
        y, L = lsec.lsec_correct_partial(lg, r, to_dev(o[r], dtype, DEV), base_e=not base2,
                                         return_lse=True)
        torch.cuda.synchronize()
        y_ref, L_ref = oracle.correct_partial(l, r, o[r], dtype, base2)
        assert_output_close(y, y_ref, dtype, max_abs_input(o[r], dtype), f"rank {r}")
        assert_lse_close(L, L_ref, f"rank {r}")
    for r in range(N):
        total += lsec.lsec_correct_partial(lg, r, to_dev(o[r], dtype, DEV),
                                           base_e=not base2).double()
    torch.cuda.synchronize()
    # the ranks' corrected partials sum to the combine (each term rounded once)
    y_all, _ = oracle.lse_combine(o, l, dtype, base2)
    err = float((total.cpu().numpy() - y_all)[np.isfinite(y_all)].__abs__().max())
    assert err <= 2 * (8e-3 if dtype == "bf16" else 1e-3) * M + 1e-6


def test_correct_partial_rank_error(lsec):
    with pytest.raises(ValueError):
        lsec.lsec_correct_partial(torch.zeros(4, 2, 3, device=DEV), 4,
                                  torch.zeros(2, 3, 8, dtype=torch.bfloat16, device=DEV))


# ---------------------------------------------------------------- degenerate cases

# Signed zeros and subnormals of each element type (smallest and largest
# subnormal of either sign, and the smallest normal): a single shard of weight
# 1 must return every one of them bit for bit.
ZERO_AND_SUBNORMAL = {
    "bf16": [0x8000, 0x0000, 0x0001, 0x8001, 0x007F, 0x807F, 0x0080, 0x8080],
    "f16": [0x8000, 0x0000, 0x0001, 0x8001, 0x03FF, 0x83FF, 0x0400, 0x8400],
    "f32": [0x80000000, 0x00000000, 0x00000001, 0x80000001, 0x007FFFFF, 0x807FFFFF,
            0x00800000, 0x80800000],
}


def _identity_inputs(dtype, D, seed):
    o, l = synth.custom_inputs(1, 33, 7, D, dtype=dtype, seed=seed)
    if dtype == "f32":
        o = o.view(np.uint32)  # element patterns, like the 16-bit types
    pat = np.array(ZERO_AND_SUBNORMAL[dtype], dtype=o.dtype)
    k = min(len(pat), D)
    o[0, :, :, :k] = pat[:k]   # the patterns at the start of every row
    o[0, 5] = pat[0]           # a whole token of -0
    o[0, 6, :, ::2] = pat[2]   # and one of alternating subnormals
    return o, l


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("base_e", [True, False])
@pytest.mark.parametrize("D", [128, 12])  # the row kernel; the element kernel
def test_single_shard_is_identity_bit_exact(lsec, dtype, base_e, D):
    """N = 1 with finite LSEs returns its input unchanged, -0 and subnormals
    included (accumulators start at -0, fp32 denormals are kept)."""
    o, l = _identity_inputs(dtype, D, seed=8 + D)
    y, L = lsec.lsec_combine(to_dev(o, dtype, DEV), f32_to_dev(l, DEV), base_e=base_e,
                             return_lse=True)
    torch.cuda.synchronize()
    assert np.array_equal(elem_bits_of(y, dtype), o[0])
    assert np.array_equal(f32_bits_of(L), l[0].view(np.uint32))


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_single_shard_unpack_combine_is_identity_bit_exact(lsec, dtype):
    """The same through the packed path: one plane packed by the oracle."""
    o, l = _identity_inputs(dtype, 128, seed=18)
    recv = oracle.pack_send(o[0], l[0], 1, dtype)
    y, L = lsec.lsec_unpack_combine(to_dev(recv, dtype, DEV), base_e=True, return_lse=True)
    torch.cuda.synchronize()
    assert np.array_equal(elem_bits_of(y, dtype), o[0])
    assert np.array_equal(f32_bits_of(L), l[0].view(np.uint32))


def test_all_shards_non_finite(lsec):
    N, B, H, D = 4, 5, 3, 128
    o, _ = synth.custom_inputs(N, B, H, D, seed=9)
    l = np.empty((N, B, H), dtype=np.float32)
    l[0], l[1], l[2], l[3] = np.nan, np.inf, -np.inf, np.nan
    for D_ in (128, 12):  # fast and general paths
        oo = np.ascontiguousarray(o[..., :D_])
        y, L = lsec.lsec_combine(to_dev(oo, "bf16", DEV), f32_to_dev(l, DEV), return_lse=True)
        torch.cuda.synchronize()
        assert torch.all(y == 0)
        assert torch.all(torch.isneginf(L))


F32_MAX = float(np.finfo(np.float32).max)
EXTREME_LSE_ROWS = [
    [F32_MAX, -F32_MAX],           # the whole fp32 range between two shards
    [3.0e38, 3.0e38],              # equal and huge: the mean, L = l + ln N
    [-3.0e38, -3.0e38],            # equal and hugely negative, still finite
    [1.0e-45, -1.0e-45, 0.0, -0.0],  # subnormal and signed-zero LSEs
    [1.0e38, float("nan"), float("inf"), -1.0e38],
    [80.0, -80.0, 0.0, 88.7],      # weights down to fp32 underflow
    [-1.0e30, 5.0],
]
# The largest finite value of each 16-bit format (patterns); fp32 partials
# use 1e38, since a weighted sum of fp32 maxima can round past the fp32 range
# in any fp32 evaluation of the page's sum.
EXTREME_OUT = {"bf16": 0x7F7F, "f16": 0x7BFF, "f32": np.float32(1e38)}


def _extreme_inputs(N, B, H, D, dtype, seed):
    o, l = synth.custom_inputs(N, B, H, D, dtype=dtype, seed=seed)
    rows = l.reshape(N, B * H)
    for r, pat in enumerate(EXTREME_LSE_ROWS):
        for n in range(N):
            rows[n, r] = pat[n % len(pat)]
    flat = o.reshape(N, B * H, D)
    flat[:, 1, :] = EXTREME_OUT[dtype]          # the equal, huge LSEs: their maxima
    flat[0, 0, : D // 2] = EXTREME_OUT[dtype]   # the dominant shard of row 0
    return o, l


def _assert_rows_close(y, y_ref, o, dtype, what):
    """Rows 0 and 1 hold the format's largest values; the tolerance of the
    other rows is set by their own inputs."""
    N, D = o.shape[0], o.shape[-1]
    of = o.reshape(N, -1, D)
    yf = y.reshape(-1, D)
    rf = np.asarray(y_ref).reshape(-1, D)
    assert_output_close(yf[:2], rf[:2], dtype, max_abs_input(of[:, :2], dtype), what)
    assert_output_close(yf[2:], rf[2:], dtype, max_abs_input(of[:, 2:], dtype), what)


def _assert_lse_close_fp32(L, L_ref, what):
    """Global LSEs within 1e-5 plus two fp32 ulps of the exact value: beyond
    |L| = 256 half an fp32 ulp alone exceeds 1e-5."""
    got = L.cpu().numpy().astype(np.float64).reshape(-1)
    want = np.asarray(L_ref, dtype=np.float64).reshape(-1)
    fin = np.isfinite(want)
    assert np.array_equal(np.isfinite(got), fin), f"{what}: non-finite LSEs differ"
    assert np.array_equal(got[~fin], want[~fin]), f"{what}: non-finite LSEs differ"
    mag = np.abs(want[fin]).astype(np.float32)
    ulp = np.spacing(np.nextafter(mag, np.float32(0))).astype(np.float64)  # finite at FLT_MAX
    err = np.abs(got[fin] - want[fin])
    assert np.all(err <= 1e-5 + 2 * ulp), f"{what}: max LSE error {err.max()}"


@pytest.mark.parametrize("N,B,H,D,dtype,base2", [
    (8, 40, 8, 128, "bf16", False),  # tiled
    (4, 40, 8, 128, "f16", True),    # tiled, base 2
    (4, 40, 8, 128, "f32", False),   # tiled, fp32 partials
    (20, 9, 3, 128, "bf16", True),   # row kernel
    (3, 5, 2, 12, "f16", False),     # element kernel
])
def test_extreme_finite_lses_and_outputs(lsec, N, B, H, D, dtype, base2):
    """LSEs at the edges of fp32 (near +-FLT_MAX, subnormal, +-0, mixed with
    NaN and +-inf) and outputs at the largest finite value of their format:
    the combine still matches the oracle."""
    _announce(f"extreme values N={N} B={B} H={H} D={D} {dtype} base2={base2}")
    o, l = _extreme_inputs(N, B, H, D, dtype, seed=600 + N)
    y, L = lsec.lsec_combine(to_dev(o, dtype, DEV), f32_to_dev(l, DEV), base_e=not base2,
                             return_lse=True)
    torch.cuda.synchronize()
    y_ref, L_ref = oracle.lse_combine(o, l, dtype, base2)
    _assert_rows_close(y, y_ref, o, dtype, "extreme")
    _assert_lse_close_fp32(L, L_ref, "extreme")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_extreme_values_through_the_span_kernels(lsec, dtype):
    """The same extreme rows through the packed receive side (span kernels)."""
    N, B, Hl, D = 8, 16, 4, 128
    _announce(f"extreme values, packed span kernel {dtype}")
    o, l = _extreme_inputs(N, B, Hl, D, dtype, seed=700)
    elem = np.uint32 if dtype == "f32" else np.uint16
    P = 4 // np.dtype(elem).itemsize
    tail = np.ascontiguousarray(l).view(np.uint32).view(elem).reshape(N, B, Hl, P)
    recv_h = np.concatenate([np.ascontiguousarray(o).view(elem).reshape(N, B, Hl, D), tail], axis=3)
    assert lsec.lsec_combine_path(N, B, Hl, D, packed=True, dtype=TDT[dtype]) in (
        "combine_span_kernel", "combine_span32_kernel")
    y, L = lsec.lsec_unpack_combine(to_dev(recv_h, dtype, DEV), return_lse=True)
    torch.cuda.synchronize()
    y_ref, L_ref = oracle.unpack_combine(recv_h, D, dtype, False)
    _assert_rows_close(y, y_ref, o, dtype, "extreme packed")
    _assert_lse_close_fp32(L, L_ref, "extreme packed")


def test_nan_output_at_zero_weight_propagates(lsec):
    """Every shard is multiplied, so a NaN output at weight 0 still gives NaN."""
    N, B, H, D = 2, 2, 2, 128
    o, l = synth.custom_inputs(N, B, H, D, seed=10)
    o[0, 0, 0, 5] = 0x7FC0  # bf16 NaN
    l[0, 0, 0] = -np.inf    # its shard has weight 0
    y = lsec.lsec_combine(to_dev(o, "bf16", DEV), f32_to_dev(l, DEV))
    torch.cuda.synchronize()
    y_ref, _ = oracle.lse_combine(o, l, "bf16")
    assert np.isnan(y_ref[0, 0, 5])
    assert_output_close(y, y_ref, "bf16", max_abs_input(o, "bf16"))


def test_extreme_lse_values(lsec):
    N, B, H, D = 4, 8, 4, 128
    o, l = synth.custom_inputs(N, B, H, D, seed=11)
    l[0] = 3e38
    l[1] = -3e38
    l[2, :4] = 1e30
    l[3] = 0.0
    for base_e in (True, False):
        y, L = lsec.lsec_combine(to_dev(o, "bf16", DEV), f32_to_dev(l, DEV), base_e=base_e,
                                 return_lse=True)
        torch.cuda.synchronize()
        y_ref, L_ref = oracle.lse_combine(o, l, "bf16", base2=not base_e)
        assert_output_close(y, y_ref, "bf16", max_abs_input(o, "bf16"))
        assert_lse_close(L, L_ref)


def test_empty_batch(lsec):
    og = torch.empty((4, 0, 8, 128), dtype=torch.bfloat16, device=DEV)
    lg = torch.empty((4, 0, 8), dtype=torch.float32, device=DEV)
    y, L = lsec.lsec_combine(og, lg, return_lse=True)
    assert y.shape == (0, 8, 128) and L.shape == (0, 8)
    s = lsec.lsec_pack_send(torch.empty((0, 8, 128), dtype=torch.float16, device=DEV),
                            torch.empty((0, 8), device=DEV), 4)
    assert s.shape == (4, 0, 2, 130)
    y2 = lsec.lsec_unpack_combine(s)
    assert y2.shape == (0, 2, 128)


def test_errors_raise(lsec):
    with pytest.raises(ValueError):
        lsec.lsec_pack_send(torch.zeros(2, 6, 8, dtype=torch.bfloat16, device=DEV),
                            torch.zeros(2, 6, device=DEV), 4)
    with pytest.raises(ValueError):
        lsec.lsec_combine(torch.zeros(2, 1, 1, 8, dtype=torch.float64, device=DEV),
                          torch.zeros(2, 1, 1, device=DEV))
    with pytest.raises(ValueError):
        lsec.lsec_combine(torch.zeros(2, 1, 1, 8, dtype=torch.bfloat16, device=DEV),
                          torch.zeros(2, 1, 1, dtype=torch.float64, device=DEV))


def test_side_stream_and_preallocated_outputs(lsec):
    N, B, H, D = 8, 64, 8, 128
    o, l = synth.custom_inputs(N, B, H, D, seed=12, special=SPECIALS)
    og, lg = to_dev(o, "bf16", DEV), f32_to_dev(l, DEV)
    out = torch.full((B, H, D), 7.0, dtype=torch.bfloat16, device=DEV)
    out_lse = torch.full((B, H), 7.0, device=DEV)
    s = torch.cuda.Stream(device=DEV)
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        lsec.lsec_combine(og, lg, return_lse=True, out=out, out_lse=out_lse)
    s.synchronize()
    y_ref, L_ref = oracle.lse_combine(o, l, "bf16")
    assert_output_close(out, y_ref, "bf16", max_abs_input(o, "bf16"))
    assert_lse_close(out_lse, L_ref)


def test_plain_name_wrappers(lsec):
    """lse_combine / pack_send / unpack_combine: the hot path under its plain
    names, on the packed workload's shapes scaled down."""
    N, B, H, D = 4, 33, 8, 128
    o, l = synth.custom_inputs(N, B, H, D, seed=55, special=SPECIALS)
    y, L = lsec.lse_combine(to_dev(o, "bf16", DEV), f32_to_dev(l, DEV), base_e=False,
                            return_lse=True)
    torch.cuda.synchronize()
    y_ref, L_ref = oracle.lse_combine(o, l, "bf16", base2=True)
    assert_output_close(y, y_ref, "bf16", max_abs_input(o, "bf16"))
    assert_lse_close(L, L_ref)
    send = lsec.pack_send(to_dev(o[0], "bf16", DEV), f32_to_dev(l[0], DEV), N)
    torch.cuda.synchronize()
    assert np.array_equal(bits_of(send), oracle.pack_send(o[0], l[0], N))
    y2, L2 = lsec.unpack_combine(send, D, return_lse=True)
    torch.cuda.synchronize()
    y2_ref, L2_ref = oracle.unpack_combine(bits_of(send), D, "bf16")
    oo, _ = oracle.unpack(bits_of(send), D)
    assert_output_close(y2, y2_ref, "bf16", max_abs_input(oo, "bf16"))
    assert_lse_close(L2, L2_ref)
    with pytest.raises(ValueError):
        lsec.unpack_combine(send, D + 2)


def test_page_signature_alias(lsec):
    """The page's function returns fp32 (bf16 outputs times fp32 weights)."""
    o, l = synth.custom_inputs(3, 4, 4, 64, seed=13)
    y, L = lsec.lse_weighted_combine(to_dev(o, "bf16", DEV), f32_to_dev(l, DEV), return_lse=True,
                                     is_lse_base_on_e=False)
    torch.cuda.synchronize()
    assert y.dtype == torch.float32
    y_ref, L_ref = oracle.lse_combine(o, l, "bf16", base2=True)
    assert_output_close(y, y_ref, "f32", max_abs_input(o, "bf16"))
    assert_lse_close(L, L_ref)
