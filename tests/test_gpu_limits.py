"""GPU parity at the limits of the kernels' index arithmetic.

The tiled combine addresses a lane's chunk by a 32-bit byte offset inside its
plane, so it serves planes below 4 GiB; larger planes take the row kernel,
which uses 64-bit offsets. The row kernels (combine, pack, unpack) count rows
in 32 bits, so 2^31 rows and more take the element-wise kernels (64-bit
throughout); those tests run each call just below and just above that line.
The corrected partial's and the combine's tiled kernels address the LSEs with
32-bit offsets (N * rows, N * LSE plane stride < 2^32); the last tests run
just below and above that. These tests run a plane just below and just above
4 GiB (8.6 GB of partial outputs each) and check sampled token ranges at the
start, the middle and the very end of the planes against the oracle (rows are
independent, so the oracle's result on a token slice of the inputs is exactly
those rows' result).
"""
import gc
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import assert_lse_close, assert_output_close, f32_to_dev, max_abs_input, to_dev

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
SPECIALS = ((0.01, float("nan")), (0.01, float("inf")), (0.01, float("-inf")))


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


def _release():
    gc.collect()
    torch.cuda.empty_cache()


def _workload(N, B, H, D, wid):
    return synth.Workload(f"limit_{wid}", wid, "combine", N, B, H, D, "bf16", ("normal", 0.0, 1.0),
                          ("uniform", -10.0, 30.0), special=SPECIALS)


def _ranges(B):
    return ((0, 64), (B // 2 - 32, B // 2 + 32), (B - 64, B))


@pytest.mark.parametrize("B,path", [
    (524287, "combine_tiled_kernel S=16"),   # plane = 4,294,959,104 B: the largest 32-bit plane here
    (524289, "combine_rows_kernel"),         # plane = 4,294,983,680 B > 2^32: 64-bit offsets
])
def test_combine_around_4gib_planes(lsec, B, path):
    N, H, D = 2, 32, 128
    _announce(f"combine N={N} B={B} H={H} D={D} bf16 ({B * H * D * 2} B per plane)")
    assert lsec.lsec_combine_path(N, B, H, D) == path
    w = _workload(N, B, H, D, 120 + (B & 7))
    o, l = synth.combine_inputs(w)
    M = max_abs_input(o[:, :64], "bf16")
    og, lg = to_dev(o, "bf16", DEV), f32_to_dev(l, DEV)
    del o, l
    y, L = lsec.lsec_combine(og, lg, base_e=True, return_lse=True)
    torch.cuda.synchronize()
    del og, lg
    for s, e in _ranges(B):
        os_, ls_ = synth.combine_inputs(w, b_lo=s, b_hi=e)
        y_ref, L_ref = oracle.lse_combine(os_, ls_, "bf16")
        Ms = max(M, max_abs_input(os_, "bf16"))
        assert_output_close(y[s:e], y_ref, "bf16", Ms, f"tokens {s}:{e}")
        assert_lse_close(L[s:e], L_ref, f"tokens {s}:{e}")
    del y, L
    _release()


@pytest.mark.parametrize("B,path", [
    (516222, "combine_tiled_kernel S=16"),   # packed plane = 4,294,967,040 B, 256 B under 2^32
    (516223, "combine_rows_kernel"),
])
def test_unpack_combine_around_4gib_planes(lsec, B, path):
    """Packed receive planes [2, B, 32, 130] built on the host from generated
    planes (output row, then the LSE's bytes)."""
    N, Hl, D = 2, 32, 128
    _announce(f"unpack_combine N={N} B={B} Hl={Hl} D={D} bf16 ({B * Hl * (D + 2) * 2} B per plane)")
    assert lsec.lsec_combine_path(N, B, Hl, D, packed=True) == path
    w = _workload(N, B, Hl, D, 130 + (B & 7))
    o, l = synth.combine_inputs(w)
    recv = np.empty((N, B, Hl, D + 2), dtype=np.uint16)
    recv[..., :D] = o
    recv[..., D:] = l.view(np.uint16).reshape(N, B, Hl, 2)
    del o, l
    rg = to_dev(recv, "bf16", DEV)
    y, L = lsec.lsec_unpack_combine(rg, base_e=True, return_lse=True)
    torch.cuda.synchronize()
    del rg
    for s, e in _ranges(B):
        part = np.ascontiguousarray(recv[:, s:e])
        y_ref, L_ref = oracle.unpack_combine(part, D, "bf16")
        oo, _ = oracle.unpack(part, D)
        assert_output_close(y[s:e], y_ref, "bf16", max_abs_input(oo, "bf16"), f"tokens {s}:{e}")
        assert_lse_close(L[s:e], L_ref, f"tokens {s}:{e}")
    del recv, y, L
    _release()


@pytest.mark.parametrize("rows,path", [
    (2**31 - 4096, "combine_rows_kernel"),
    (2**31 + 4096, "combine_elems_kernel"),
])
def test_combine_around_2g_rows(lsec, rows, path):
    """N=2 planes of `rows` rows of D=8 bf16 (68.7 GB of partial outputs, about
    129 GB with LSEs and results). The inputs repeat one seeded 4096-row block
    (tiled on the device), so every row's oracle result is that of its row in
    the block; rows are checked at the start, across 2^31 and at the end."""
    N, D, K = 2, 8, 4096
    _announce(f"combine N={N} rows={rows} D={D} bf16 ({path})")
    assert lsec.lsec_combine_path(N, rows, 1, D) == path
    o, l = synth.custom_inputs(N, K, 1, D, seed=2031, lse_dist=("uniform", -10.0, 30.0),
                               special=SPECIALS)
    y_ref, L_ref = oracle.lse_combine(o, l, "bf16")
    M = max_abs_input(o, "bf16")
    og = torch.empty((N, rows, 1, D), dtype=torch.bfloat16, device=DEV)
    lg = torch.empty((N, rows, 1), dtype=torch.float32, device=DEV)
    og.view(N, rows // K, K, D).copy_(to_dev(o, "bf16", DEV).view(N, 1, K, D).expand(N, rows // K, K, D))
    lg.view(N, rows // K, K).copy_(f32_to_dev(l, DEV).view(N, 1, K).expand(N, rows // K, K))
    y, L = lsec.lsec_combine(og, lg, base_e=True, return_lse=True)
    torch.cuda.synchronize()
    del og, lg
    _release()
    for s in (0, 2**31 - K, 2**31, rows - K):
        if s + K > rows:
            continue
        assert_output_close(y[s:s + K], y_ref, "bf16", M, f"rows {s}:{s + K}")
        assert_lse_close(L[s:s + K], L_ref, f"rows {s}:{s + K}")
    del y, L
    _release()


@pytest.mark.parametrize("B", [2**30 - 4096, 2**30 + 4096])
def test_pack_and_unpack_around_2g_rows(lsec, B):
    """pack_send of [B, H=2, D=8] bf16 (2 * B rows: 2^31 -+ 8192, fast kernel
    below, element kernel above) and lsec_unpack of the result (N * B * Hl rows,
    the same count), bit for bit. The input repeats one seeded 4096-token
    block, so the send planes repeat the oracle's pack of that block."""
    N, H, D, K = 2, 2, 8, 4096
    _announce(f"pack_send + unpack N={N} B={B} H={H} D={D} bf16 ({B * H} rows)")
    o, l = synth.custom_inputs(1, K, H, D, seed=2032, special=SPECIALS)
    send_ref = oracle.pack_send(o[0], l[0], N)                # [N, K, 1, D + 2]
    og = torch.empty((B, H, D), dtype=torch.bfloat16, device=DEV)
    lg = torch.empty((B, H), dtype=torch.float32, device=DEV)
    og.view(B // K, K, H, D).copy_(to_dev(o[0], "bf16", DEV).view(1, K, H, D).expand(B // K, K, H, D))
    lg.view(B // K, K, H).copy_(f32_to_dev(l[0], DEV).view(1, K, H).expand(B // K, K, H))
    send = lsec.lsec_pack_send(og, lg, N)
    torch.cuda.synchronize()
    del og, lg
    _release()
    starts = [s for s in (0, 2**30 - K, 2**30, B - K) if s + K <= B]
    for s in starts:
        got = send[:, s:s + K].view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(got, send_ref), f"send tokens {s}:{s + K}"
    outs, lses = lsec.lsec_unpack(send)
    torch.cuda.synchronize()
    del send
    _release()
    for s in starts:
        got_o = outs[:, s:s + K].view(torch.int16).cpu().numpy().view(np.uint16)
        got_l = lses[:, s:s + K].view(torch.int32).cpu().numpy().view(np.uint32)
        assert np.array_equal(got_o, o[0].transpose(1, 0, 2).reshape(N, K, 1, D)), f"outputs {s}"
        assert np.array_equal(got_l, l[0].view(np.uint32).T.reshape(N, K, 1)), f"lses {s}"
    del outs, lses
    _release()


@pytest.mark.parametrize("B,path", [
    (2**31 - 4096, "combine_rows_kernel"),
    (2**31 + 4096, "combine_elems_kernel"),
])
def test_unpack_combine_around_2g_rows(lsec, B, path):
    """unpack_combine of receive planes [2, B, 1, 10] bf16 (86 GB) that repeat
    one packed 4096-token block, checked at the start, across 2^31 and at the
    end against the oracle's unpack + combine of the block."""
    N, Hl, D, K = 2, 1, 8, 4096
    _announce(f"unpack_combine N={N} B={B} Hl={Hl} D={D} bf16 ({path})")
    assert lsec.lsec_combine_path(N, B, Hl, D, packed=True) == path
    o, l = synth.custom_inputs(N, K, Hl, D, seed=2033, lse_dist=("uniform", -10.0, 30.0),
                               special=SPECIALS)
    blk = np.empty((N, K, Hl, D + 2), dtype=np.uint16)
    blk[..., :D] = o
    blk[..., D:] = l.view(np.uint16).reshape(N, K, Hl, 2)
    y_ref, L_ref = oracle.unpack_combine(blk, D, "bf16")
    oo, _ = oracle.unpack(blk, D)
    M = max_abs_input(oo, "bf16")
    rg = torch.empty((N, B, Hl, D + 2), dtype=torch.bfloat16, device=DEV)
    rg.view(N, B // K, K, Hl, D + 2).copy_(
        to_dev(blk, "bf16", DEV).view(N, 1, K, Hl, D + 2).expand(N, B // K, K, Hl, D + 2))
    y, L = lsec.lsec_unpack_combine(rg, base_e=True, return_lse=True)
    torch.cuda.synchronize()
    del rg
    _release()
    for s in (0, 2**31 - K, 2**31, B - K):
        if s + K > B:
            continue
        assert_output_close(y[s:s + K], y_ref, "bf16", M, f"tokens {s}:{s + K}")
        assert_lse_close(L[s:s + K], L_ref, f"tokens {s}:{s + K}")
    del y, L
    _release()


@pytest.mark.parametrize("B", [2**28 - 4096, 2**28 + 4096])
def test_correct_partial_around_2_32_lse_entries(lsec, B):
    """lsec_correct_partial with N=16 gathered LSEs of B rows (D=128 bf16): the
    tiled kernel addresses the LSEs with 32-bit offsets, so it serves
    N * B < 2^32 and the element kernel the rest (about 155 GB in all here).
    The inputs repeat one seeded 4096-row block; rows are checked at the start,
    across 2^28 and at the end against the oracle's result on the block."""
    N, D, K, rank = 16, 128, 4096, 5
    _announce(f"correct_partial N={N} B={B} D={D} bf16 rank {rank} ({N * B} LSE entries)")
    o, l = synth.custom_inputs(N, K, 1, D, seed=2034, lse_dist=("uniform", -10.0, 30.0),
                               special=SPECIALS)
    y_ref, L_ref = oracle.correct_partial(l, rank, o[rank], "bf16")
    M = max_abs_input(o[rank], "bf16")
    pg = torch.empty((B, 1, D), dtype=torch.bfloat16, device=DEV)
    lg = torch.empty((N, B, 1), dtype=torch.float32, device=DEV)
    pg.view(B // K, K, D).copy_(to_dev(o[rank], "bf16", DEV).view(1, K, D).expand(B // K, K, D))
    lg.view(N, B // K, K).copy_(f32_to_dev(l, DEV).view(N, 1, K).expand(N, B // K, K))
    y, L = lsec.lsec_correct_partial(lg, rank, pg, return_lse=True)
    torch.cuda.synchronize()
    del pg, lg
    _release()
    for s in (0, 2**28 - K, 2**28, B - K):
        if s + K > B:
            continue
        assert_output_close(y[s:s + K], y_ref, "bf16", M, f"rows {s}:{s + K}")
        assert_lse_close(L[s:s + K], L_ref, f"rows {s}:{s + K}")
    del y, L
    _release()


@pytest.mark.parametrize("lse_stride", [2**29 - 1, 2**29])
def test_combine_planes_around_2_32_lse_offsets(lsec, lse_stride):
    """lsec_combine_planes whose LSE planes sit lse_stride floats apart (N=8):
    the tiled kernel addresses the LSEs with 32-bit offsets, so it serves
    N * lse_stride < 2^32 (the first case) and the row kernel the second. Only
    each plane's first T * H floats are written; the gaps (17 GB in all) are
    never read."""
    N, T, H, D = 8, 2048, 8, 128
    _announce(f"combine_planes N={N} T={T} H={H} D={D} bf16, LSE plane stride {lse_stride}")
    o, l = synth.custom_inputs(N, T, H, D, seed=2035, lse_dist=("uniform", -10.0, 30.0),
                               special=SPECIALS)
    y_ref, L_ref = oracle.lse_combine(o, l, "bf16")
    big = torch.empty((N, lse_stride), dtype=torch.float32, device=DEV)
    lses = big[:, :T * H].view(N, T, H)
    assert lses.stride(0) == lse_stride
    lses.copy_(f32_to_dev(l, DEV))
    y, L = lsec.lsec_combine_planes(to_dev(o, "bf16", DEV), lses, T, return_lse=True)
    torch.cuda.synchronize()
    del big, lses
    assert_output_close(y, y_ref, "bf16", max_abs_input(o, "bf16"), f"LSE stride {lse_stride}")
    assert_lse_close(L, L_ref, f"LSE stride {lse_stride}")
    del y, L
    _release()
