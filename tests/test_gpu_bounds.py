"""Every writing entry point writes its outputs and nothing else.

Each output (and global LSE) buffer is a view inside a larger allocation whose
bands before and after it hold a sentinel byte. After the call the bands must
be unchanged, the view must hold the same bits as the same call on plain
tensors (whose parity with the oracle the other GPU tests check), and the
inputs must be bit for bit what they were. One case per kernel family, with
ragged tails, multi-tile walks and odd widths.
"""
import math
import os

import pytest
import torch

import synth
from gpu_helpers import f32_to_dev, to_dev

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
TDT = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}
GUARD = 4096      # bytes before and after each output view
SENTINEL = 0x5A
SPECIALS = ((0.03, float("nan")), (0.03, float("inf")), (0.05, float("-inf")))


@pytest.fixture(scope="module")
def lsec():
    import lse_weighted_merge_combine_amd as m
    if not os.path.exists(m.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    m.load_library()
    return m


class Guarded:
    """A tensor of `shape` that starts GUARD + offset bytes into a buffer
    filled with the sentinel byte."""

    def __init__(self, shape, dtype, offset=0):
        esize = torch.empty(0, dtype=dtype).element_size()
        self.nbytes = math.prod(shape) * esize
        self.start = GUARD + offset
        self.raw = torch.full((self.start + self.nbytes + GUARD,), SENTINEL, dtype=torch.uint8,
                              device=DEV)
        self.t = self.raw[self.start:self.start + self.nbytes].view(dtype).view(shape)

    def bands_intact(self):
        return (bool(torch.all(self.raw[:self.start] == SENTINEL)) and
                bool(torch.all(self.raw[self.start + self.nbytes:] == SENTINEL)))


def _same_bits(a, b):
    return bool(torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8)))


def _inputs(N, B, H, D, dtype, seed):
    o, l = synth.custom_inputs(N, B, H, D, dtype=dtype, seed=seed, special=SPECIALS)
    return to_dev(o, dtype, DEV), f32_to_dev(l, DEV)


def _packed(lsec, N, B, Hl, D, dtype, seed):
    """A receive buffer [N, B, Hl, D + P]: what N ranks' packs deliver."""
    o, l = synth.custom_inputs(1, B, N * Hl, D, dtype=dtype, seed=seed, special=SPECIALS)
    return lsec.lsec_pack_send(to_dev(o[0], dtype, DEV), f32_to_dev(l[0], DEV), N)


def _check(results_guarded, results_plain, guards, what, inputs=()):
    """`inputs`: (tensor, its copy from before the calls) pairs."""
    torch.cuda.synchronize()
    for g in guards:
        assert g.bands_intact(), f"{what}: a write outside the output buffer"
    for a, b in zip(results_guarded, results_plain):
        assert _same_bits(a, b), f"{what}: guarded and plain results differ"
    for now, before in inputs:
        assert _same_bits(now, before), f"{what}: an input was written"


def _kept(*tensors):
    return [(t, t.clone()) for t in tensors]


@pytest.mark.parametrize("N,B,H,D,dtype,out_f32", [
    (8, 37, 5, 128, "bf16", False),    # tiled S = 1, ragged last block
    (8, 4095, 32, 128, "bf16", False),  # tiled, larger S, ragged
    (8, 2047, 16, 512, "bf16", False),  # a wave per row, ragged
    (5, 1001, 7, 256, "f16", False),   # N at run time
    (1, 5, 3, 512, "bf16", False),     # row kernel, N = 1
    (20, 6, 4, 128, "bf16", False),    # row kernel, N > 16
    (3, 5, 2, 3, "f16", False),        # element kernel
    (4, 300, 8, 256, "bf16", True),    # fp32 result, split loads
    (4, 100, 8, 128, "f32", False),    # fp32 partials
])
def test_combine_writes_only_its_outputs(lsec, N, B, H, D, dtype, out_f32):
    print(f"[case] combine bounds N={N} B={B} H={H} D={D} {dtype} out_f32={out_f32}", flush=True)
    og, lg = _inputs(N, B, H, D, dtype, seed=N * 7 + B)
    kept = _kept(og, lg)
    rdt = torch.float32 if (out_f32 or dtype == "f32") else TDT[dtype]
    out, out_lse = Guarded((B, H, D), rdt), Guarded((B, H), torch.float32)
    kw = {"out_dtype": torch.float32} if out_f32 else {}
    lsec.lsec_combine(og, lg, return_lse=True, out=out.t, out_lse=out_lse.t, **kw)
    y, L = lsec.lsec_combine(og, lg, return_lse=True, **kw)
    _check((out.t, out_lse.t), (y, L), (out, out_lse), "combine", kept)


@pytest.mark.parametrize("N,B,Hl,D,dtype", [
    (8, 64, 8, 128, "bf16"),   # span kernel
    (8, 64, 8, 128, "f32"),    # fp32 span kernel
    (8, 63, 3, 128, "bf16"),   # rows not a multiple of 4: tiled kernel on packed rows
    (17, 10, 4, 128, "f16"),   # N > 16: row kernel on packed rows
    (4, 9, 3, 6, "bf16"),      # element kernel
])
def test_unpack_combine_and_unpack_write_only_their_outputs(lsec, N, B, Hl, D, dtype):
    print(f"[case] receive-side bounds N={N} B={B} Hl={Hl} D={D} {dtype}", flush=True)
    recv = _packed(lsec, N, B, Hl, D, dtype, seed=B + D)
    kept = _kept(recv)
    out, out_lse = Guarded((B, Hl, D), TDT[dtype]), Guarded((B, Hl), torch.float32)
    lsec.lsec_unpack_combine(recv, return_lse=True, out=out.t, out_lse=out_lse.t)
    y, L = lsec.lsec_unpack_combine(recv, return_lse=True)
    _check((out.t, out_lse.t), (y, L), (out, out_lse), "unpack_combine", kept)
    outs, lses = Guarded((N, B, Hl, D), TDT[dtype]), Guarded((N, B, Hl), torch.float32)
    lsec.lsec_unpack(recv, outputs=outs.t, lses=lses.t)
    uo, ul = lsec.lsec_unpack(recv)
    _check((outs.t, lses.t), (uo, ul), (outs, lses), "unpack", kept)


@pytest.mark.parametrize("N,B,H,D,dtype,offset", [
    (4, 4099, 16, 128, "bf16", 0),  # pipelined LDS pack: 1025 tiles, the last one ragged
    (8, 37, 64, 128, "f16", 0),     # pipelined LDS pack: one tile per block
    (2, 257, 16, 1024, "f32", 0),   # fp32, 4-row tiles, 1028 of them
    (4, 37, 16, 128, "bf16", 4),    # send buffer 4-byte aligned only: row kernel
    (2, 5, 4, 5, "f16", 2),         # odd D: element kernel
])
def test_pack_writes_only_the_send_buffer(lsec, N, B, H, D, dtype, offset):
    print(f"[case] pack bounds N={N} B={B} H={H} D={D} {dtype} offset={offset}", flush=True)
    og, lg = _inputs(1, B, H, D, dtype, seed=H + D)
    kept = _kept(og, lg)
    P = lsec.lsec_pack_dim(TDT[dtype])
    send = Guarded((N, B, H // N, D + P), TDT[dtype], offset=offset)
    lsec.lsec_pack_send(og[0], lg[0], N, send=send.t)
    ref = lsec.lsec_pack_send(og[0], lg[0], N)
    _check((send.t,), (ref,), (send,), "pack_send", kept)


@pytest.mark.parametrize("token_dim", [1, 2])
def test_merge_writes_only_its_outputs(lsec, token_dim):
    print(f"[case] merge bounds token_dim={token_dim}", flush=True)
    N, A, C, D = 8, 37, 5, 128
    og, lg = _inputs(N, A, C, D, "bf16", seed=token_dim)
    kept = _kept(og, lg)
    y, L = lsec.lsec_merge(og, lg, token_dim, return_lse=True)
    out, out_lse = Guarded(tuple(y.shape), torch.bfloat16), Guarded(tuple(L.shape), torch.float32)
    lsec.lsec_merge(og, lg, token_dim, return_lse=True, out=out.t, out_lse=out_lse.t)
    _check((out.t, out_lse.t), (y, L), (out, out_lse), "merge", kept)


def test_correct_partial_writes_only_its_outputs(lsec):
    print("[case] corrected partial bounds", flush=True)
    N, B, H, D = 8, 50, 16, 512
    og, lg = _inputs(N, B, H, D, "bf16", seed=5)
    kept = _kept(og, lg)
    out, out_lse = Guarded((B, H, D), torch.bfloat16), Guarded((B, H), torch.float32)
    lsec.lsec_correct_partial(lg, 3, og[3], return_lse=True, out=out.t, out_lse=out_lse.t)
    y, L = lsec.lsec_correct_partial(lg, 3, og[3], return_lse=True)
    _check((out.t, out_lse.t), (y, L), (out, out_lse), "correct_partial", kept)


def test_combine_planes_writes_only_its_outputs(lsec):
    """The first T of T_max tokens of each plane: only [T, H, D] is written."""
    print("[case] combine_planes bounds", flush=True)
    W, Tmax, T, H, D = 8, 96, 61, 8, 128
    og, lg = _inputs(W, Tmax, H, D, "bf16", seed=9)
    kept = _kept(og, lg)
    out, out_lse = Guarded((T, H, D), torch.bfloat16), Guarded((T, H), torch.float32)
    lsec.lsec_combine_planes(og, lg, T, return_lse=True, out=out.t, out_lse=out_lse.t)
    y, L = lsec.lsec_combine_planes(og, lg, T, return_lse=True)
    _check((out.t, out_lse.t), (y, L), (out, out_lse), "combine_planes", kept)
    qsl = torch.tensor([0, 20, 45], dtype=torch.int32, device=DEV)
    out2, lse2 = Guarded((T, H, D), torch.bfloat16), Guarded((T, H), torch.float32)
    lsec.lsec_combine_planes(og, lg, T, return_lse=True, out=out2.t, out_lse=lse2.t,
                             query_start_loc=qsl)
    torch.cuda.synchronize()
    assert out2.bands_intact() and lse2.bands_intact(), "combine_planes_valid: a stray write"
    assert _same_bits(out2.t[:45], y[:45]) and _same_bits(lse2.t[:45], L[:45])
    pad = out2.raw[out2.start + 45 * H * D * 2:out2.start + out2.nbytes]
    lpad = lse2.raw[lse2.start + 45 * H * 4:lse2.start + lse2.nbytes]
    assert bool(torch.all(pad == SENTINEL)) and bool(torch.all(lpad == SENTINEL)), \
        "combine_planes_valid wrote a padding row"
