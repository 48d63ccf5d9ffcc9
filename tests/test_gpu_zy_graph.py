"""The library's calls inside a captured HIP graph.

The entry points allocate nothing and never synchronise, so a caller can
capture them on its stream and replay them (what a serving loop does to drop
the launch overhead of the small packed calls). The graph holds only this
library's kernels (the buffers are allocated and filled before capture); it
is replayed several times with eager work and synchronisations in between,
and every replay is checked against the eager results and the oracle.
"""
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import assert_lse_close, assert_output_close, bits_of, f32_to_dev, max_abs_input, to_dev

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


@pytest.fixture(scope="module")
def lsec():
    import lse_weighted_merge_combine_amd as m
    if not os.path.exists(m.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    m.load_library()
    return m


def test_pack_unpack_combine_and_combine_replayed_from_a_graph(lsec):
    print("[case] graph capture and replay", flush=True)
    N, B, H, D = 8, 64, 64, 128
    Hl = H // N
    a, l = synth.custom_inputs(1, B, H, D, seed=71)
    o, ol = synth.custom_inputs(N, B, Hl, D, seed=72, special=((0.05, float("-inf")),))
    attn, attn_lse = to_dev(a[0], "bf16", DEV), f32_to_dev(l[0], DEV)
    planes, plane_lses = to_dev(o, "bf16", DEV), f32_to_dev(ol, DEV)
    # every buffer exists before capture
    send = torch.empty((N, B, Hl, D + 2), dtype=torch.bfloat16, device=DEV)
    y_pk = torch.empty((B, Hl, D), dtype=torch.bfloat16, device=DEV)
    L_pk = torch.empty((B, Hl), dtype=torch.float32, device=DEV)
    y_c = torch.empty((B, Hl, D), dtype=torch.bfloat16, device=DEV)
    L_c = torch.empty((B, Hl), dtype=torch.float32, device=DEV)

    def step():
        lsec.lsec_pack_send(attn, attn_lse, N, send=send)
        lsec.lsec_unpack_combine(send, return_lse=True, out=y_pk, out_lse=L_pk)
        lsec.lsec_combine(planes, plane_lses, return_lse=True, out=y_c, out_lse=L_c)

    # eager reference (warm-up on a side stream, as graph capture requires)
    s = torch.cuda.Stream(device=DEV)
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    ref = [t.clone() for t in (send, y_pk, L_pk, y_c, L_c)]
    # the eager results themselves match the oracle
    assert np.array_equal(bits_of(ref[0]), oracle.pack_send(a[0], l[0], N))
    yr, Lr = oracle.unpack_combine(bits_of(ref[0]), D, "bf16")
    oo, _ = oracle.unpack(bits_of(ref[0]), D)
    assert_output_close(ref[1], yr, "bf16", max_abs_input(oo, "bf16"))
    assert_lse_close(ref[2], Lr)
    yc, Lc = oracle.lse_combine(o, ol, "bf16")
    assert_output_close(ref[3], yc, "bf16", max_abs_input(o, "bf16"))
    assert_lse_close(ref[4], Lc)

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for i in range(4):
        for t in (send, y_pk, L_pk, y_c, L_c):
            t.fill_(float("nan")) if t.dtype.is_floating_point else t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, want in zip((send, y_pk, L_pk, y_c, L_c), ref):
            assert torch.equal(got.view(torch.int16) if got.dtype == torch.bfloat16 else got.view(torch.int32),
                               want.view(torch.int16) if want.dtype == torch.bfloat16 else want.view(torch.int32)), \
                f"replay {i} differs from the eager result"
        # eager work between replays
        lsec.lsec_combine(planes, plane_lses)
        torch.cuda.synchronize()


def test_valid_count_changes_between_replays_of_one_graph(lsec):
    """A captured combine of receive planes padded to T tokens, replayed after
    the step's query_start_loc changes in device memory (written by an eager
    copy, outside the graph): each replay combines exactly the valid tokens and
    leaves the padding rows as they were."""
    print("[case] graph replay with a changing valid-token count", flush=True)
    W, T, H, D = 8, 512, 16, 128
    o, l = synth.custom_inputs(W, T, H, D, seed=73, special=((0.02, float("nan")),))
    planes, lplanes = to_dev(o, "bf16", DEV), f32_to_dev(l, DEV)
    qsl = torch.zeros(3, dtype=torch.int32, device=DEV)
    out = torch.empty((T, H, D), dtype=torch.bfloat16, device=DEV)
    out_lse = torch.empty((T, H), dtype=torch.float32, device=DEV)

    def step():
        lsec.lsec_combine_planes(planes, lplanes, T, return_lse=True, out=out, out_lse=out_lse,
                                 query_start_loc=qsl)

    qsl.copy_(torch.tensor([0, 100, 200], dtype=torch.int32))
    s = torch.cuda.Stream(device=DEV)
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    M = max_abs_input(o, "bf16")
    for offsets in ([0, 300, 511], [0, 7, 9], [0, 0, 0], [0, 256, 512], [0, 400, 700]):
        q = np.array(offsets, dtype=np.int32)
        qsl.copy_(torch.from_numpy(q))
        out.fill_(-7.0)
        out_lse.fill_(-7.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        y_ref, L_ref, tv = oracle.lse_combine_valid(o, l, q, "bf16")
        if tv:
            assert_output_close(out[:tv], y_ref, "bf16", M, f"offsets {offsets}")
            assert_lse_close(out_lse[:tv], L_ref, f"offsets {offsets}")
        assert bool(torch.all(out[tv:] == -7.0)) and bool(torch.all(out_lse[tv:] == -7.0)), \
            f"offsets {offsets}: a padding row was written"


FIRST_PACK_IN_CAPTURE = r"""
import sys
import torch
sys.path.insert(0, sys.argv[1])
import lse_weighted_merge_combine_amd as lsec
lsec.load_library()
dev = torch.device("cuda:0")
N, B, H, D = 8, 3000, 64, 128  # 192,000 send rows: 3,000 tiles, several per block
assert lsec.lsec_pack_path(N, B, H, D) == "pack_pipe_kernel"
gen = torch.Generator().manual_seed(5)
a = torch.randn(B, H, D, generator=gen).to(torch.bfloat16).to(dev)
l = (torch.rand(B, H, generator=gen) * 20 - 5).to(dev)
send = torch.empty((N, B, H // N, D + 2), dtype=torch.bfloat16, device=dev)
torch.cuda.synchronize()
graph = torch.cuda.CUDAGraph()
with torch.cuda.graph(graph):
    lsec.lsec_pack_send(a, l, N, send=send)  # the first pack of this process
for i in range(3):
    send.zero_()
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    ref = lsec.lsec_pack_send(a, l, N)
    torch.cuda.synchronize()
    assert torch.equal(send.view(torch.int16), ref.view(torch.int16)), f"replay {i}"
print("first pack captured: replays match the eager pack")
"""


def test_first_pack_of_a_process_inside_capture(lsec):
    """The pack sizes its persistent grid from the device's compute units,
    queried on the first pack call of a process; a process whose first pack is
    captured in a graph (run here in a fresh child process) must replay the
    same bytes as an eager pack."""
    import subprocess
    import sys
    print("[case] first pack of a fresh process inside graph capture", flush=True)
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    res = subprocess.run([sys.executable, "-c", FIRST_PACK_IN_CAPTURE, root],
                         capture_output=True, text=True, timeout=240)
    assert res.returncode == 0, res.stdout[-2000:] + res.stderr[-4000:]
    assert "replays match" in res.stdout
