"""The measurement aids of include/lsec_floor.h on the GPU: the plain read
touches every byte once (its per-block XORs match numpy's), the plain copy
reproduces its source bit for bit and writes nothing past it, and the empty
launch runs. They are not part of the combine; bench.py times the combining
kernels against them."""
import os

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
BLOCK_BYTES = 16384  # one sink word per 16 KiB of input


@pytest.fixture(scope="module")
def lsec():
    import lse_weighted_merge_combine_amd as m
    if not os.path.exists(m.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    m.load_library()
    return m


def _xor_words(a: np.ndarray) -> int:
    return int(np.bitwise_xor.reduce(a.view(np.uint32))) if a.size else 0


@pytest.mark.parametrize("nbytes", [16, 4096, BLOCK_BYTES, 3 * BLOCK_BYTES + 48,
                                    (1 << 20) + 16 * 37, 64 << 20])
def test_floor_read_touches_every_byte(lsec, nbytes):
    print(f"[case] floor_read {nbytes} bytes", flush=True)
    rng = np.random.default_rng(nbytes)
    host = rng.integers(0, 2**32, size=nbytes // 4, dtype=np.uint32)
    src = torch.from_numpy(host.view(np.int32)).to(DEV)
    sink = lsec.lsec_floor_read(src)
    torch.cuda.synchronize()
    got = sink.cpu().numpy().view(np.uint32)
    nblk = -(-nbytes // BLOCK_BYTES)
    assert got.size == nblk
    for b in range(nblk):
        want = _xor_words(host[b * BLOCK_BYTES // 4:(b + 1) * BLOCK_BYTES // 4])
        assert int(got[b]) == want, f"block {b}"


def test_floor_read_rejects_ragged_bytes(lsec):
    with pytest.raises(ValueError):
        lsec.lsec_floor_read(torch.zeros(3, dtype=torch.int32, device=DEV))


def test_floor_read_empty_input(lsec):
    sink = torch.full((1,), 7, dtype=torch.int32, device=DEV)
    lsec.lsec_floor_read(torch.zeros(0, dtype=torch.int32, device=DEV), sink)
    torch.cuda.synchronize()
    assert int(sink.item()) == 7  # nothing launched, nothing written


def test_floor_empty_launch(lsec):
    s = torch.cuda.Stream(DEV)
    for _ in range(3):
        lsec.lsec_floor_empty(DEV)
        lsec.lsec_floor_empty(DEV, stream=s)
    torch.cuda.synchronize()


@pytest.mark.parametrize("nbytes", [16, 4096, 3 * BLOCK_BYTES + 48, (1 << 20) + 16 * 37])
def test_floor_copy_is_exact(lsec, nbytes):
    print(f"[case] floor_copy {nbytes} bytes", flush=True)
    rng = np.random.default_rng(nbytes + 1)
    host = rng.integers(0, 2**32, size=nbytes // 4, dtype=np.uint32)
    src = torch.from_numpy(host.view(np.int32)).to(DEV)
    guard = torch.full((nbytes // 4 + 64,), -7, dtype=torch.int32, device=DEV)
    dst = guard[:nbytes // 4]
    lsec.lsec_floor_copy(src, dst)
    torch.cuda.synchronize()
    got = guard.cpu().numpy()
    assert np.array_equal(got[:nbytes // 4].view(np.uint32), host)
    assert np.all(got[nbytes // 4:] == -7)  # nothing written past the end


def test_floor_copy_rejects_bad_sizes(lsec):
    a = torch.zeros(8, dtype=torch.int32, device=DEV)
    with pytest.raises(ValueError):
        lsec.lsec_floor_copy(a, torch.zeros(4, dtype=torch.int32, device=DEV))
    with pytest.raises(ValueError):
        lsec.lsec_floor_copy(a[:3], torch.zeros(3, dtype=torch.int32, device=DEV))


def test_time_next_launch_times_one_kernel(lsec):
    """lsec_time_next_launch: the armed launch records its own start and end;
    a 256 MiB read takes about 40 us at 6.5-7 TB/s, and the dispatch-timed
    duration is positive and not above the time between event markers around
    the same launch. Only the armed launch is timed (the next one leaves the
    pair as it was), and the results of a timed call are those of a plain one."""
    print("[case] lsec_time_next_launch", flush=True)
    src = torch.ones((256 << 20) // 4, dtype=torch.int32, device=DEV)
    sink = torch.empty(lsec.load_library().lsec_floor_read_blocks(256 << 20), dtype=torch.int32,
                       device=DEV)
    lsec.lsec_floor_read(src, sink)  # warm up
    timer = lsec.LaunchTimer(2)
    try:
        for i in range(2):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            timer.arm(i)
            lsec.lsec_floor_read(src, sink)
            b.record()
            torch.cuda.synchronize()
            k_ms, m_ms = timer.elapsed_ms(i), a.elapsed_time(b)
            print(f"dispatch {k_ms * 1e3:.1f} us, markers {m_ms * 1e3:.1f} us", flush=True)
            assert 0.0 < k_ms <= m_ms + 1e-3
            assert k_ms < 1.0  # 256 MiB in well under a millisecond
        # an unarmed launch does not touch the pairs
        before = timer.elapsed_ms(1)
        lsec.lsec_floor_read(src, sink)
        torch.cuda.synchronize()
        assert timer.elapsed_ms(1) == before
        # armed and disarmed: the next launch is plain
        timer.arm(0)
        timer.disarm()
        lsec.lsec_floor_empty()
        torch.cuda.synchronize()
    finally:
        timer.close()
    # the words the read produced are the same with and without timing
    plain = lsec.lsec_floor_read(src)
    torch.cuda.synchronize()
    assert torch.equal(plain, sink)


def test_timed_launches_of_the_hot_path_match_plain_ones(lsec):
    """A combine, a pack and an unpack + combine launched with events armed
    (hipExtLaunchKernelGGL) produce the same bits as plain launches, and each
    armed pair times exactly its own call's kernel."""
    import synth
    print("[case] timed hot-path launches", flush=True)
    N, B, H, D = 8, 512, 16, 128
    o, l = synth.custom_inputs(N, B, H, D, dtype="bf16", seed=71)
    og = torch.from_numpy(o.view(np.int16)).view(torch.bfloat16).to(DEV)
    lg = torch.from_numpy(l).to(DEV)
    ref_y, ref_L = lsec.lsec_combine(og, lg, return_lse=True)
    send_ref = lsec.lsec_pack_send(og[0], lg[0], N)
    uc_ref = lsec.lsec_unpack_combine(send_ref, return_lse=True)
    torch.cuda.synchronize()
    timer = lsec.LaunchTimer(3)
    try:
        timer.arm(0)
        y, L = lsec.lsec_combine(og, lg, return_lse=True)
        timer.arm(1)
        send = lsec.lsec_pack_send(og[0], lg[0], N)
        timer.arm(2)
        uy, uL = lsec.lsec_unpack_combine(send, return_lse=True)
        torch.cuda.synchronize()
        assert all(timer.elapsed_ms(i) > 0.0 for i in range(3))
    finally:
        timer.close()
    for a, b in ((y, ref_y), (uy, uc_ref[0]), (send, send_ref)):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    for a, b in ((L, ref_L), (uL, uc_ref[1])):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))
