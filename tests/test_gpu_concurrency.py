"""Concurrent calls: the library keeps no state between calls (no handles, no
workspace, no per-device caches), so host threads may call it at the same time
on different streams. ctypes releases the GIL around each call, so the
library's host code runs concurrently too. Every result is checked against the
oracle after all threads have finished.
"""
import os
import threading

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import assert_lse_close, assert_output_close, f32_to_dev, max_abs_input, to_dev

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
SPECIALS = ((0.02, float("nan")), (0.02, float("inf")), (0.02, float("-inf")))


@pytest.fixture(scope="module")
def lsec():
    import lse_weighted_merge_combine_amd as m
    if not os.path.exists(m.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    m.load_library()
    return m


def test_threads_on_separate_streams(lsec):
    print("[case] 4 host threads x 3 calls each on their own streams", flush=True)
    cases = [  # N, B, H, D, dtype, base2
        (16, 512, 32, 128, "bf16", False),
        (8, 256, 16, 512, "bf16", True),
        (4, 300, 8, 256, "f16", False),
        (3, 100, 12, 128, "f32", True),
    ]
    inputs, results, errors = [], [None] * len(cases), []
    for i, (N, B, H, D, dtype, base2) in enumerate(cases):
        o, l = synth.custom_inputs(N, B, H, D, dtype=dtype, seed=900 + i, special=SPECIALS)
        inputs.append((o, l, to_dev(o, dtype, DEV), f32_to_dev(l, DEV)))
    streams = [torch.cuda.Stream(device=DEV) for _ in cases]
    torch.cuda.synchronize()
    start = threading.Barrier(len(cases))

    def work(i):
        try:
            N, B, H, D, dtype, base2 = cases[i]
            _, _, og, lg = inputs[i]
            start.wait()
            outs = []
            for _ in range(3):
                outs.append(lsec.lsec_combine(og, lg, base_e=not base2, return_lse=True,
                                              stream=streams[i]))
            streams[i].synchronize()
            results[i] = outs
        except Exception as e:  # noqa: BLE001 - re-raised in the main thread
            errors.append(e)

    threads = [threading.Thread(target=work, args=(i,)) for i in range(len(cases))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=60)
    assert not any(t.is_alive() for t in threads), "a thread did not finish"
    if errors:
        raise errors[0]
    torch.cuda.synchronize()
    for i, (N, B, H, D, dtype, base2) in enumerate(cases):
        o, l, _, _ = inputs[i]
        y_ref, L_ref = oracle.lse_combine(o, l, dtype, base2)
        M = max_abs_input(o, dtype)
        first = results[i][0]
        for k, (y, L) in enumerate(results[i]):
            assert_output_close(y, y_ref, dtype, M, f"case {i} call {k}")
            assert_lse_close(L, L_ref, f"case {i} call {k}")
            idt = torch.int32 if y.dtype == torch.float32 else torch.int16
            assert torch.equal(y.view(idt), first[0].view(idt)), "repeated calls differ"
            assert torch.equal(L.view(torch.int32), first[1].view(torch.int32))
