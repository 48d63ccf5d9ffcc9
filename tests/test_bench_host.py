"""Host logic of bench.py (no GPU): the kernel-source hash that keys the PMC
traffic records, the record builder, the record lookup and the one-GPU guard."""
import csv
import json
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


@pytest.fixture
def kernel_copy(tmp_path, monkeypatch):
    d = tmp_path / "csrc"
    shutil.copytree(bench.KERNEL_DIR, d)
    monkeypatch.setattr(bench, "KERNEL_DIR", str(d))
    return d


def test_source_sha_keys_the_code_not_its_comments(kernel_copy):
    base = bench.source_sha()
    tiled = kernel_copy / "lsec_tiled.hip"
    text = tiled.read_text()
    tiled.write_text("// a new comment line\n" + text.replace("{", "{  /* note */", 1) + "\n\n")
    assert bench.source_sha() == base
    tiled.write_text(text.replace("kBlock", "kBlock ", 1).replace("1e-10f", "1e-9f", 1))
    assert bench.source_sha() != base


def test_source_sha_leaves_out_the_measurement_aids(kernel_copy):
    base = bench.source_sha()
    floor = kernel_copy / "lsec_floor.hip"
    floor.write_text(floor.read_text().replace("kFloorLoads = 4", "kFloorLoads = 8"))
    assert bench.source_sha() == base


def _write_counters(path, counter, rows):
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "pmc_counter_collection.csv"), "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for i, (name, value) in enumerate(rows, 1):
            w.writerow([i, name, counter, value])


def test_traffic_record_scales_by_the_copy_calibration(tmp_path):
    alg = 1000 * 1024
    line = {"config": {"workload": "packed"},
            "roofline": {"kernel": "pack_pipe_kernel (bf16)", "bytes_per_launch": alg},
            "kernels": [{"kernel": "pack_pipe_kernel (bf16)", "bytes": alg},
                        {"kernel": "combine_tiled_kernel S=1 (bf16, N=8, D=128, packed rows)",
                         "bytes": 2 * alg}]}
    log = tmp_path / "bench.log"
    log.write_text("[bench] something\n" + json.dumps(line) + "\n")
    gib_kib = float(1 << 20)
    pack = "void lsec_detail::(anonymous namespace)::pack_pipe_kernel<unsigned short>(...)"
    comb = "void lsec_detail::(anonymous namespace)::combine_tiled_kernel<0, 8, 16, 1, true, false>(...)"
    copy = "__amd_rocclr_copyBuffer"
    # FETCH counts 0.5 per KiB read, WRITE 1.0 per KiB written (as measured on the device)
    _write_counters(tmp_path / "f", "FETCH_SIZE",
                    [(copy, 7.0), (pack, 250.0), (comb, 1000.0), (pack, 250.0), (comb, 1010.0),
                     (copy, gib_kib / 2), (copy, gib_kib / 2), (copy, gib_kib / 2)])
    _write_counters(tmp_path / "w", "WRITE_SIZE",
                    [(copy, 7.0), (pack, 500.0), (comb, 40.0), (pack, 500.0), (comb, 40.0),
                     (copy, gib_kib), (copy, gib_kib), (copy, gib_kib)])
    rec = bench.traffic_record(str(log), str(tmp_path / "f"), str(tmp_path / "w"), "abc123")
    assert rec["workload"] == "packed"
    assert rec["kernel"] == "pack_pipe_kernel (bf16)"
    assert rec["counters_taken_at_commit"] == "abc123"
    assert rec["copy_calibration"]["fetch_factor"] == pytest.approx(0.5)
    assert rec["copy_calibration"]["write_factor"] == pytest.approx(1.0)
    assert rec["traffic_bytes_per_launch"] == (500 + 500) * 1024
    assert rec["traffic_over_algorithmic"] == pytest.approx(1.0)
    comb_rec = rec["per_kernel"][1]
    assert comb_rec["traffic_bytes_per_launch"] == round((2010 + 40) * 1024)
    assert rec["source_sha256"] == bench.source_sha()


def test_traffic_record_of_an_fp32_result_is_keyed_apart(tmp_path):
    line = {"config": {"workload": "ag_correct", "result_dtype": "f32"},
            "roofline": {"kernel": "correct_tiled_kernel (bf16 -> f32)", "bytes_per_launch": 1024},
            "kernels": [{"kernel": "correct_tiled_kernel (bf16 -> f32)", "bytes": 1024}]}
    log = tmp_path / "bench.log"
    log.write_text(json.dumps(line) + "\n")
    k = "void lsec_detail::(anonymous namespace)::correct_tiled_kernel<0, 64, 8, true>(...)"
    copies = [("__amd_rocclr_copyBuffer", 1.0)] * 3
    _write_counters(tmp_path / "f", "FETCH_SIZE", [(k, 0.5)] + copies)
    _write_counters(tmp_path / "w", "WRITE_SIZE", [(k, 0.5)] + copies)
    rec = bench.traffic_record(str(log), str(tmp_path / "f"), str(tmp_path / "w"), "x")
    assert rec["workload"] == "ag_correct_f32out"
    assert "--out-f32" in rec["commands"][0]


def test_load_traffic_needs_the_current_source_and_kernel(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    (tmp_path / "profiles").mkdir()
    rec = {"kernel": "k (bf16)", "source_sha256": bench.source_sha(),
           "traffic_bytes_per_launch": 1234}
    (tmp_path / "profiles" / "traffic_w.json").write_text(json.dumps(rec))
    assert bench.load_traffic("w", "k (bf16)") == 1234
    assert bench.load_traffic("w", "other kernel") is None
    assert bench.load_traffic("missing", "k (bf16)") is None
    rec["source_sha256"] = "0" * 64
    (tmp_path / "profiles" / "traffic_w.json").write_text(json.dumps(rec))
    assert bench.load_traffic("w", "k (bf16)") is None


def test_committed_traffic_records_are_used_only_on_their_sources():
    """A committed record taken on the kernels as they are now is within 10 %
    of the algorithmic bytes; one taken on other kernel sources is never
    reported (load_traffic gives None for it)."""
    d = os.path.join(ROOT, "profiles")
    names = [n for n in os.listdir(d) if n.startswith("traffic_") and n.endswith(".json")]
    assert names
    for n in names:
        with open(os.path.join(d, n)) as f:
            rec = json.load(f)
        assert 1.0 <= rec["traffic_over_algorithmic"] < 1.1, n
        got = bench.load_traffic(n[len("traffic_"):-len(".json")], rec["kernel"])
        if rec["source_sha256"] == bench.source_sha():
            assert got == rec["traffic_bytes_per_launch"], n
        else:
            assert got is None, n


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr


# ---------------------------------------------------------------- the CPU leg (oracle timing and parity)

def _fake_combine_work(N=3, B=40, H=4, D=128, dtype="bf16", base2=False):
    """A combine workload whose 'GPU' outputs are the oracle's own results
    rounded to the result dtype (no GPU here)."""
    from types import SimpleNamespace

    import numpy as np
    import torch

    import oracle
    import synth

    w = synth.Workload("fake", 77, "combine", N, B, H, D, dtype, ("normal", 0.0, 1.0),
                       ("uniform", -5.0, 15.0), special=((0.05, float("nan")),),
                       base2=base2, return_lse=True)
    o, l = synth.combine_inputs(w)
    y, L = oracle.lse_combine(o, l, dtype, base2=base2)
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16}[dtype]
    saved = {"out": torch.from_numpy(y).to(tdt), "out_lse": torch.from_numpy(L).float()}
    work = SimpleNamespace(w=w, kind="combine", host=(o, l), result_dtype=dtype,
                           cpu_bytes=bench.combine_bytes(N, B, H, D, 2, True))
    return work, saved, np


def test_cpu_leg_checks_every_row_and_times_the_oracle():
    work, saved, _ = _fake_combine_work()
    parity, cpu = bench.cpu_leg(work, saved, threads=3, time_it=True)
    assert [c["buffer"] for c in parity] == ["out", "out_lse"]
    assert all(c["ok"] for c in parity), parity
    assert parity[0]["elements"] == 40 * 4 * 128 and parity[1]["elements"] == 40 * 4
    assert cpu["kind"] == "oracle" and cpu["cores"] == 3 and cpu["unit"] == "GB/s"
    assert len(cpu["seconds_runs"]) == 3 and cpu["single_thread"]["threads"] == 1
    assert len(cpu["single_thread"]["seconds_runs"]) == 3
    assert cpu["nproc"] == os.cpu_count() and cpu["value"] > 0


@pytest.mark.parametrize("where", ["out", "out_lse", "nan"])
def test_cpu_leg_catches_a_wrong_output(where):
    import torch

    work, saved, np = _fake_combine_work(dtype="f16", base2=True)
    if where == "out":
        saved["out"][17, 2, 5] += 0.05            # beyond 1e-3 * M
    elif where == "out_lse":
        saved["out_lse"][39, 3] += 1e-3            # beyond 1e-5
    else:
        saved["out"][0, 0, 0] = float("nan")       # a NaN where the oracle has none
    parity, _ = bench.cpu_leg(work, saved, threads=2, time_it=False)
    bad = [c["buffer"] for c in parity if not c["ok"]]
    assert bad == (["out_lse"] if where == "out_lse" else ["out"]), parity
    del torch


def test_cpu_leg_packed_is_bit_exact():
    from types import SimpleNamespace

    import numpy as np
    import torch

    import oracle
    import synth

    w = synth.Workload("fake_packed", 78, "packed", 4, 24, 8, 128, "bf16", ("normal", 0.0, 1.0),
                       ("uniform", -5.0, 15.0), base2=False, return_lse=True)
    ranks = [synth.rank_inputs(w, r) for r in range(w.N)]
    outs, lses = [a for a, _ in ranks], [b for _, b in ranks]
    Hl = w.H // w.N
    send = oracle.pack_send(outs[0], lses[0], w.N)
    so = np.stack([a[:, :Hl] for a in outs])
    sl = np.stack([b[:, :Hl] for b in lses])
    y, L = oracle.lse_combine(so, sl, "bf16")
    saved = {"send": torch.from_numpy(send.view(np.int16)).view(torch.bfloat16),
             "out": torch.from_numpy(y).to(torch.bfloat16), "out_lse": torch.from_numpy(L).float()}
    work = SimpleNamespace(w=w, kind="packed", host=(outs, lses), result_dtype="bf16",
                           cpu_bytes=0)
    parity, _ = bench.cpu_leg(work, saved, threads=1, time_it=False)
    assert all(c["ok"] for c in parity), parity
    saved["send"].view(torch.int16)[1, 3, 0, 129] ^= 1  # one bit of an LSE tail
    parity, _ = bench.cpu_leg(work, saved, threads=1, time_it=False)
    assert [c["buffer"] for c in parity if not c["ok"]] == ["send"]


def test_step_statistics():
    st = bench.stats_us([0.001 * i for i in range(1, 101)])  # 1 .. 100 us
    assert st["median_us"] == pytest.approx(50.5)
    assert st["p10_us"] == pytest.approx(10.9) and st["p90_us"] == pytest.approx(90.1)
    assert st["mean_us"] == pytest.approx(50.5) and st["min_us"] == 1.0 and st["max_us"] == 100.0
