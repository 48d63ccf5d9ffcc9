#!/usr/bin/env python3
"""Throughput of the LSE-weighted combine on one MI355X.

One step is one pass of the hot path over one batch of synthetic input that is
already resident in HBM:

* ``large_batch`` (default): lsec_combine of N=16 partial outputs
  [16, 16384, 32, 128] bf16 + LSEs [16, 16384, 32] (base e, global LSE
  returned) -- the largest workload; 2.3 GB per step, far beyond the 256 MB
  last-level cache, so every step streams from HBM.
* ``mla_decode``: lsec_combine, N=8 [8, 4096, 16, 512] bf16, base 2.
* ``fp16_base2``: lsec_combine, N=4 [4, 256, 32, 128] fp16, base 2, LSE out.
* ``packed``: one rank's lsec_pack_send ([2048, 64, 128] -> [8, 2048, 8, 130])
  followed by lsec_unpack_combine of an 8-rank receive buffer (the exchange
  in between is not part of a single GPU's work).
* ``merge_heads``: lsec_merge of received planes [8, 8, 2048, 128] bf16 into
  token-major [2048, 8, 128] (the head-scattered exchange of the Ascend merge).
* ``ag_correct``: lsec_correct_partial of rank 3's [4096, 16, 512] bf16 partial
  with the gathered LSEs [8, 4096, 16] (the local step of an all-gather +
  reduce-scatter combine).
* ``mla_decode_f32``: lsec_combine of fp32 partials [8, 4096, 16, 512], base 2.
* ``direct_planes``: lsec_combine_planes over one ubatch slot of a direct
  exchange's receive buffer: 8 planes of [4096, 8, 128] bf16 of which the
  first 2048 tokens are combined into [2048, 8, 128] (+ LSE).
* ``packed_f32``: the ``packed`` pair on fp32 outputs (packed rows of D + 1
  fp32 elements, the LSE in the last).

``--out-f32`` asks the combine and corrected-partial workloads for an fp32
result from 16-bit partials (the promoted dtype of the page's CPU combine)
instead of a result in the input dtype.

The library's measurement aids (include/lsec_floor.h) are timed under the
same protocol after the steps (``--no-floor`` skips them): a launch of one
wave that does nothing, and for each kernel of the step a plain streaming read
of as many bytes as that kernel moves and a plain copy of half of them. They bound what any kernel can reach on
the same box, process and cache state, and appear in the JSON line as
``floor``.

Workloads under 1 GiB are timed cold: a 1 GiB buffer is rewritten before each
step, outside the timed events. Kernel time comes from HIP events recorded on
the stream the kernels run on (torch's current stream). The JSON line also
carries the roofline of the dominant kernel and the CPU oracle's throughput on
the host cores (a baseline for context, not a target).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0  # MI355X HBM3E peak, GB/s
METRIC = "LSE-combine achieved HBM GB/s and (token·head) rows/s; % of peak HBM BW"
KERNEL_DIR = os.path.join(ROOT, "lse_weighted_merge_combine_amd", "csrc")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# Algorithmic HBM bytes per launch: every input byte read once, every output
# byte written once. s / os = element bytes of the partials / of the result;
# a packed row is D * s + 4 bytes (the LSE takes 4 / s elements).
def combine_bytes(N, B, H, D, s=2, return_lse=False, os_=None):
    os_ = s if os_ is None else os_
    return N * B * H * (D * s + 4) + B * H * D * os_ + (B * H * 4 if return_lse else 0)


def unpack_combine_bytes(N, B, Hl, D, s=2, return_lse=False, os_=None):
    os_ = s if os_ is None else os_
    return N * B * Hl * (D * s + 4) + B * Hl * D * os_ + (B * Hl * 4 if return_lse else 0)


def pack_bytes(N, B, H, D, s=2):
    return B * H * (D * s + 4) + B * H * (D * s + 4)


def source_sha() -> str:
    """SHA-256 of the kernel sources' code (every csrc/*.hip and *.h, in name
    order, except lsec_floor.hip: the measurement aids, which share no code
    with the combining kernels): comments, trailing blanks and empty lines
    removed, so that only a change to the code (not to its comments)
    invalidates counters taken on it."""
    import re
    parts = []
    for name in sorted(os.listdir(KERNEL_DIR)):
        if not name.endswith((".hip", ".h")) or name == "lsec_floor.hip":
            continue
        with open(os.path.join(KERNEL_DIR, name)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        lines = [re.sub(r"//.*$", "", ln).rstrip() for ln in text.splitlines()]
        parts.append(name + "\n" + "\n".join(ln for ln in lines if ln.strip()))
    return hashlib.sha256("\n".join(parts).encode()).hexdigest()


def load_traffic(workload: str, kernel: str):
    """HBM bytes per launch from committed rocprofv3 PMC counters, if they were
    taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256") != source_sha() or rec.get("kernel") != kernel:
        return None
    return rec.get("traffic_bytes_per_launch")


def traffic_record(bench_log: str, fetch_dir: str, write_dir: str, commit: str) -> dict:
    """Build profiles/traffic_<workload>.json from two rocprofv3 PMC runs of the
    same bench command with --copy-calibration (FETCH_SIZE, then WRITE_SIZE,
    in KiB per dispatch) and that command's JSON line. The counters are scaled
    by what they read for the run's own 1 GiB device copies (the last three
    __amd_rocclr_copyBuffer dispatches), and averaged over the dominant
    kernel's dispatches (matched on the first word of its bench name)."""
    import csv
    import glob

    with open(bench_log) as f:
        line = json.loads(f.read().strip().splitlines()[-1])
    workload = line["config"]["workload"] + \
        ("_f32out" if line["config"].get("result_dtype") == "f32" else "")
    kernel = line["roofline"]["kernel"]
    symbol = kernel.split()[0]

    def counters(d, symbol):
        files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        if len(files) != 1:
            raise SystemExit(f"expected one counter_collection.csv under {d}, found {len(files)}")
        with open(files[0]) as f:
            rows = sorted(csv.DictReader(f), key=lambda r: int(r["Dispatch_Id"]))
        mine = [float(r["Counter_Value"]) for r in rows
                if symbol + "<" in r["Kernel_Name"] or symbol + "(" in r["Kernel_Name"]]
        copies = [float(r["Counter_Value"]) for r in rows
                  if r["Kernel_Name"].startswith("__amd_rocclr_copyBuffer")][-3:]
        if not mine or len(copies) != 3:
            raise SystemExit(f"{d}: {len(mine)} dispatches of {symbol}, {len(copies)} copies")
        return mine, sum(copies) / 3

    fetch, fetch_copy = counters(fetch_dir, symbol)
    write, write_copy = counters(write_dir, symbol)
    gib_kib = float(1 << 20)
    ff, wf = fetch_copy / gib_kib, write_copy / gib_kib
    f_kib, w_kib = sum(fetch) / len(fetch), sum(write) / len(write)
    traffic = int(round((f_kib / ff + w_kib / wf) * 1024))
    alg = line["roofline"]["bytes_per_launch"]
    per_kernel = []
    for k in line["kernels"]:
        kf, _ = counters(fetch_dir, k["kernel"].split()[0])
        kw, _ = counters(write_dir, k["kernel"].split()[0])
        t = int(round((sum(kf) / len(kf) / ff + sum(kw) / len(kw) / wf) * 1024))
        per_kernel.append({"kernel": k["kernel"], "traffic_bytes_per_launch": t,
                           "algorithmic_bytes_per_launch": k["bytes"],
                           "traffic_over_algorithmic": round(t / k["bytes"], 4)})
    return {
        "workload": workload, "kernel": kernel, "source_sha256": source_sha(),
        "source_sha256_of": "every csrc/*.hip and *.h except lsec_floor.hip, in name order, "
                            "with comments and blank lines removed (bench.source_sha)",
        "counters_taken_at_commit": commit,
        "fetch_size_kib_per_dispatch": f_kib, "write_size_kib_per_dispatch": w_kib,
        "dispatches": min(len(fetch), len(write)),
        "copy_calibration": {"bytes_read": 1 << 30, "bytes_written": 1 << 30,
                             "fetch_size_kib": fetch_copy, "write_size_kib": write_copy,
                             "fetch_factor": ff, "write_factor": wf},
        "traffic_bytes_per_launch": traffic, "algorithmic_bytes_per_launch": alg,
        "traffic_over_algorithmic": round(traffic / alg, 4),
        "per_kernel": per_kernel,
        "commands": [
            f"cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc {c} --output-format csv -d "
            f"<outdir>/{c}_{workload} -o pmc -- python3 <repo>/bench.py --workload "
            f"{line['config']['workload']}{' --out-f32' if workload.endswith('_f32out') else ''} "
            "--steps 3 --warmup 1 --no-cpu-baseline --no-floor --copy-calibration"
            for c in ("FETCH_SIZE", "WRITE_SIZE")],
    }


# ---------------------------------------------------------------- workloads

def build_workload(name: str, dev, out_f32: bool = False, valid_tokens=None):
    """Inputs on the device, preallocated outputs and the step's kernels.
    valid_tokens (direct_planes only): the count of valid tokens is read by the
    kernels from a query_start_loc array in device memory; the other tokens of
    the padded step are neither read nor written.

    Returns a namespace: w (the workload), kind, info (the JSON config),
    kernels [(name, algorithmic bytes, launch fn)], rows, outputs (the step's
    output buffers by name), host (the host inputs the CPU leg needs),
    result_dtype and cpu_bytes (the algorithmic bytes of the oracle's pass)."""
    from types import SimpleNamespace

    import numpy as np
    import torch

    import lse_weighted_merge_combine_amd as lsec
    import synth

    w = synth.WORKLOADS[name]
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[w.dtype]
    s = 4 if w.dtype == "f32" else 2
    if out_f32 and w.kind not in ("combine", "correct"):
        raise SystemExit("--out-f32 applies to the combine and correct workloads only")
    if valid_tokens is not None and w.kind != "planes":
        raise SystemExit("--valid-tokens applies to the direct_planes workload only")
    odt = torch.float32 if out_f32 else tdt
    os_ = 4 if odt == torch.float32 else 2

    def dev_bits(a):
        a = np.ascontiguousarray(a)
        if s == 4:
            return torch.from_numpy(a.view(np.float32)).to(dev)
        return torch.from_numpy(a.view(np.int16)).view(tdt).to(dev)

    info = {"workload": name, "desc": w.desc, "N": w.N, "B": w.B, "H": w.H, "D": w.D,
            "io_dtype": w.dtype, "lse_base": "2" if w.base2 else "e",
            "return_lse": w.return_lse, "parallelism": "none (one GPU)"}
    if out_f32:
        info["result_dtype"] = "f32"
    if w.kind == "correct":
        rank = 3
        o, l = synth.combine_inputs(w)
        part = dev_bits(o[rank])
        lg = torch.from_numpy(l).to(dev)
        out = torch.empty((w.B, w.H, w.D), dtype=odt, device=dev)
        rows = w.B * w.H
        nbytes = w.N * rows * 4 + rows * w.D * s + rows * w.D * os_
        res = " -> f32" if out_f32 and s == 2 else ""
        kname = f"correct_tiled_kernel ({w.dtype}{res}, N={w.N}, D={w.D}, rank {rank})"

        def step():
            lsec.lsec_correct_partial(lg, rank, part, base_e=not w.base2, out=out, out_dtype=odt)

        kernels = [(kname, nbytes, step)]
        host = (o, l, rank)
        outputs = {"out": out}
        info["rank"] = rank
    elif w.kind == "planes":
        T_max = 2 * w.B
        o, l = synth.combine_inputs(w)
        buf = torch.zeros((w.N, T_max, w.H, w.D), dtype=tdt, device=dev)
        lbuf = torch.zeros((w.N, T_max, w.H), dtype=torch.float32, device=dev)
        buf[:, :w.B] = dev_bits(o)
        lbuf[:, :w.B] = torch.from_numpy(l).to(dev)
        out = torch.empty((w.B, w.H, w.D), dtype=tdt, device=dev)
        out_lse = torch.empty((w.B, w.H), dtype=torch.float32, device=dev)
        kname = f"{lsec.lsec_combine_path(w.N, w.B, w.H, w.D, dtype=tdt)} ({w.dtype}, N={w.N}, " \
                f"D={w.D}, {w.B} of {T_max} tokens per plane"
        if valid_tokens is None:
            K, qsl = w.B, None
            kname += ")"
        else:  # the step is padded to B tokens; K of them are valid
            K = min(max(int(valid_tokens), 0), w.B)
            qsl = torch.tensor([0, K], dtype=torch.int32, device=dev)
            kname += f", {K} valid by query_start_loc)"
            info["valid_tokens"] = K
        nbytes = combine_bytes(w.N, K, w.H, w.D, s, True) + (4 if qsl is not None else 0)

        def step():
            lsec.lsec_combine_planes(buf, lbuf, w.B, base_e=not w.base2, return_lse=True, out=out,
                                     out_lse=out_lse, query_start_loc=qsl)

        kernels = [(kname, nbytes, step)]
        host = (np.ascontiguousarray(o[:, :K]), np.ascontiguousarray(l[:, :K]))
        outputs = {"out": out[:K], "out_lse": out_lse[:K]}
        rows = K * w.H
        info["T_max"] = T_max
    elif w.kind == "merge":
        o, l = synth.combine_inputs(w)
        og, lg = dev_bits(o), torch.from_numpy(l).to(dev)
        out = torch.empty((w.H, w.B, w.D), dtype=tdt, device=dev)   # token-major [C, A, D]
        nbytes = combine_bytes(w.N, w.B, w.H, w.D, s, False)
        kname = f"{lsec.lsec_combine_path(w.N, w.B, w.H, w.D)} ({w.dtype}, N={w.N}, D={w.D}, " \
                f"token-major store)"

        def step():
            lsec.lsec_merge(og, lg, 2, base_e=True, return_lse=False, out=out)

        kernels = [(kname, nbytes, step)]
        host = (o, l)
        outputs = {"out": out}
        rows = w.B * w.H
        info["token_dim"] = 2
    elif w.kind == "combine":
        t0 = time.time()
        o, l = synth.combine_inputs(w)
        log(f"[bench] generated {name} inputs in {time.time() - t0:.1f}s")
        og, lg = dev_bits(o), torch.from_numpy(l).to(dev)
        out = torch.empty((w.B, w.H, w.D), dtype=odt, device=dev)
        out_lse = torch.empty((w.B, w.H), dtype=torch.float32, device=dev) if w.return_lse else None
        nbytes = combine_bytes(w.N, w.B, w.H, w.D, s, w.return_lse, os_)
        path = lsec.lsec_combine_path(w.N, w.B, w.H, w.D, dtype=tdt, out_dtype=odt)
        res = " -> f32" if out_f32 and s == 2 else ""
        kname = f"{path} ({w.dtype}{res}, N={w.N}, D={w.D})"

        def step():
            lsec.lsec_combine(og, lg, base_e=not w.base2, return_lse=w.return_lse, out=out,
                              out_lse=out_lse, out_dtype=odt)

        kernels = [(kname, nbytes, step)]
        host = (o, l)
        outputs = {"out": out}
        if out_lse is not None:
            outputs["out_lse"] = out_lse
        rows = w.B * w.H
    else:
        Hl = w.H // w.N
        outs = [synth.rank_inputs(w, r) for r in range(w.N)]
        a0 = dev_bits(outs[0][0])
        l0 = torch.from_numpy(outs[0][1]).to(dev)
        send = torch.empty((w.N, w.B, Hl, w.D + lsec.lsec_pack_dim(tdt)), dtype=tdt, device=dev)
        # rank 0's receive buffer: plane r is what rank r's pack put in its plane 0
        recv = torch.empty_like(send)
        for r in range(w.N):
            s_r = lsec.lsec_pack_send(dev_bits(outs[r][0]), torch.from_numpy(outs[r][1]).to(dev),
                                      w.N)
            recv[r].copy_(s_r[0])
        torch.cuda.synchronize()
        out = torch.empty((w.B, Hl, w.D), dtype=tdt, device=dev)
        out_lse = torch.empty((w.B, Hl), dtype=torch.float32, device=dev)

        def pack():
            lsec.lsec_pack_send(a0, l0, w.N, send=send)

        def unpack_combine():
            lsec.lsec_unpack_combine(recv, base_e=not w.base2, return_lse=True, out=out,
                                     out_lse=out_lse)

        send_align = next(a for a in (16, 8, 4, 2, 1) if send.data_ptr() % a == 0)
        pack_kernel = lsec.lsec_pack_path(w.N, w.B, w.H, w.D, tdt, a0.data_ptr() % 16 == 0,
                                          send_align)
        kernels = [(f"{pack_kernel} ({w.dtype})", pack_bytes(w.N, w.B, w.H, w.D, s), pack),
                   (f"{lsec.lsec_combine_path(w.N, w.B, Hl, w.D, packed=True, dtype=tdt)} "
                    f"({w.dtype}, N={w.N}, D={w.D}, packed rows)",
                    unpack_combine_bytes(w.N, w.B, Hl, w.D, s, True), unpack_combine)]
        host = ([a for a, _ in outs], [b for _, b in outs])
        outputs = {"send": send, "out": out, "out_lse": out_lse}
        rows = w.B * Hl
    rdt = "f32" if (out_f32 or w.dtype == "f32") else w.dtype
    cpu_bytes = combine_bytes(w.N, host[0].shape[1] if w.kind in ("combine", "planes") else w.B,
                              w.H, w.D, s, w.return_lse, os_)
    return SimpleNamespace(w=w, kind=w.kind, info=info, kernels=kernels, rows=rows,
                           outputs=outputs, host=host, result_dtype=rdt, cpu_bytes=cpu_bytes)


# ---------------------------------------------------------------- timing

def time_steps(kernels, steps, warmup, flush_bytes, dev, flush_read=False, dispatch=True):
    """Time `steps` steps after `warmup`. With flush_bytes, a buffer of that
    size is rewritten (or, with flush_read, summed) before each step, outside
    the timed events, so the step's inputs come from HBM. `kernels` is one
    step's list of (name, bytes, fn), or a list of such lists (input sets that
    hold the same work in different memory): step i then runs set i mod the
    number of sets. Every fn makes one library call, which launches one kernel.

    Returns a dict: "wall" (s, the timed loop on the host clock); "step_ms"
    (per step, by HIP events on the current stream, the one the kernels are
    launched on): without a flush the steps run back to back and one pair of
    events spans all of them, so every entry is the region's time divided by
    the steps; with a flush, events around each step, which include the
    event markers' own time; and, with `dispatch`, "kernel_ms": per kernel,
    the list of its launch times by the kernel's own dispatch
    (lsec_time_next_launch: events that the launch itself records), the
    kernel's duration as a kernel trace reports it (else None). Timing the
    dispatch adds work to the stream around each launch, so the step times of
    a dispatch-timed loop are not those of plain launches."""
    import torch

    import lse_weighted_merge_combine_amd as lsec

    sets = kernels if kernels and isinstance(kernels[0], list) else [kernels]
    flush = torch.ones(max(flush_bytes // 4, 1), dtype=torch.float32, device=dev) \
        if flush_bytes else None
    for i in range(warmup):
        for _, _, fn in sets[i % len(sets)]:
            fn()
    torch.cuda.synchronize()
    nk = len(sets[0])
    region = flush is None
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)]
          for _ in range(1 if region else steps)]
    timer = lsec.LaunchTimer(steps * nk) if dispatch else None
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    if flush is None:
        # Steps back to back: without a backlog the GPU would wait for the
        # host to enqueue each launch (small steps), or at least the first
        # one, after the region's start event (every step). A spin of ~2 ms,
        # or of ~20 ms + 0.1 ms per launch for steps under 1 GiB (about 2.4e6
        # cycles per ms on MI355X), lets the host get ahead before the first
        # step runs; wall_s then includes the spin, the events do not.
        small = sum(b for _, b, _ in sets[0]) < (1 << 30)
        torch.cuda._sleep(int(2.4e6 * ((20 + 0.1 * steps * nk) if small else 2)))
    if region:
        ev[0][0].record()
    for i in range(steps):
        if flush is not None:
            if flush_read:
                flush.sum()
            else:
                flush.fill_(float(i))
            ev[i][0].record()
        for k, (_, _, fn) in enumerate(sets[i % len(sets)]):
            if timer is not None:
                timer.arm(i * nk + k)
            fn()
        if not region:
            ev[i][1].record()
    if region:
        ev[0][1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    if region:
        step_ms = [ev[0][0].elapsed_time(ev[0][1]) / steps] * steps
    else:
        step_ms = [ev[i][0].elapsed_time(ev[i][1]) for i in range(steps)]
    kernel_ms = None
    if timer is not None:
        kernel_ms = [[timer.elapsed_ms(i * nk + k) for i in range(steps)] for k in range(nk)]
        timer.close()
    return {"wall": wall, "step_ms": step_ms, "kernel_ms": kernel_ms, "region": region}


def stats_us(ms):
    """Mean, median, p10 / p90, min / max of launch times given in ms, in µs."""
    import numpy as np

    a = np.asarray(ms, dtype=np.float64) * 1e3
    return {"mean_us": round(float(a.mean()), 3), "median_us": round(float(np.median(a)), 3),
            "p10_us": round(float(np.percentile(a, 10)), 3),
            "p90_us": round(float(np.percentile(a, 90)), 3),
            "min_us": round(float(a.min()), 3), "max_us": round(float(a.max()), 3)}


def time_floor(kernels, ktimes, steps, warmup, flush_bytes, dev, flush_read=False, rotate=0):
    """Time the measurement aids under the protocol of the workload's steps:
    an empty launch (one wave), and for each of the step's kernels a plain
    streaming read of as many bytes as that kernel moves (rounded down to 16)
    and a plain copy of half of them (as many bytes read as written), from
    buffers of their own. Each kernel's time per launch is reported as a
    multiple of both (means and medians of the kernels' own dispatch times,
    on both sides): the read bounds the combining kernels, the copy the pack
    and the corrected partial. With `rotate` the reads and copies cycle
    through that many buffers, as the steps cycle through their input sets."""
    import numpy as np
    import torch

    import lse_weighted_merge_combine_amd as lsec

    e_ms = time_steps([("empty", 0, lambda: lsec.lsec_floor_empty(dev))], steps, warmup,
                      flush_bytes, dev, flush_read)["kernel_ms"]
    reads = []
    n_sets = max(rotate, 1)
    for k, (name, nbytes, _) in enumerate(kernels):
        nbytes -= nbytes % 16
        bufs = [torch.ones(nbytes // 4, dtype=torch.int32, device=dev) for _ in range(n_sets)]
        sink = torch.empty(max(lsec.load_library().lsec_floor_read_blocks(nbytes), 1),
                           dtype=torch.int32, device=dev)
        r_ms = time_steps([[("read", nbytes, lambda b=b: lsec.lsec_floor_read(b, sink))]
                           for b in bufs], steps, warmup, flush_bytes, dev, flush_read)["kernel_ms"]
        del bufs, sink
        half = (nbytes // 2) - (nbytes // 2) % 16
        pairs = [(torch.ones(half // 4, dtype=torch.int32, device=dev),
                  torch.empty(half // 4, dtype=torch.int32, device=dev)) for _ in range(n_sets)]
        c_ms = time_steps([[("copy", 2 * half, lambda a=a, c=c: lsec.lsec_floor_copy(a, c))]
                           for a, c in pairs], steps, warmup, flush_bytes, dev,
                          flush_read)["kernel_ms"]
        del pairs
        read_ms, copy_ms = float(np.mean(r_ms[0])), float(np.mean(c_ms[0]))
        read_med, copy_med = float(np.median(r_ms[0])), float(np.median(c_ms[0]))
        kernel_ms_k, kernel_med = float(np.mean(ktimes[k])), float(np.median(ktimes[k]))
        reads.append({"kernel": name, "bytes": nbytes, "read_us": round(read_ms * 1e3, 3),
                      "read_median_us": round(read_med * 1e3, 3),
                      "read_GBps": round(nbytes / (read_ms * 1e-3) / 1e9, 1),
                      "kernel_over_read": round(kernel_ms_k / read_ms, 3),
                      "kernel_over_read_median": round(kernel_med / read_med, 3),
                      "copy_us": round(copy_ms * 1e3, 3),
                      "copy_median_us": round(copy_med * 1e3, 3),
                      "copy_GBps": round(2 * half / (copy_ms * 1e-3) / 1e9, 1),
                      "kernel_over_copy": round(kernel_ms_k / copy_ms, 3),
                      "kernel_over_copy_median": round(kernel_med / copy_med, 3)})
    return {"empty_launch_us": round(float(np.mean(e_ms[0])) * 1e3, 3), "reads": reads,
            "kernels": ["floor_empty_kernel", "floor_read_kernel", "floor_copy_kernel"],
            "timing": "the kernels' own dispatch times (lsec_time_next_launch), the same flush "
                      "protocol as the steps"}


# ---------------------------------------------------------------- CPU leg: oracle timing and parity
#
# The oracle (oracle/, plain fp64 C) is called from here only: the leg times
# it on the host's cores over the workload, and compares the output buffers
# the GPU produced from the same inputs (saved before the timed steps) with
# its results.

TOL = {"bf16": 8e-3, "f16": 1e-3, "f32": 2e-5}  # |y - y_oracle| <= TOL * M + 1e-6
LSE_TOL = 1e-5                                    # absolute


def host_threads() -> int:
    """The host threads used for oracle work: the CPUs this process may use,
    at most 16 (one GPU's share of a host's CPUs)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def max_abs_bits(bits, dtype: str) -> float:
    """Largest finite |value| of an array of element patterns (uint16 bf16 /
    fp16, float32 or uint32 fp32)."""
    import numpy as np

    b = np.ascontiguousarray(bits)
    if dtype == "f32":
        x = b.view(np.float32)
    elif dtype == "bf16":
        x = (b.astype(np.uint32) << 16).view(np.float32)
    else:
        x = b.view(np.float16)
    with np.errstate(invalid="ignore"):
        x = np.abs(x.astype(np.float64))
    x = x[np.isfinite(x)]
    return float(x.max()) if x.size else 0.0


def _f64(t):
    """A host tensor's values as float64 numpy."""
    return t.float().numpy().astype("float64")


class Check:
    """Running maximum of |gpu - oracle| for one output buffer."""

    def __init__(self, name, kind, dtype=None, M=None):
        self.name, self.kind, self.dtype, self.M = name, kind, dtype, M
        self.err, self.ok, self.n = 0.0, True, 0

    def values(self, got, ref):
        import numpy as np

        got = np.asarray(got, dtype=np.float64)
        ref = np.asarray(ref, dtype=np.float64)
        self.n += ref.size
        same_nan = np.array_equal(np.isnan(got), np.isnan(ref))
        inf = np.isinf(ref)
        fin = np.isfinite(ref)
        same_inf = np.array_equal(got[inf], ref[inf]) and bool(np.all(np.isfinite(got[fin])))
        if not (same_nan and same_inf):
            self.ok = False
        if fin.any():
            self.err = max(self.err, float(np.max(np.abs(got[fin] - ref[fin]))))
        if self.err > self.tol():
            self.ok = False

    def bits(self, got, ref):
        import numpy as np

        self.n += np.asarray(ref).size
        if not np.array_equal(np.asarray(got), np.asarray(ref)):
            self.ok = False

    def tol(self):
        if self.kind == "lse":
            return LSE_TOL
        if self.kind == "bits":
            return 0.0
        return TOL[self.dtype] * self.M + 1e-6

    def record(self):
        r = {"buffer": self.name, "elements": self.n, "ok": bool(self.ok)}
        if self.kind == "bits":
            r["rule"] = "bit-exact"
        else:
            r.update({"max_abs_err": self.err, "tol": self.tol(),
                      "rule": "|gpu - oracle| <= 1e-5" if self.kind == "lse" else
                      f"|gpu - oracle| <= {TOL[self.dtype]} * M + 1e-6, M = {self.M:.6g}"})
        return r


def _token_parts(B, parts):
    import numpy as np

    parts = max(1, min(parts, B))
    b = np.linspace(0, B, parts + 1).astype(int)
    return list(zip(b[:-1].tolist(), b[1:].tolist()))


def _run_parts(fn, parts, threads):
    """Run fn(part) for every part on `threads` host threads (ctypes drops the
    GIL inside the oracle); returns (wall seconds, results in part order)."""
    from concurrent.futures import ThreadPoolExecutor

    t0 = time.perf_counter()
    if threads == 1:
        res = [fn(p) for p in parts]
    else:
        with ThreadPoolExecutor(max_workers=threads) as ex:
            res = list(ex.map(fn, parts))
    return time.perf_counter() - t0, res


def cpu_leg(work, saved, threads: int, time_it: bool):
    """The oracle over the workload: parity of the GPU's saved output buffers
    and, with time_it (combine workloads), the CPU baseline: the oracle as it
    stands over the whole workload on one thread and on `threads` threads
    (token ranges split statically), median of 3 runs each."""
    import numpy as np

    import oracle

    oracle._load()
    w = work.w
    checks = []
    cpu = None
    if work.kind in ("combine", "planes"):
        o, l = work.host
        B = o.shape[1]
        rdt = work.result_dtype
        M = max_abs_bits(o, w.dtype)
        y_chk = Check("out", "values", rdt, M)
        l_chk = Check("out_lse", "lse") if "out_lse" in saved else None

        def part(r):
            a, b = r
            return oracle.lse_combine(np.ascontiguousarray(o[:, a:b]), np.ascontiguousarray(l[:, a:b]),
                                      w.dtype, base2=w.base2)

        def compare(parts, res):
            for (a, b), (y, L) in zip(parts, res):
                y_chk.values(_f64(saved["out"][a:b]), y)
                if l_chk is not None:
                    l_chk.values(_f64(saved["out_lse"][a:b]), L)

        many = _token_parts(B, threads)
        runs = []
        for _ in range(3 if time_it else 1):
            dt, res = _run_parts(part, many, threads)
            runs.append(dt)
        compare(many, res)
        del res
        checks = [y_chk] + ([l_chk] if l_chk is not None else [])
        if time_it and B:
            single = []
            for _ in range(3):
                dt, res = _run_parts(part, [(0, B)], 1)
                single.append(dt)
                del res
            nbytes = work.cpu_bytes
            rows = B * w.H

            def leg(ts, nthreads):
                med = float(np.median(ts))
                return {"value": round(nbytes / med / 1e9, 3), "unit": "GB/s",
                        "seconds": round(med, 4), "seconds_runs": [round(t, 4) for t in ts],
                        "rows_per_s": round(rows / med, 1), "threads": nthreads}
            multi = leg(runs, len(many))
            cpu = {"value": multi["value"], "unit": "GB/s", "cores": len(many), "kind": "oracle",
                   "sample": f"the whole workload ({rows} rows, N={w.N}, D={w.D}) through the "
                             f"fp64 C oracle, median of 3 runs: token ranges split statically over "
                             f"{len(many)} threads, and once more on 1 thread",
                   "seconds": multi["seconds"], "seconds_runs": multi["seconds_runs"],
                   "rows_per_s": multi["rows_per_s"], "single_thread": leg(single, 1),
                   "nproc": os.cpu_count(), "affinity_cpus": len(os.sched_getaffinity(0)),
                   "cpu_model": cpu_info()}
        else:
            cpu = {"oracle_s": round(runs[0], 4), "threads": len(many)}
    elif work.kind == "packed":
        outs, lses = work.host
        N, Hl = w.N, w.H // w.N
        t0 = time.perf_counter()
        send_ref = oracle.pack_send(outs[0], lses[0], N, w.dtype)
        c = Check("send", "bits")
        c.bits(saved["send"].view(_int_view(w.dtype)).numpy().view(send_ref.dtype), send_ref)
        so = np.stack([np.ascontiguousarray(a[:, :Hl]) for a in outs])
        sl = np.stack([np.ascontiguousarray(b[:, :Hl]) for b in lses])
        y, L = oracle.lse_combine(so, sl, w.dtype, base2=w.base2)
        yc = Check("out", "values", w.dtype, max_abs_bits(so, w.dtype))
        yc.values(_f64(saved["out"]), y)
        lc = Check("out_lse", "lse")
        lc.values(_f64(saved["out_lse"]), L)
        checks = [c, yc, lc]
        cpu = {"oracle_s": round(time.perf_counter() - t0, 4), "threads": 1}
    elif work.kind == "merge":
        o, l = work.host
        t0 = time.perf_counter()
        y, _ = oracle.merge(o, l, w.dtype, 2, base2=w.base2)
        yc = Check("out", "values", w.dtype, max_abs_bits(o, w.dtype))
        yc.values(_f64(saved["out"]), y)
        checks = [yc]
        cpu = {"oracle_s": round(time.perf_counter() - t0, 4), "threads": 1}
    elif work.kind == "correct":
        o, l, rank = work.host
        t0 = time.perf_counter()
        y, _ = oracle.correct_partial(l, rank, o[rank], w.dtype, base2=w.base2)
        yc = Check("out", "values", work.result_dtype, max_abs_bits(o[rank], w.dtype))
        yc.values(_f64(saved["out"]), y)
        checks = [yc]
        cpu = {"oracle_s": round(time.perf_counter() - t0, 4), "threads": 1}
    return [c.record() for c in checks], cpu


def _int_view(dtype):
    import torch

    return torch.int32 if dtype == "f32" else torch.int16


def cpu_info():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# ---------------------------------------------------------------- one workload, end to end

def snapshot(work):
    """Device copies of the step's output buffers (taken after one untimed
    run of the step, before any timing) and their host copies."""
    return {k: t.clone() for k, t in work.outputs.items()}


def same_bits(a, b) -> bool:
    import torch

    if a.dtype in (torch.bfloat16, torch.float16):
        return bool(torch.equal(a.view(torch.int16), b.view(torch.int16)))
    return bool(torch.equal(a.view(torch.int32), b.view(torch.int32)))


def measure(name, dev, steps, warmup, flush_mib, floor=True, warm_steps=0, out_f32=False,
            valid_tokens=None, cpu=True, time_cpu=False, rotate=0, flush_read=False,
            plain=False):
    """Build a workload, run its step once and save its outputs, time it,
    time the floor under the same protocol, check that the timed launches
    left the outputs bit for bit as saved, then run the CPU leg (parity of the
    saved outputs against the oracle; with time_cpu the CPU baseline).

    Kernel figures come from the kernels' own dispatch times over `steps`
    steps after `warmup`. With `plain`, the steps are then timed once more
    with plain launches, after the floor: the timed region of the headline,
    `steps` steps after `warmup` (see time_steps for its events). The GPU
    runs its first few milliseconds of work after an idle spell measurably
    slower (the first 20 launches of the large-batch combine 1-2 %), so the
    measurement passes run first."""
    import torch

    work = build_workload(name, dev, out_f32, valid_tokens)
    step_bytes = sum(b for _, b, _ in work.kernels)
    for _, _, fn in work.kernels:
        fn()
    torch.cuda.synchronize()
    saved_dev = snapshot(work)
    sets = [work.kernels]
    if rotate:
        sets += [build_workload(name, dev, out_f32, valid_tokens).kernels
                 for _ in range(rotate - 1)]
    if flush_mib < 0:
        flush_mib = 0 if rotate else (1024 if step_bytes < (1 << 30) else 0)
    log(f"[bench] {name}: {step_bytes / 1e6:.1f} MB per step, warmup {warmup}, steps {steps}, " +
        (f"{rotate} input sets in rotation" if rotate else
         f"flush {flush_mib} MiB{' (read)' if flush_read else ''}"))
    res = {"work": work, "step_bytes": step_bytes, "flush_mib": flush_mib}
    t = time_steps(sets, steps, warmup, flush_mib << 20, dev, flush_read)
    res["ktimes"] = t["kernel_ms"]
    if not plain:
        res["wall"], res["step_ms"], res["region"] = t["wall"], t["step_ms"], t["region"]
    if warm_steps:
        res["warm"] = time_steps(work.kernels, warm_steps, warmup, 0, dev)["kernel_ms"]
    if floor:
        res["floor"] = time_floor(work.kernels, res["ktimes"], steps, warmup, flush_mib << 20,
                                  dev, flush_read, rotate)
    if plain:
        # the timed region last: `warmup` untimed steps, then exactly `steps`
        # steps of plain launches
        t = time_steps(sets, steps, warmup, flush_mib << 20, dev, flush_read, dispatch=False)
        res["wall"], res["step_ms"], res["region"] = t["wall"], t["step_ms"], t["region"]
    torch.cuda.synchronize()
    res["unchanged"] = all(same_bits(work.outputs[k], saved_dev[k]) for k in saved_dev)
    res["ktimes_of_steps"] = [sum(kt[i] for kt in res["ktimes"]) for i in range(steps)]
    if cpu:
        saved = {k: t.cpu() for k, t in saved_dev.items()}
        del saved_dev
        log(f"[bench] {name}: oracle on the host (parity{', CPU baseline' if time_cpu else ''}) ...")
        res["parity"], res["cpu"] = cpu_leg(work, saved, host_threads(), time_cpu)
        bad = [c["buffer"] for c in res["parity"] if not c["ok"]]
        log(f"[bench] {name}: parity " + ("ok" if not bad else f"FAILED on {bad}"))
    return res


def kernel_records(res, target=None):
    """Per-kernel figures of a measured workload: the kernel's own dispatch
    times (µs: mean, median, p10, p90, min, max), GB/s and frac of the 8 TB/s
    peak by mean and by median, the floor ratios, and the mean and median of
    the same launches timed by event markers around them."""
    recs = []
    floor = res.get("floor")
    for k, (kname, kbytes, _) in enumerate(res["work"].kernels):
        st = stats_us(res["ktimes"][k])
        r = {"kernel": kname, "bytes": kbytes, **st,
             "GB/s": round(kbytes / (st["mean_us"] * 1e-6) / 1e9, 1),
             "GB/s_median": round(kbytes / (st["median_us"] * 1e-6) / 1e9, 1)}
        r["frac"] = round(r["GB/s"] / PEAK_HBM_GBS, 4)
        r["frac_median"] = round(r["GB/s_median"] / PEAK_HBM_GBS, 4)
        if target is not None:
            r["target_frac"] = target
        r["timing"] = "the kernel's own dispatch (lsec_time_next_launch)"
        if floor is not None:
            f = floor["reads"][k]
            r.update({"read_floor_us": f["read_us"], "kernel_over_read": f["kernel_over_read"],
                      "kernel_over_read_median": f["kernel_over_read_median"],
                      "copy_floor_us": f["copy_us"], "kernel_over_copy": f["kernel_over_copy"],
                      "kernel_over_copy_median": f["kernel_over_copy_median"]})
        if "warm" in res:
            ws = stats_us(res["warm"][k])
            r["warm"] = {"median_us": ws["median_us"], "p10_us": ws["p10_us"],
                         "p90_us": ws["p90_us"],
                         "GB/s_median": round(kbytes / (ws["median_us"] * 1e-6) / 1e9, 1),
                         "cache": "warm: no flush, steps back to back (inputs may sit in the "
                                  "256 MB Infinity Cache)"}
        recs.append(r)
    return recs


# Configurations the >= 80 % of peak HBM bandwidth target covers: the packed
# unpack + combine, the MLA decode combine and the large-batch combine.
TARGET = {("packed", 1): 0.80, ("mla_decode", 0): 0.80, ("large_batch", 0): 0.80}
SUITE = ["fp16_base2", "packed", "mla_decode"]
# Suite workloads also timed under the other cold protocol: this many input
# sets in rotation (a working set several times the 256 MB Infinity Cache) and
# no flush kernel before the steps.
SUITE_ROTATION = {"mla_decode": 8}


# ---------------------------------------------------------------- main

def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=None,
                    choices=["large_batch", "mla_decode", "fp16_base2", "packed", "small",
                             "merge_heads", "ag_correct", "mla_decode_f32", "packed_f32",
                             "direct_planes"],
                    help="time this workload only (default: large_batch, after the suite)")
    ap.add_argument("--no-suite", action="store_true",
                    help="default command: skip the suite of the other configurations")
    ap.add_argument("--suite-steps", type=int, default=100)
    ap.add_argument("--suite-warmup", type=int, default=10)
    ap.add_argument("--out-f32", action="store_true",
                    help="combine workloads: fp32 result from 16-bit partials")
    ap.add_argument("--flush-mib", type=int, default=-1,
                    help="cache flush before each step (default: 1024 MiB if the step's "
                         "working set is under 1 GiB, else none)")
    ap.add_argument("--valid-tokens", type=int, default=None,
                    help="direct_planes: combine only this many tokens, the count read by "
                         "the kernels from query_start_loc in device memory")
    ap.add_argument("--rotate", type=int, default=0, metavar="K",
                    help="workloads under 1 GiB: instead of a flush, cycle through K input "
                         "sets of the step (different memory), so each step's inputs were last "
                         "touched K - 1 steps before; pick K with K x the step's bytes well "
                         "above the 256 MB Infinity Cache (the steps then run back to back "
                         "behind a GPU spin that lets the host enqueue them all)")
    ap.add_argument("--flush-read", action="store_true",
                    help="flush by reading the buffer instead of rewriting it (leaves no "
                         "dirty lines in the caches)")
    ap.add_argument("--floor", dest="floor", action="store_true", default=True,
                    help="also time an empty launch and, per kernel, a plain read of its "
                         "bytes (the floor any kernel is measured against; on by default)")
    ap.add_argument("--no-floor", dest="floor", action="store_false",
                    help="skip the floor measurements")
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the CPU leg (the oracle: parity of the outputs and the CPU "
                         "baseline)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after timing, run a 1 GiB device copy (PMC calibration)")
    ap.add_argument("--traffic-record", nargs=3, metavar=("BENCH_LOG", "FETCH_DIR", "WRITE_DIR"),
                    help="no GPU: write profiles/traffic_<workload>.json from a bench JSON line "
                         "and the FETCH_SIZE / WRITE_SIZE PMC runs of the same command")
    ap.add_argument("--commit", default="unknown",
                    help="with --traffic-record: the commit the counters were taken on")
    args = ap.parse_args()

    if args.traffic_record:
        rec = traffic_record(*args.traffic_record, commit=args.commit)
        path = os.path.join(ROOT, "profiles", f"traffic_{rec['workload']}.json")
        with open(path, "w") as f:
            json.dump(rec, f, indent=1)
            f.write("\n")
        print(f"{path}: {rec['traffic_over_algorithmic']} x the algorithmic bytes")
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} (WORLD_SIZE={world}) is not "
              "supported; the combine's multi-GPU exchange is not part of this build.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import __graft_entry__
    __graft_entry__._ensure_built()
    import lse_weighted_merge_combine_amd as lsec
    lsec.load_library()
    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    use_cpu = not args.no_cpu_baseline
    name = args.workload or "large_batch"
    if args.rotate and (args.rotate < 2 or args.flush_mib > 0):
        raise SystemExit("--rotate K needs K >= 2 and no --flush-mib")

    # The suite of the other configurations runs first (cold, its own step
    # count), then the headline workload over exactly --steps steps.
    suite = []
    if args.workload is None and not args.no_suite:
        for sname in SUITE:
            r = measure(sname, dev, args.suite_steps, args.suite_warmup, -1, floor=args.floor,
                        warm_steps=args.suite_steps if sname == "packed" else 0, cpu=use_cpu)
            entry = {"workload": sname, "config": r["work"].info["desc"],
                     "steps": args.suite_steps, "warmup": args.suite_warmup,
                     "cache": f"cold: {r['flush_mib']} MiB written before each step, outside "
                              "the timed events",
                     "kernels": kernel_records(r), "outputs_unchanged_by_timed_steps":
                         r["unchanged"]}
            for k, rec in enumerate(entry["kernels"]):
                if (sname, k) in TARGET:
                    rec["target_frac"] = TARGET[(sname, k)]
            if use_cpu:
                entry["parity"] = r["parity"]
                entry["oracle"] = r["cpu"]
            # the outputs the parity check above saw, for the rotation's check below
            flush_outputs = {k: t.cpu() for k, t in r["work"].outputs.items()}
            del r
            torch.cuda.empty_cache()
            if sname in SUITE_ROTATION:
                sets = SUITE_ROTATION[sname]
                rr = measure(sname, dev, args.suite_steps, args.suite_warmup, -1,
                             floor=args.floor, cpu=False, rotate=sets)
                entry["rotation"] = {
                    "cache": f"cold: {sets} input sets in rotation "
                             f"({sets * rr['step_bytes'] / 1e9:.1f} GB), no flush kernel",
                    "kernels": kernel_records(rr),
                    "outputs_unchanged_by_timed_steps": rr["unchanged"],
                    # the first set holds the same seeded inputs as the flush run
                    "outputs_identical_to_the_flush_run": all(
                        same_bits(rr["work"].outputs[k].cpu(), t)
                        for k, t in flush_outputs.items())}
                del rr
                torch.cuda.empty_cache()
            del flush_outputs
            suite.append(entry)

    r = measure(name, dev, args.steps, args.warmup, args.flush_mib, floor=args.floor,
                out_f32=args.out_f32, valid_tokens=args.valid_tokens, cpu=use_cpu,
                time_cpu=use_cpu, rotate=args.rotate, flush_read=args.flush_read, plain=True)
    work = r["work"]
    step_ms = r["step_ms"]
    ms_per_step = sum(step_ms) / args.steps
    value = r["step_bytes"] / (ms_per_step * 1e-3) / 1e9
    log(f"[bench] wall {r['wall']:.3f}s for {args.steps} steps; kernels {sum(step_ms):.3f} ms")

    recs = kernel_records(r, TARGET.get((name, 0)))
    # dominant kernel: the one with the largest share of the step's time; its
    # launch duration is the kernel's own dispatch time (events the launch
    # itself records, as a kernel trace reports it)
    k = max(range(len(work.kernels)), key=lambda i: sum(r["ktimes"][i]))
    kname, kbytes, _ = work.kernels[k]
    k_ms = sum(r["ktimes"][k]) / args.steps
    achieved = kbytes / (k_ms * 1e-3) / 1e9
    roofline = {"bound": "hbm", "kernel": kname, "achieved": round(achieved, 1),
                "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                "bytes_per_launch": kbytes, "avg_launch_us": round(k_ms * 1e3, 3),
                "median_launch_us": stats_us(r["ktimes"][k])["median_us"],
                "launch_timing": "HIP events recorded by the kernel's own dispatch on the stream "
                                 "it runs on (lsec_time_next_launch), over --steps launches before "
                                 "the timed region; value and ms_per_step come from the timed "
                                 "region's plain launches",
                "traffic": load_traffic(name + ("_f32out" if args.out_f32 else ""), kname)}
    if args.floor:
        fl = r["floor"]
        log(f"[bench] floor: empty launch {fl['empty_launch_us']} us; " + "; ".join(
            f"plain read of {x['bytes'] / 1e6:.1f} MB {x['read_us']} us ({x['read_GBps']} GB/s), "
            f"copy of half {x['copy_us']} us ({x['copy_GBps']} GB/s)" for x in fl["reads"]))

    if args.copy_calibration:
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("[bench] copy calibration: 3 x 1 GiB device copies done")

    cpu = r.get("cpu") if use_cpu and work.kind in ("combine", "planes") else None
    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic (seeded counter-based generator)", "config": work.info,
        "rows_per_s": round(work.rows / (ms_per_step * 1e-3), 1),
        "pct_peak_hbm": round(100 * value / PEAK_HBM_GBS, 2),
        "step_bytes": r["step_bytes"], "cache_flush_mib": r["flush_mib"],
        "cache_flush_kind": (f"rotation over {args.rotate} input sets" if args.rotate else
                             ("read" if args.flush_read else "write") if r["flush_mib"] else
                             "none"),
        "wall_s": round(r["wall"], 4), "kernels": recs,
        "step_timing": ({"timing": "one pair of HIP events around the timed region's plain "
                                   "launches, back to back: ms_per_step is its time / steps",
                         "region_us": round(sum(step_ms) * 1e3, 3)} if r["region"] else
                        {**stats_us(step_ms), "timing": "HIP events around each step of the "
                                                        "timed region (plain launches)"}),
        "dispatch_step_timing": {**stats_us(r["ktimes_of_steps"]), "first_steps_us":
                                 [round(t * 1e3, 3) for t in r["ktimes_of_steps"][:5]],
                                 "timing": "the step's kernels by their own dispatch, over --steps "
                                           "launches before the timed region"},
        "roofline": roofline, "cpu_baseline": cpu,
        "outputs_unchanged_by_timed_steps": r["unchanged"],
    }
    if use_cpu:
        line["parity"] = r["parity"]
    if args.floor:
        line["floor"] = r["floor"]
    if suite:
        line["suite"] = suite
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
