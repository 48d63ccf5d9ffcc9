"""Seeded synthetic inputs shared by the oracle side and the HIP side.

This package draws random numbers and rounds them to storage formats; it holds
none of the combine's arithmetic. Both the CPU oracle and the GPU kernels read
the bytes it produces, so the two sides see identical inputs.

Streams are counter-based SplitMix64 (see ``synth.c``): element ``i`` of a
tensor is a pure function of ``(seed, workload id, tensor id, sub-stream, i)``,
so any slice of a tensor can be generated on its own and equals the same slice
of the whole tensor.

The workloads are the shapes the combine is specified and measured on:

==============  ======  ======  ====  ====  =====  ===========  =============  =====================
name            N       B       H     D     dtype  outputs      LSE            special LSE entries
==============  ======  ======  ====  ====  =====  ===========  =============  =====================
small           2       4       8     128   bf16   N(0,1)       U[-2,8] e      row (b=3,h=7) all -inf
fp16_base2      4       256     32    128   fp16   N(0,1)       U[0,20] 2      2% NaN, 2% +inf
packed          8       2048    64    128   bf16   N(0,1)       U[-5,15] e     none (per-rank [B,H,D])
mla_decode      8       4096    16    512   bf16   N(0,0.5)     N(10,3) 2      1% -inf
large_batch     16      16384   32    128   bf16   N(0,1)       U[-10,30] e    0.5% split NaN/+inf/-inf
merge_heads     8       8       2048  128   bf16   N(0,1)       U[-5,15] e     none (B = heads, H = tokens)
ag_correct      8       4096    16    512   bf16   N(0,0.5)     N(10,3) 2      1% -inf (rank 3's plane used)
==============  ======  ======  ====  ====  =====  ===========  =============  =====================

For ``packed`` the shape is one rank's ``[B, H, D]`` attention output plus its
``[B, H]`` LSE; rank ``r`` of ``N`` draws its own tensors (sub-stream ``r``).
``merge_heads`` is the received planes ``[N, A=8 heads, C=2048 tokens, D=128]``
of a head-scattered exchange (base e, no LSE), merged token-major.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB = os.path.join(_HERE, "libsynth.so")

_DIST = {"uniform": 0, "normal": 1}
_OUT = {"f64": 0, "f32": 1, "bf16": 2, "f16": 3}

# tensor ids inside one workload
T_OUTPUTS, T_LSE, T_SPECIAL = 1, 2, 3


def build() -> str:
    """Compile ``synth.c`` into ``libsynth.so`` (plain gcc, no fast-math)."""
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-shared", "-fPIC",
           "-o", _LIB + ".tmp", _SRC, "-lm", "-lpthread"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        # LSEC_SYNTH_LIB: another build of the same source (the sanitizer test's)
        path = os.environ.get("LSEC_SYNTH_LIB")
        if path is None:
            path = _LIB
            if not os.path.exists(path):
                build()
        lib = ctypes.CDLL(path)
        lib.synth_key.restype = ctypes.c_uint64
        lib.synth_key.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint32]
        lib.synth_hash.restype = ctypes.c_uint64
        lib.synth_hash.argtypes = [ctypes.c_uint64, ctypes.c_uint64]
        lib.synth_fill.restype = ctypes.c_int
        lib.synth_fill.argtypes = [ctypes.c_uint64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
                                   ctypes.c_double, ctypes.c_double, ctypes.c_int, ctypes.c_void_p,
                                   ctypes.c_int]
        lib.synth_u01.restype = ctypes.c_int
        lib.synth_u01.argtypes = [ctypes.c_uint64, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                                  ctypes.c_int]
        lib.synth_f32_to_bf16.restype = ctypes.c_uint16
        lib.synth_f32_to_bf16.argtypes = [ctypes.c_float]
        lib.synth_f32_to_f16.restype = ctypes.c_uint16
        lib.synth_f32_to_f16.argtypes = [ctypes.c_float]
        _lib = lib
    return _lib


def _threads() -> int:
    n = os.cpu_count() or 1
    return max(1, min(16, n))


def key(seed: int, workload_id: int, tensor: int, sub: int = 0) -> int:
    return int(_load().synth_key(seed, workload_id, tensor, sub))


def fill(k: int, n: int, dist: str, a: float, b: float, out: str, offset: int = 0) -> np.ndarray:
    """``n`` stream elements starting at ``offset``; bf16/f16 are returned as uint16 bits."""
    dt = {"f64": np.float64, "f32": np.float32, "bf16": np.uint16, "f16": np.uint16}[out]
    arr = np.empty(n, dtype=dt)
    if n:
        rc = _load().synth_fill(k, offset, n, _DIST[dist], a, b, _OUT[out],
                                arr.ctypes.data, _threads())
        if rc != 0:
            raise ValueError("synth_fill rejected its arguments")
    return arr


def u01(k: int, n: int, offset: int = 0) -> np.ndarray:
    arr = np.empty(n, dtype=np.float64)
    if n:
        _load().synth_u01(k, offset, n, arr.ctypes.data, _threads())
    return arr


def f32_to_bf16(x: float) -> int:
    return int(_load().synth_f32_to_bf16(x))


def f32_to_f16(x: float) -> int:
    return int(_load().synth_f32_to_f16(x))


@dataclass(frozen=True)
class Workload:
    name: str
    wid: int
    kind: str  # "combine", "packed", "merge", "correct" or "planes"
    N: int
    B: int
    H: int
    D: int
    dtype: str  # "bf16" | "f16" | "f32"
    out_dist: tuple  # (dist, a, b)
    lse_dist: tuple
    special: tuple = ()  # ((probability, value), ...) applied in order on one uniform per entry
    allneg_row: tuple | None = None  # (b, h) whose LSE is -inf on every shard
    base2: bool = False
    return_lse: bool = False
    desc: str = field(default="", compare=False)

    @property
    def rows(self) -> int:
        """(token, head) rows the combine produces."""
        return self.B * (self.H // self.N if self.kind == "packed" else self.H)


WORKLOADS = {
    w.name: w for w in [
        Workload("small", 1, "combine", 2, 4, 8, 128, "bf16", ("normal", 0.0, 1.0),
                 ("uniform", -2.0, 8.0), allneg_row=(3, 7), base2=False, return_lse=False,
                 desc="N=2 B=4 H=8 D=128 bf16, LSE base e U[-2,8], row (3,7) all -inf"),
        Workload("fp16_base2", 2, "combine", 4, 256, 32, 128, "f16", ("normal", 0.0, 1.0),
                 ("uniform", 0.0, 20.0), special=((0.02, float("nan")), (0.02, float("inf"))),
                 base2=True, return_lse=True,
                 desc="N=4 B=256 H=32 D=128 fp16, LSE base 2 U[0,20], 2% NaN 2% +inf"),
        Workload("packed", 3, "packed", 8, 2048, 64, 128, "bf16", ("normal", 0.0, 1.0),
                 ("uniform", -5.0, 15.0), base2=False, return_lse=True,
                 desc="per-rank [2048,64,128] bf16 + [2048,64] fp32 -> [8,2048,8,130] bf16"),
        Workload("mla_decode", 4, "combine", 8, 4096, 16, 512, "bf16", ("normal", 0.0, 0.5),
                 ("normal", 10.0, 3.0), special=((0.01, float("-inf")),), base2=True,
                 return_lse=False,
                 desc="N=8 B=4096 H=16 D=512 bf16, LSE base 2 N(10,3), 1% -inf"),
        Workload("merge_heads", 6, "merge", 8, 8, 2048, 128, "bf16", ("normal", 0.0, 1.0),
                 ("uniform", -5.0, 15.0), base2=False, return_lse=False,
                 desc="received planes [8, 8 heads, 2048 tokens, 128] bf16 + [8, 8, 2048] -> "
                      "token-major [2048, 8, 128] (head-scattered exchange, token_dim 2)"),
        Workload("ag_correct", 7, "correct", 8, 4096, 16, 512, "bf16", ("normal", 0.0, 0.5),
                 ("normal", 10.0, 3.0), special=((0.01, float("-inf")),), base2=True,
                 return_lse=False,
                 desc="gathered LSEs [8,4096,16] base 2 + rank 3's partial [4096,16,512] bf16 -> "
                      "its share of the combine (all-gather + reduce-scatter local step)"),
        Workload("mla_decode_f32", 8, "combine", 8, 4096, 16, 512, "f32", ("normal", 0.0, 0.5),
                 ("normal", 10.0, 3.0), special=((0.01, float("-inf")),), base2=True,
                 return_lse=False,
                 desc="N=8 B=4096 H=16 D=512 fp32 partials, LSE base 2 N(10,3), 1% -inf"),
        Workload("packed_f32", 9, "packed", 8, 2048, 64, 128, "f32", ("normal", 0.0, 1.0),
                 ("uniform", -5.0, 15.0), base2=False, return_lse=True,
                 desc="per-rank [2048,64,128] fp32 + [2048,64] fp32 -> [8,2048,8,129] fp32"),
        Workload("direct_planes", 10, "planes", 8, 2048, 8, 128, "bf16", ("normal", 0.0, 1.0),
                 ("uniform", -5.0, 15.0), base2=False, return_lse=True,
                 desc="receive planes of a direct exchange: 8 ranks x [2048 of 4096 tokens, "
                      "8 heads, 128] bf16 + LSEs -> [2048, 8, 128] (one ubatch slot)"),
        Workload("large_batch", 5, "combine", 16, 16384, 32, 128, "bf16", ("normal", 0.0, 1.0),
                 ("uniform", -10.0, 30.0),
                 special=((0.005 / 3, float("nan")), (0.005 / 3, float("inf")),
                          (0.005 / 3, float("-inf"))),
                 base2=False, return_lse=True,
                 desc="N=16 B=16384 H=32 D=128 bf16, LSE base e U[-10,30], 0.5% NaN/+inf/-inf"),
    ]
}


def _draw(w: Workload, seed: int, tensor: int, sub: int, dist: tuple, out: str,
          shape_outer: int, inner_total: int, lo: int, hi: int, inner: int) -> np.ndarray:
    """Rows [lo,hi) of every outer plane of a tensor shaped [outer, inner_total/inner, inner]."""
    k = key(seed, w.wid, tensor, sub)
    per_plane = inner_total
    parts = [fill(k, (hi - lo) * inner, dist[0], dist[1], dist[2], out,
                  offset=p * per_plane + lo * inner) for p in range(shape_outer)]
    return np.concatenate(parts) if parts else np.empty(0)


def _apply_special(w: Workload, seed: int, sub: int, lse: np.ndarray, outer: int,
                   per_plane: int, lo: int, hi: int, H: int) -> None:
    if not w.special:
        return
    k = key(seed, w.wid, T_SPECIAL, sub)
    u = np.concatenate([u01(k, (hi - lo) * H, offset=p * per_plane + lo * H)
                        for p in range(outer)]).reshape(lse.shape)
    lo_t = 0.0
    for prob, val in w.special:
        lse[(u >= lo_t) & (u < lo_t + prob)] = np.float32(val)
        lo_t += prob


def combine_inputs(w: Workload | str, seed: int = 0, b_lo: int = 0, b_hi: int | None = None):
    """(outputs uint16 bits [N, b_hi-b_lo, H, D], lses float32 [N, b_hi-b_lo, H]).

    Tokens ``b_lo:b_hi`` of the full workload tensors, bit-identical to the same
    slice of the whole.
    """
    w = WORKLOADS[w] if isinstance(w, str) else w
    if w.kind == "packed":
        raise ValueError(f"{w.name} is a packed workload; use rank_inputs()")
    # "correct" workloads draw all N shards; the caller uses one rank's plane;
    # "planes" workloads draw the B valid tokens of each receive plane
    b_hi = w.B if b_hi is None else b_hi
    if not (0 <= b_lo <= b_hi <= w.B):
        raise ValueError("token range out of bounds")
    nb = b_hi - b_lo
    o = _draw(w, seed, T_OUTPUTS, 0, w.out_dist, w.dtype, w.N, w.B * w.H * w.D,
              b_lo, b_hi, w.H * w.D).reshape(w.N, nb, w.H, w.D)
    lse = _draw(w, seed, T_LSE, 0, w.lse_dist, "f32", w.N, w.B * w.H,
                b_lo, b_hi, w.H).reshape(w.N, nb, w.H)
    _apply_special(w, seed, 0, lse, w.N, w.B * w.H, b_lo, b_hi, w.H)
    if w.allneg_row is not None:
        b, h = w.allneg_row
        if b_lo <= b < b_hi:
            lse[:, b - b_lo, h] = np.float32(-np.inf)
    return o, lse


def rank_inputs(w: Workload | str, rank: int, seed: int = 0, b_lo: int = 0,
                b_hi: int | None = None):
    """One rank's (attention output uint16 bits [nb, H, D], LSE float32 [nb, H])."""
    w = WORKLOADS[w] if isinstance(w, str) else w
    if w.kind != "packed":
        raise ValueError(f"{w.name} is not a packed workload")
    if not 0 <= rank < w.N:
        raise ValueError("rank out of range")
    b_hi = w.B if b_hi is None else b_hi
    if not (0 <= b_lo <= b_hi <= w.B):
        raise ValueError("token range out of bounds")
    nb = b_hi - b_lo
    o = _draw(w, seed, T_OUTPUTS, rank, w.out_dist, w.dtype, 1, w.B * w.H * w.D,
              b_lo, b_hi, w.H * w.D).reshape(nb, w.H, w.D)
    lse = _draw(w, seed, T_LSE, rank, w.lse_dist, "f32", 1, w.B * w.H,
                b_lo, b_hi, w.H).reshape(nb, w.H)
    _apply_special(w, seed, rank, lse[None], 1, w.B * w.H, b_lo, b_hi, w.H)
    return o, lse


def custom_inputs(N: int, B: int, H: int, D: int, dtype: str = "bf16", seed: int = 0,
                  out_dist=("normal", 0.0, 1.0), lse_dist=("uniform", -5.0, 15.0),
                  special=(), wid: int = 99):
    """Inputs of any shape with the same recipe machinery (edge-case tests)."""
    w = Workload("custom", wid, "combine", N, B, H, D, dtype, out_dist, lse_dist,
                 special=tuple(special))
    return combine_inputs(w, seed)
