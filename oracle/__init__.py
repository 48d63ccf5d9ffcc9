"""CPU fp64 oracle for the LSE-weighted combine and its pack / unpack layout.

TEST INFRASTRUCTURE: only the test suite, ``__graft_entry__.smoke()`` and the
benchmark's CPU-baseline leg may import this package. The HIP library and its
Python binding never do; the two share no code.

The arithmetic lives in ``oracle.c`` (plain C, fp64, no fast-math); this module
only marshals numpy arrays through ctypes. Each function follows the page
"vllm.v1.attention.ops.dcp_alltoall": ``lse_combine`` / ``combine_f64`` are its
``_lse_weighted_combine``; ``pack_send``, ``unpack`` and ``unpack_combine`` are
the steps of its ``dcp_a2a_lse_reduce`` (``_dcp_a2a_pack_send``, the
all-to-all's chunk-r-to-rank-r placement, ``_dcp_a2a_unpack_combine``).
``merge`` is ``_merge_dcp_outputs_with_torch`` of the page
"vllm_ascend/attention/context_parallel/sfa_cp.py" (the same combine, stored
token-major). ``correct_partial`` is the local step of the LSE all-gather +
output reduce-scatter strategies that the page "vllm.v1.attention.ops.dcp"
names (``cp_lse_ag_out_rs`` / ``cp_lse_ag_out_ar``; a reading, since their
bodies are not shown): pinned by "the corrected partials of all ranks sum to
the combine".

Element dtypes: "bf16" and "f16" arrays hold 16-bit patterns (uint16);
"f32" arrays are float32 values or their uint32 patterns. A packed row holds D
elements and then P = 4 / element size elements carrying the fp32 LSE (P = 2
for 16-bit elements, 1 for fp32).

Parity status: every function here is pinned by the CPU tests (closed forms,
brute-force sharded attention, library log-sum-exp / softmax, the second
formulation of the merge on the Ascend SFA context-parallel page, the simulated
all-to-all; for ``valid_tokens`` / ``lse_combine_valid`` hand-derived counts in
tests/golden/valid_tokens.json and a padded step of requests whose real tokens
must combine to unsharded attention whatever the padding holds). One reading
is not pinned against any source: the order of the LSE's bytes inside the two
tail elements of a 16-bit packed row (memory order is taken; the round trip
through pack and unpack is pinned). ``valid_tokens`` restates a reading of the
direct all-to-all's masking (the page does not show that op's body); its pins
fix what the reading says, not that the page's op says the same.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liblsec_oracle.so")

BF16, F16, F32 = 0, 1, 2
_DT = {"bf16": BF16, "f16": F16, "f32": F32}
_EB = {"bf16": 2, "f16": 2, "f32": 4}


def build() -> str:
    """Compile ``oracle.c`` with gcc (no fast-math)."""
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-shared", "-fPIC",
           "-o", _LIB + ".tmp", _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


_lib = None
_P = ctypes.c_void_p
_I = ctypes.c_int64


def _load():
    global _lib
    if _lib is None:
        # LSEC_ORACLE_LIB: another build of the same source (the sanitizer test's)
        path = os.environ.get("LSEC_ORACLE_LIB")
        if path is None:
            path = _LIB
            if not os.path.exists(path):
                build()
        lib = ctypes.CDLL(path)
        lib.oracle_bf16_to_f64.restype = ctypes.c_double
        lib.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
        lib.oracle_f16_to_f64.restype = ctypes.c_double
        lib.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
        lib.oracle_f32_to_f64.restype = ctypes.c_double
        lib.oracle_f32_to_f64.argtypes = [ctypes.c_uint32]
        lib.oracle_bits_to_f64.argtypes = [_P, ctypes.c_int, _I, _P]
        lib.oracle_combine_f64.restype = None
        lib.oracle_combine_f64.argtypes = [_P, _P, _I, _I, _I, ctypes.c_int, _P, _P]
        lib.oracle_lse_combine.argtypes = [_P, ctypes.c_int, _P, _I, _I, _I, _I, ctypes.c_int,
                                           _P, _P]
        lib.oracle_merge.argtypes = [_P, ctypes.c_int, _P, _I, _I, _I, _I, ctypes.c_int,
                                     ctypes.c_int, _P, _P]
        lib.oracle_correct_partial.argtypes = [_P, _I, _I, _P, ctypes.c_int, _I, _I, _I,
                                               ctypes.c_int, _P, _P]
        lib.oracle_pack_dim.argtypes = [ctypes.c_int]
        lib.oracle_pack_send.argtypes = [_P, _P, _I, _I, _I, _I, _I, _P]
        lib.oracle_unpack.argtypes = [_P, _I, _I, _I, _I, _I, _P, _P]
        lib.oracle_unpack_combine.argtypes = [_P, ctypes.c_int, _I, _I, _I, _I, ctypes.c_int,
                                              _P, _P]
        lib.oracle_valid_tokens.restype = _I
        lib.oracle_valid_tokens.argtypes = [_P, _I, _I]
        lib.oracle_lse_combine_valid.argtypes = [_P, ctypes.c_int, _P, _P, _I, _I, _I, _I, _I,
                                                 ctypes.c_int, _P, _P, _P]
        _lib = lib
    return _lib


def _c(a: np.ndarray, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


def _bits(a: np.ndarray, dtype: str) -> np.ndarray:
    """Contiguous storage patterns of an element array: uint16 for bf16 / f16,
    uint32 for f32 (float32 values are reinterpreted, not converted)."""
    if dtype not in _DT:
        raise ValueError(f"unknown dtype {dtype!r}")
    a = np.ascontiguousarray(a)
    if dtype == "f32":
        if a.dtype == np.float32:
            return a.view(np.uint32)
        if a.dtype != np.uint32:
            raise ValueError("f32 elements must be float32 values or uint32 patterns")
        return a
    return np.ascontiguousarray(a, dtype=np.uint16)


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise ValueError(f"oracle {what}: bad arguments (rc={rc})")


def bits_to_f64(bits: np.ndarray, dtype: str) -> np.ndarray:
    """bf16 / fp16 / fp32 elements -> exact fp64 values."""
    b = _bits(bits, dtype)
    out = np.empty(b.shape, dtype=np.float64)
    _check(_load().oracle_bits_to_f64(b.ctypes.data, _DT[dtype], b.size, out.ctypes.data),
           "bits_to_f64")
    return out


def combine_f64(o: np.ndarray, lse: np.ndarray, base2: bool = False):
    """The combine on fp64 planes: o [N, R, D], lse [N, R] -> (y [R, D], L [R])."""
    o = _c(o, np.float64)
    lse = _c(lse, np.float64)
    N, R, D = o.shape
    if lse.shape != (N, R):
        raise ValueError("lse shape must be o.shape[:2]")
    y = np.empty((R, D), dtype=np.float64)
    L = np.empty((R,), dtype=np.float64)
    _load().oracle_combine_f64(o.ctypes.data, lse.ctypes.data, N, R, D, int(base2),
                               y.ctypes.data, L.ctypes.data)
    return y, L


def lse_combine(outputs: np.ndarray, lses: np.ndarray, dtype: str, base2: bool = False):
    """outputs [N,B,H,D] elements, lses [N,B,H] fp32 -> (y [B,H,D] f64, L [B,H] f64)."""
    o = _bits(outputs, dtype)
    l = _c(lses, np.float32)
    N, B, H, D = o.shape
    if l.shape != (N, B, H):
        raise ValueError("lses shape must be outputs.shape[:3]")
    y = np.empty((B, H, D), dtype=np.float64)
    L = np.empty((B, H), dtype=np.float64)
    _check(_load().oracle_lse_combine(o.ctypes.data, _DT[dtype], l.ctypes.data, N, B, H, D,
                                      int(base2), y.ctypes.data, L.ctypes.data), "lse_combine")
    return y, L


def valid_tokens(query_start_loc, capacity: int, num_reqs: int | None = None) -> int:
    """The count of valid tokens of a padded step (``oracle_valid_tokens``):
    entry ``num_reqs`` of the requests' cumulative token offsets (by default
    the last entry), clamped to [0, capacity]. A reading of the ``seq_lens`` /
    ``query_start_loc`` arguments of ``DirectDCPA2AWorkspace.lse_reduce``
    (page "vllm.v1.attention.ops.dcp"), whose body the page does not give:
    tokens past the last request are padding with no result."""
    q = np.ascontiguousarray(np.asarray(query_start_loc).reshape(-1), dtype=np.int32)
    nr = q.size - 1 if num_reqs is None else int(num_reqs)
    if q.size == 0 or nr < 0 or nr >= q.size:
        raise ValueError("query_start_loc needs num_reqs + 1 entries")
    t = int(_load().oracle_valid_tokens(q.ctypes.data, nr, int(capacity)))
    if t < 0:
        raise ValueError("oracle valid_tokens: bad arguments")
    return t


def lse_combine_valid(outputs: np.ndarray, lses: np.ndarray, query_start_loc, dtype: str,
                      base2: bool = False, num_reqs: int | None = None):
    """outputs [N,T,H,D], lses [N,T,H] of a step padded to T tokens ->
    (y [Tv,H,D] f64, L [Tv,H] f64, Tv) (``oracle_lse_combine_valid``): the
    combine of ``lse_combine`` over the first Tv = ``valid_tokens(
    query_start_loc, T, num_reqs)`` tokens of every plane; tokens [Tv, T) have
    no result."""
    o = _bits(outputs, dtype)
    l = _c(lses, np.float32)
    N, T, H, D = o.shape
    if l.shape != (N, T, H):
        raise ValueError("lses shape must be outputs.shape[:3]")
    q = np.ascontiguousarray(np.asarray(query_start_loc).reshape(-1), dtype=np.int32)
    nr = q.size - 1 if num_reqs is None else int(num_reqs)
    tv_expect = valid_tokens(q, T, nr)
    y = np.empty((tv_expect, H, D), dtype=np.float64)
    L = np.empty((tv_expect, H), dtype=np.float64)
    tv = ctypes.c_int64(-1)
    _check(_load().oracle_lse_combine_valid(o.ctypes.data, _DT[dtype], l.ctypes.data, q.ctypes.data,
                                            nr, N, T, H, D, int(base2), y.ctypes.data,
                                            L.ctypes.data, ctypes.byref(tv)), "lse_combine_valid")
    if tv.value != tv_expect:
        raise ValueError("oracle lse_combine_valid: inconsistent valid count")
    return y, L, tv.value


def merge(outputs: np.ndarray, lses: np.ndarray, dtype: str, token_dim: int,
          base2: bool = False):
    """Token-major merge (Ascend SFA page, `_merge_dcp_outputs_with_torch`):
    outputs [N,A,C,D] bits, lses [N,A,C] -> y [A,C,D] (token_dim 1) or
    [C,A,D] (token_dim 2) in fp64, and L laid out the same way."""
    o = _bits(outputs, dtype)
    l = _c(lses, np.float32)
    N, A, C, D = o.shape
    if l.shape != (N, A, C):
        raise ValueError("lses shape must be outputs.shape[:3]")
    shape = (A, C) if token_dim == 1 else (C, A)
    y = np.empty(shape + (D,), dtype=np.float64)
    L = np.empty(shape, dtype=np.float64)
    _check(_load().oracle_merge(o.ctypes.data, _DT[dtype], l.ctypes.data, N, A, C, D,
                                int(token_dim), int(base2), y.ctypes.data, L.ctypes.data),
           "merge")
    return y, L


def correct_partial(lses: np.ndarray, rank: int, partial: np.ndarray, dtype: str,
                    base2: bool = False):
    """Local step of an LSE all-gather + output reduce-scatter (reading of the
    strategy names on the page "vllm.v1.attention.ops.dcp"): lses [N,B,H] of
    all shards, rank r's partial [B,H,D] elements -> (partial * normalised
    weight of shard r [B,H,D] f64, global LSE [B,H] f64)."""
    l = _c(lses, np.float32)
    p = _bits(partial, dtype)
    N, B, H = l.shape
    if p.shape[:2] != (B, H):
        raise ValueError("partial must be [B,H,D] with lses [N,B,H]")
    D = p.shape[2]
    y = np.empty((B, H, D), dtype=np.float64)
    L = np.empty((B, H), dtype=np.float64)
    _check(_load().oracle_correct_partial(l.ctypes.data, N, rank, p.ctypes.data, _DT[dtype], B, H,
                                          D, int(base2), y.ctypes.data, L.ctypes.data),
           "correct_partial")
    return y, L


def pack_dim(elem_bytes: int) -> int:
    return int(_load().oracle_pack_dim(elem_bytes))


def pack_send(out: np.ndarray, lse: np.ndarray, N: int, dtype: str = "bf16") -> np.ndarray:
    """out [B,H,D] elements, lse [B,H] fp32 -> send [N,B,H/N,D+P] patterns
    (uint16 with P = 2 for bf16 / f16, uint32 with P = 1 for f32)."""
    o = _bits(out, dtype)
    l = _c(lse, np.float32)
    B, H, D = o.shape
    if l.shape != (B, H) or N < 1 or H % N:
        raise ValueError("bad pack_send arguments")
    E = _EB[dtype]
    send = np.empty((N, B, H // N, D + 4 // E), dtype=o.dtype)
    _check(_load().oracle_pack_send(o.ctypes.data, l.ctypes.data, N, B, H, D, E,
                                    send.ctypes.data), "pack_send")
    return send


def unpack(recv: np.ndarray, D: int, dtype: str = "bf16"):
    """recv [N,B,Hl,D+P] -> (outputs [N,B,Hl,D] patterns, lses [N,B,Hl] fp32)."""
    r = _bits(recv, dtype)
    N, B, Hl, W = r.shape
    E = _EB[dtype]
    if W != D + 4 // E:
        raise ValueError("recv last dim must be D + P")
    outs = np.empty((N, B, Hl, D), dtype=r.dtype)
    lses = np.empty((N, B, Hl), dtype=np.float32)
    _check(_load().oracle_unpack(r.ctypes.data, N, B, Hl, D, E, outs.ctypes.data,
                                 lses.ctypes.data), "unpack")
    return outs, lses


def unpack_combine(recv: np.ndarray, D: int, dtype: str, base2: bool = False):
    """recv [N,B,Hl,D+P] -> (y [B,Hl,D] f64, L [B,Hl] f64)."""
    r = _bits(recv, dtype)
    N, B, Hl, W = r.shape
    if W != D + 4 // _EB[dtype]:
        raise ValueError("recv last dim must be D + P")
    y = np.empty((B, Hl, D), dtype=np.float64)
    L = np.empty((B, Hl), dtype=np.float64)
    _check(_load().oracle_unpack_combine(r.ctypes.data, _DT[dtype], N, B, Hl, D, int(base2),
                                         y.ctypes.data, L.ctypes.data), "unpack_combine")
    return y, L


def exchange(sends: list) -> list:
    """All-to-all placement on N simulated ranks: recv_p[r] = send_r[p].

    ``all_to_all_single`` on a flat buffer sends the r-th equal chunk to rank r
    and stores what rank r sent in the r-th chunk of the receive buffer.
    """
    N = len(sends)
    return [np.stack([sends[r][p] for r in range(N)]) for p in range(N)]
