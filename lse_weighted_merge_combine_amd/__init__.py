"""LSE-weighted combine of partial attention outputs on MI355X (gfx950).

Thin Python binding over the C ABI of ``liblsec.so`` (declared in
``include/lsec.h``). Every step of the computation runs in the library's HIP
kernels; this module only checks tensors, allocates outputs with PyTorch and
passes raw device pointers and the current HIP stream. There is no CPU or
PyTorch fallback: if the library is missing the import of an entry point fails.

Entry points (same names as the C ABI):

* ``lsec_combine(outputs, lses, ...)`` -- ``_lse_weighted_combine`` of the page
  "vllm.v1.attention.ops.dcp_alltoall": ``[N,B,H,D]`` + ``[N,B,H]`` ->
  ``[B,H,D]`` (+ ``[B,H]``).
* ``lsec_pack_send(attn_out, attn_lse, N)`` -- that page's
  ``_dcp_a2a_pack_send``: ``[B,H,D]`` + ``[B,H]`` -> ``[N,B,H/N,D+P]``
  (P = 2 for bf16 / fp16, 1 for fp32).
* ``lsec_unpack_combine(recv, ...)`` -- ``_dcp_a2a_unpack_combine``.
* ``lsec_unpack(recv)`` -- the layout half of the receive step.
* ``lsec_pack_dim(dtype)`` -- ``_dcp_a2a_lse_pack_dim``.
* ``dcp_a2a_lse_reduce(out, lse, world_size, exchange)`` -- the page's
  ``dcp_a2a_lse_reduce``: pack, the caller's all-to-all, unpack + combine;
  ``dcp_a2a_send_recv_buffers(shape, device, dtype)`` keeps its buffers.

* ``lsec_merge(outputs, lses, token_dim)`` -- ``_merge_dcp_outputs_with_torch``
  of the page "vllm_ascend/attention/context_parallel/sfa_cp.py": the same
  combine over received planes, stored token-major.

* ``lsec_combine_planes(outputs, lses, num_tokens)`` -- the local combine of
  the fused direct all-to-all on the page "vllm.v1.attention.ops.dcp"
  (``DirectDCPA2AWorkspace.lse_reduce``): the first ``num_tokens`` tokens of
  one ubatch slot's receive planes; with ``query_start_loc`` the valid count
  is read on the device and ``num_tokens`` is the padded capacity.

* ``lsec_correct_partial(lses, rank, partial)`` -- the local step of the LSE
  all-gather + output reduce-scatter strategies named on the page
  "vllm.v1.attention.ops.dcp" (``cp_lse_ag_out_rs`` / ``cp_lse_ag_out_ar``).

``lse_weighted_combine`` and ``merge_dcp_outputs`` keep the argument names of
the pages' functions; ``lse_combine``, ``pack_send`` and ``unpack_combine`` are
the plain names of the three hot-path calls.

Element dtypes: bfloat16, float16 and float32. The combining calls take
``out_dtype=torch.float32`` to return an fp32 result from 16-bit inputs (the
dtype the page's CPU function promotes to); by default the result has the
input dtype.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "liblsec.so")

LSEC_OK = 0
LSEC_ERR_NULL = 1
LSEC_ERR_SHAPE = 2
LSEC_ERR_DIVISIBILITY = 3
LSEC_ERR_DTYPE = 4
LSEC_ERR_ALIGNMENT = 5
LSEC_ERR_BASE = 6
LSEC_ERR_LAUNCH = 7
LSEC_ERR_TOKEN_DIM = 8
LSEC_ERR_RANK = 9
LSEC_BF16 = 0
LSEC_FP16 = 1
LSEC_FP32 = 2
LSEC_OUT_FP32 = 256
LSEC_BASE_E = 0
LSEC_BASE_2 = 1

_DTYPES = {torch.bfloat16: LSEC_BF16, torch.float16: LSEC_FP16, torch.float32: LSEC_FP32}
_VALUE_ERRORS = (LSEC_ERR_SHAPE, LSEC_ERR_DIVISIBILITY, LSEC_ERR_DTYPE, LSEC_ERR_BASE,
                 LSEC_ERR_RANK)

_lib = None


class LsecError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_string(status)} (status {status})")
        self.status = status


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load liblsec.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build the HIP library first "
            "(python -c 'import __graft_entry__ as g; g.build()')")
    lib = ctypes.CDLL(path)
    P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.lsec_version.restype = I
    lib.lsec_version.argtypes = []
    lib.lsec_pack_dim.restype = I
    lib.lsec_pack_dim.argtypes = [I]
    lib.lsec_status_string.restype = ctypes.c_char_p
    lib.lsec_status_string.argtypes = [I]
    lib.lsec_combine.restype = I
    lib.lsec_combine.argtypes = [P, P, I64, I64, I64, I64, I, I, P, P, P]
    lib.lsec_pack_send.restype = I
    lib.lsec_pack_send.argtypes = [P, P, I64, I64, I64, I64, I, P, P]
    lib.lsec_unpack_combine.restype = I
    lib.lsec_unpack_combine.argtypes = [P, I64, I64, I64, I64, I, I, P, P, P]
    lib.lsec_unpack.restype = I
    lib.lsec_unpack.argtypes = [P, I64, I64, I64, I64, I, P, P, P]
    lib.lsec_combine_planes.restype = I
    lib.lsec_combine_planes.argtypes = [P, I64, P, I64, I64, I64, I64, I64, I, I, P, P, P]
    lib.lsec_combine_planes_valid.restype = I
    lib.lsec_combine_planes_valid.argtypes = [P, I64, P, I64, I64, I64, I64, I64, I, I, P, I64, P,
                                              P, P]
    lib.lsec_merge.restype = I
    lib.lsec_merge.argtypes = [P, P, I64, I64, I64, I64, I, I, I, P, P, P]
    lib.lsec_correct_partial.restype = I
    lib.lsec_correct_partial.argtypes = [P, I64, I64, P, I64, I64, I64, I, I, P, P, P]
    lib.lsec_combine_path.restype = ctypes.c_char_p
    lib.lsec_combine_path.argtypes = [I64, I64, I64, I64, I, I, I]
    lib.lsec_pack_path.restype = ctypes.c_char_p
    lib.lsec_pack_path.argtypes = [I64, I64, I64, I64, I, I, I]
    lib.lsec_floor_empty.restype = I
    lib.lsec_floor_empty.argtypes = [P]
    lib.lsec_floor_read_blocks.restype = I64
    lib.lsec_floor_read_blocks.argtypes = [I64]
    lib.lsec_floor_read.restype = I
    lib.lsec_floor_read.argtypes = [P, I64, P, P]
    lib.lsec_floor_copy.restype = I
    lib.lsec_floor_copy.argtypes = [P, P, I64, P]
    lib.lsec_time_next_launch.restype = I
    lib.lsec_time_next_launch.argtypes = [P, P]
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().lsec_status_string(int(status)).decode()


def _raise_on(status: int, what: str) -> None:
    if status == LSEC_OK:
        return
    if status in _VALUE_ERRORS:
        raise ValueError(f"{what}: {status_string(status)}")
    raise LsecError(status, what)


def _dtype_code(t: torch.Tensor) -> int:
    try:
        return _DTYPES[t.dtype]
    except KeyError:
        raise ValueError(f"unsupported dtype {t.dtype}: bfloat16, float16 or float32 only") \
            from None


def _result_dtype(t: torch.Tensor, out_dtype) -> tuple[int, torch.dtype]:
    """(dtype code for a combining call, torch dtype of its result)."""
    code = _dtype_code(t)
    if out_dtype is None or out_dtype == t.dtype:
        return code, t.dtype
    if out_dtype == torch.float32:
        return code | LSEC_OUT_FP32, torch.float32
    raise ValueError(f"out_dtype must be None, {t.dtype} or torch.float32, got {out_dtype}")


def _check_dev(*ts: torch.Tensor) -> torch.device:
    dev = ts[0].device
    for t in ts:
        if t.device.type != "cuda":
            raise ValueError("tensors must live on a GPU device")
        if t.device != dev:
            raise ValueError("all tensors must be on the same device")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
    return dev


def _stream(dev: torch.device, stream) -> int:
    if stream is None:
        return torch.cuda.current_stream(dev).cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


def lsec_pack_dim(dtype: torch.dtype) -> int:
    """Output-dtype elements per packed fp32 LSE (2 for bf16 / fp16, 1 for fp32)."""
    code = _DTYPES.get(dtype, -1)
    r = load_library().lsec_pack_dim(code)
    if r < 0:
        raise ValueError(f"unsupported dtype {dtype}")
    return r


def lsec_combine(outputs: torch.Tensor, lses: torch.Tensor, base_e: bool = True,
                 return_lse: bool = False, out: torch.Tensor | None = None,
                 out_lse: torch.Tensor | None = None, stream=None, out_dtype=None):
    """Combine partial outputs [N,B,H,D] by their LSEs [N,B,H] (fp32).

    Returns the combined [B,H,D] output in the input dtype (or ``out_dtype``
    torch.float32), and the [B,H] fp32 global LSE when ``return_lse``.
    ``base_e`` False means base-2 LSEs.
    """
    lib = load_library()
    if outputs.dim() != 4 or lses.dim() != 3 or tuple(lses.shape) != tuple(outputs.shape[:3]):
        raise ValueError(f"expected outputs [N,B,H,D] and lses [N,B,H], got "
                         f"{tuple(outputs.shape)} and {tuple(lses.shape)}")
    if lses.dtype != torch.float32:
        raise ValueError("lses must be float32")
    dt, rdt = _result_dtype(outputs, out_dtype)
    N, B, H, D = outputs.shape
    dev = _check_dev(outputs, lses)
    if out is None:
        out = torch.empty((B, H, D), dtype=rdt, device=dev)
    if return_lse and out_lse is None:
        out_lse = torch.empty((B, H), dtype=torch.float32, device=dev)
    _check_out(out, (B, H, D), rdt, dev)
    if return_lse:
        _check_out(out_lse, (B, H), torch.float32, dev)
    st = lib.lsec_combine(_ptr(outputs), _ptr(lses), N, B, H, D, dt,
                          LSEC_BASE_E if base_e else LSEC_BASE_2, _ptr(out),
                          _ptr(out_lse) if return_lse else None, _stream(dev, stream))
    _raise_on(st, "lsec_combine")
    return (out, out_lse) if return_lse else out


def lsec_combine_planes(outputs: torch.Tensor, lses: torch.Tensor, num_tokens: int,
                        base_e: bool = True, return_lse: bool = False,
                        out: torch.Tensor | None = None, out_lse: torch.Tensor | None = None,
                        stream=None, out_dtype=None, query_start_loc: torch.Tensor | None = None):
    """Combine the first ``num_tokens`` tokens of receive planes
    outputs [N,T_max,H,D] + lses [N,T_max,H] -> [num_tokens,H,D] (+ [num_tokens,H]).

    The planes of the fused direct all-to-all's receive buffers
    (``received_output[ubatch][slot]``). Each plane must be contiguous; the
    stride between planes may be anything at least a plane's size (so a view
    such as ``buf[u, s]`` or ``buf[u, s, :, :T]`` works as is).

    ``query_start_loc`` (int32 [num_reqs + 1] on the same device, as passed to
    ``DirectDCPA2AWorkspace.lse_reduce``) makes ``num_tokens`` a capacity: the
    kernels read the valid count ``query_start_loc[-1]`` (clamped to
    [0, num_tokens]) and leave the rows of later tokens (padding) unwritten,
    as the page's ``new_empty`` output leaves them (lsec_combine_planes_valid).
    """
    lib = load_library()
    if outputs.dim() != 4 or lses.dim() != 3 or tuple(lses.shape) != tuple(outputs.shape[:3]):
        raise ValueError(f"expected outputs [N,T_max,H,D] and lses [N,T_max,H], got "
                         f"{tuple(outputs.shape)} and {tuple(lses.shape)}")
    if lses.dtype != torch.float32:
        raise ValueError("lses must be float32")
    N, T_max, H, D = outputs.shape
    if not 0 <= num_tokens <= T_max:
        raise ValueError(f"num_tokens must be in [0, {T_max}], got {num_tokens}")
    for t in (outputs, lses):
        if t.device.type != "cuda":
            raise ValueError("tensors must live on a GPU device")
        if N > 0 and not t[0].is_contiguous():
            raise ValueError("each plane (dimension 0 index) must be contiguous")
    if outputs.device != lses.device:
        raise ValueError("all tensors must be on the same device")
    dt, rdt = _result_dtype(outputs, out_dtype)
    dev = outputs.device
    T = int(num_tokens)
    if out is None:
        out = torch.empty((T, H, D), dtype=rdt, device=dev)
    if return_lse and out_lse is None:
        out_lse = torch.empty((T, H), dtype=torch.float32, device=dev)
    _check_out(out, (T, H, D), rdt, dev)
    if return_lse:
        _check_out(out_lse, (T, H), torch.float32, dev)
    pstride = outputs.stride(0) if N > 1 else T * H * D
    lstride = lses.stride(0) if N > 1 else T * H
    base = LSEC_BASE_E if base_e else LSEC_BASE_2
    if query_start_loc is None:
        st = lib.lsec_combine_planes(_ptr(outputs), pstride, _ptr(lses), lstride, N, T, H, D, dt,
                                     base, _ptr(out), _ptr(out_lse) if return_lse else None,
                                     _stream(dev, stream))
        _raise_on(st, "lsec_combine_planes")
    else:
        q = query_start_loc
        if (q.dtype != torch.int32 or q.dim() != 1 or q.numel() < 1 or q.device != dev
                or not q.is_contiguous()):
            raise ValueError("query_start_loc must be a contiguous 1-D int32 tensor of "
                             f"num_reqs + 1 offsets on {dev}, got {q.dtype} {tuple(q.shape)} "
                             f"stride {tuple(q.stride())} on {q.device}")
        st = lib.lsec_combine_planes_valid(_ptr(outputs), pstride, _ptr(lses), lstride, N, T, H, D,
                                           dt, base, _ptr(q), q.numel() - 1, _ptr(out),
                                           _ptr(out_lse) if return_lse else None,
                                           _stream(dev, stream))
        _raise_on(st, "lsec_combine_planes_valid")
    return (out, out_lse) if return_lse else out


def lsec_merge(outputs: torch.Tensor, lses: torch.Tensor, token_dim: int, base_e: bool = True,
               return_lse: bool = False, out: torch.Tensor | None = None,
               out_lse: torch.Tensor | None = None, stream=None, out_dtype=None):
    """Token-major merge of received planes outputs [N,A,C,D] + lses [N,A,C].

    token_dim 1: tokens are A -> [A,C,D] (+ [A,C]); token_dim 2: tokens are C
    -> [C,A,D] (+ [C,A]), i.e. row (a, c) is stored at (c, a).
    """
    lib = load_library()
    if outputs.dim() != 4 or lses.dim() != 3 or tuple(lses.shape) != tuple(outputs.shape[:3]):
        raise RuntimeError("merge expects matching rank/token/head dimensions, got "
                           f"{tuple(outputs.shape)} and {tuple(lses.shape)}")
    if token_dim not in (1, 2):
        raise RuntimeError(f"merge token_dim must be 1 or 2, got {token_dim}")
    if lses.dtype != torch.float32:
        raise ValueError("lses must be float32")
    dt, rdt = _result_dtype(outputs, out_dtype)
    N, A, C, D = outputs.shape
    dev = _check_dev(outputs, lses)
    rows = (A, C) if token_dim == 1 else (C, A)
    if out is None:
        out = torch.empty(rows + (D,), dtype=rdt, device=dev)
    if return_lse and out_lse is None:
        out_lse = torch.empty(rows, dtype=torch.float32, device=dev)
    _check_out(out, rows + (D,), rdt, dev)
    if return_lse:
        _check_out(out_lse, rows, torch.float32, dev)
    st = lib.lsec_merge(_ptr(outputs), _ptr(lses), N, A, C, D, int(token_dim), dt,
                        LSEC_BASE_E if base_e else LSEC_BASE_2, _ptr(out),
                        _ptr(out_lse) if return_lse else None, _stream(dev, stream))
    _raise_on(st, "lsec_merge")
    return (out, out_lse) if return_lse else out


def lsec_correct_partial(lses: torch.Tensor, rank: int, partial: torch.Tensor,
                         base_e: bool = True, return_lse: bool = False,
                         out: torch.Tensor | None = None, out_lse: torch.Tensor | None = None,
                         stream=None, out_dtype=None):
    """Scale rank ``rank``'s partial output [B,H,D] by its normalised LSE weight
    among the gathered LSEs [N,B,H] (fp32); summing the results over the N
    ranks (a reduce-scatter or all-reduce) gives the combine."""
    lib = load_library()
    if lses.dim() != 3 or partial.dim() != 3 or tuple(partial.shape[:2]) != tuple(lses.shape[1:]):
        raise ValueError(f"expected lses [N,B,H] and partial [B,H,D], got {tuple(lses.shape)} "
                         f"and {tuple(partial.shape)}")
    if lses.dtype != torch.float32:
        raise ValueError("lses must be float32")
    dt, rdt = _result_dtype(partial, out_dtype)
    N, B, H = lses.shape
    D = partial.shape[2]
    dev = _check_dev(lses, partial)
    if out is None:
        out = torch.empty((B, H, D), dtype=rdt, device=dev)
    if return_lse and out_lse is None:
        out_lse = torch.empty((B, H), dtype=torch.float32, device=dev)
    _check_out(out, (B, H, D), rdt, dev)
    if return_lse:
        _check_out(out_lse, (B, H), torch.float32, dev)
    st = lib.lsec_correct_partial(_ptr(lses), N, int(rank), _ptr(partial), B, H, D, dt,
                                  LSEC_BASE_E if base_e else LSEC_BASE_2, _ptr(out),
                                  _ptr(out_lse) if return_lse else None, _stream(dev, stream))
    _raise_on(st, "lsec_correct_partial")
    return (out, out_lse) if return_lse else out


def merge_dcp_outputs(output_recv: torch.Tensor, lse_recv: torch.Tensor, token_dim: int):
    """The Ascend page's ``_merge_dcp_outputs_with_torch(output_recv, lse_recv,
    token_dim)`` (base e, no LSE), computed by the HIP kernel in the input dtype."""
    return lsec_merge(output_recv, lse_recv, token_dim, base_e=True, return_lse=False)


def lsec_pack_send(attn_out: torch.Tensor, attn_lse: torch.Tensor, N: int,
                   send: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Pack [B,H,D] output + [B,H] fp32 LSE into the [N,B,H/N,D+P] send buffer."""
    lib = load_library()
    if attn_out.dim() != 3 or attn_lse.dim() != 2 or \
            tuple(attn_lse.shape) != tuple(attn_out.shape[:2]):
        raise ValueError(f"expected attn_out [B,H,D] and attn_lse [B,H], got "
                         f"{tuple(attn_out.shape)} and {tuple(attn_lse.shape)}")
    if attn_lse.dtype != torch.float32:
        raise ValueError("attn_lse must be float32")
    dt = _dtype_code(attn_out)
    B, H, D = attn_out.shape
    if N < 1 or H % N != 0:
        raise ValueError(f"H={H} must be divisible by the number of ranks {N}.")
    dev = _check_dev(attn_out, attn_lse)
    shape = (N, B, H // N, D + lsec_pack_dim(attn_out.dtype))
    if send is None:
        send = torch.empty(shape, dtype=attn_out.dtype, device=dev)
    _check_out(send, shape, attn_out.dtype, dev)
    st = lib.lsec_pack_send(_ptr(attn_out), _ptr(attn_lse), N, B, H, D, dt, _ptr(send),
                            _stream(dev, stream))
    _raise_on(st, "lsec_pack_send")
    return send


def _recv_dims(recv: torch.Tensor):
    if recv.dim() != 4:
        raise ValueError(f"expected recv [N,B,Hl,D+P], got {tuple(recv.shape)}")
    N, B, Hl, W = recv.shape
    D = W - lsec_pack_dim(recv.dtype)
    if D < 1:
        raise ValueError("recv rows are too short to hold an output and an LSE")
    return N, B, Hl, D


def lsec_unpack_combine(recv: torch.Tensor, base_e: bool = True, return_lse: bool = False,
                        out: torch.Tensor | None = None, out_lse: torch.Tensor | None = None,
                        stream=None, out_dtype=None):
    """Combine the N packed planes of recv [N,B,Hl,D+P] -> [B,Hl,D] (+ [B,Hl])."""
    lib = load_library()
    dt, rdt = _result_dtype(recv, out_dtype)
    N, B, Hl, D = _recv_dims(recv)
    dev = _check_dev(recv)
    if out is None:
        out = torch.empty((B, Hl, D), dtype=rdt, device=dev)
    if return_lse and out_lse is None:
        out_lse = torch.empty((B, Hl), dtype=torch.float32, device=dev)
    _check_out(out, (B, Hl, D), rdt, dev)
    if return_lse:
        _check_out(out_lse, (B, Hl), torch.float32, dev)
    st = lib.lsec_unpack_combine(_ptr(recv), N, B, Hl, D, dt,
                                 LSEC_BASE_E if base_e else LSEC_BASE_2, _ptr(out),
                                 _ptr(out_lse) if return_lse else None, _stream(dev, stream))
    _raise_on(st, "lsec_unpack_combine")
    return (out, out_lse) if return_lse else out


def lsec_unpack(recv: torch.Tensor, outputs: torch.Tensor | None = None,
                lses: torch.Tensor | None = None, stream=None):
    """Split recv [N,B,Hl,D+P] into outputs [N,B,Hl,D] and fp32 lses [N,B,Hl]."""
    lib = load_library()
    dt = _dtype_code(recv)
    N, B, Hl, D = _recv_dims(recv)
    dev = _check_dev(recv)
    if outputs is None:
        outputs = torch.empty((N, B, Hl, D), dtype=recv.dtype, device=dev)
    if lses is None:
        lses = torch.empty((N, B, Hl), dtype=torch.float32, device=dev)
    _check_out(outputs, (N, B, Hl, D), recv.dtype, dev)
    _check_out(lses, (N, B, Hl), torch.float32, dev)
    st = lib.lsec_unpack(_ptr(recv), N, B, Hl, D, dt, _ptr(outputs), _ptr(lses),
                         _stream(dev, stream))
    _raise_on(st, "lsec_unpack")
    return outputs, lses


def lsec_combine_path(N: int, B: int, H: int, D: int, packed: bool = False,
                      aligned: bool = True, dtype: torch.dtype = torch.bfloat16,
                      out_dtype=None) -> str:
    """Name of the kernel a combine of these sizes launches (diagnostics)."""
    code = _DTYPES.get(dtype)
    if code is None:
        raise ValueError(f"unsupported dtype {dtype}")
    if out_dtype == torch.float32 and dtype != torch.float32:
        code |= LSEC_OUT_FP32
    return load_library().lsec_combine_path(N, B, H, D, code, int(packed), int(aligned)).decode()


def lsec_pack_path(N: int, B: int, H: int, D: int, dtype: torch.dtype = torch.bfloat16,
                   in_aligned: bool = True, send_align: int = 16) -> str:
    """Name of the kernel lsec_pack_send launches for these sizes (diagnostics)."""
    code = _DTYPES.get(dtype)
    if code is None:
        raise ValueError(f"unsupported dtype {dtype}")
    return load_library().lsec_pack_path(N, B, H, D, code, int(in_aligned), int(send_align)).decode()


def lse_weighted_combine(outputs: torch.Tensor, lses: torch.Tensor, return_lse: bool = False,
                         is_lse_base_on_e: bool = True):
    """The page's ``_lse_weighted_combine(outputs, lses, return_lse, is_lse_base_on_e)``,
    computed by the HIP kernel. Like the page's function it returns fp32 for
    every input dtype: bf16 / fp16 outputs times fp32 weights promote to fp32."""
    return lsec_combine(outputs, lses, base_e=is_lse_base_on_e, return_lse=return_lse,
                        out_dtype=torch.float32)


_A2A_BUFFERS: dict = {}


def dcp_a2a_send_recv_buffers(shape, device, dtype: torch.dtype):
    """Send and receive buffers of one packed shape [N, B, H/N, D + P] for the
    exchange (the page's ``_dcp_a2a_send_recv_buffers``, whose body is not
    shown). They are kept per (shape, device, dtype), so that repeated steps,
    and a captured HIP graph, reuse the same memory: pass them to
    ``dcp_a2a_lse_reduce(..., send=, recv=)``. Calls that overlap in time (on
    different streams) must not share them."""
    shape = tuple(int(x) for x in shape)
    if len(shape) != 4 or any(x < 0 for x in shape):
        raise ValueError(f"expected a packed shape [N, B, H/N, D + P], got {shape}")
    if dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {dtype}: bfloat16, float16 or float32 only")
    device = torch.device(device)
    if device.type == "cuda" and device.index is None:
        device = torch.device("cuda", torch.cuda.current_device())
    key = (shape, device, dtype)
    bufs = _A2A_BUFFERS.get(key)
    if bufs is None:
        bufs = (torch.empty(shape, dtype=dtype, device=device),
                torch.empty(shape, dtype=dtype, device=device))
        _A2A_BUFFERS[key] = bufs
    return bufs


def dcp_a2a_lse_reduce(cp_attn_out: torch.Tensor, cp_attn_lse: torch.Tensor, world_size: int,
                       exchange=None, return_lse: bool = False, is_lse_base_on_e: bool = True,
                       send: torch.Tensor | None = None, recv: torch.Tensor | None = None):
    """The page's ``dcp_a2a_lse_reduce`` with the all-to-all left to the caller.

    cp_attn_out [B,H,D] and cp_attn_lse [B,H] (fp32) are this rank's partial
    attention over all H heads. They are packed into send [N,B,H/N,D+P]
    (``lsec_pack_send``), ``exchange(send, recv)`` must fill recv so that
    plane n holds what rank n packed for this rank (the chunk order of
    ``all_to_all_single``; with torch.distributed:
    ``lambda s, r: dist.all_to_all_single(r.view(-1), s.view(-1), group=g)``),
    and recv is combined (``lsec_unpack_combine``) into this rank's [B,H/N,D]
    heads (+ their [B,H/N] global LSE). As on the page, world_size 1 returns
    the inputs unchanged and H must be divisible by world_size (ValueError).
    ``send`` / ``recv`` may be preallocated buffers of the packed shape.
    """
    if world_size == 1:
        return (cp_attn_out, cp_attn_lse) if return_lse else cp_attn_out
    if cp_attn_out.dim() != 3:
        raise ValueError(f"expected cp_attn_out [B,H,D], got {tuple(cp_attn_out.shape)}")
    H = cp_attn_out.shape[1]
    if world_size < 1 or H % world_size != 0:
        raise ValueError(f"H={H} must be divisible by DCP world size {world_size}.")
    if exchange is None:
        raise ValueError("world_size > 1 needs an exchange(send, recv) function")
    send = lsec_pack_send(cp_attn_out, cp_attn_lse, world_size, send=send)
    if recv is None:
        recv = torch.empty_like(send)
    _check_out(recv, tuple(send.shape), send.dtype, send.device)
    exchange(send, recv)
    return lsec_unpack_combine(recv, base_e=is_lse_base_on_e, return_lse=return_lse)


def lse_combine(outputs: torch.Tensor, lses: torch.Tensor, base_e: bool = True,
                return_lse: bool = False):
    """The combine under its plain name: [N,B,H,D] + [N,B,H] -> [B,H,D] in the
    input dtype (+ the [B,H] fp32 global LSE when ``return_lse``)."""
    return lsec_combine(outputs, lses, base_e=base_e, return_lse=return_lse)


def pack_send(out: torch.Tensor, lse: torch.Tensor, N: int) -> torch.Tensor:
    """The pack under its plain name: [B,H,D] + [B,H] -> [N,B,H/N,D+P]."""
    return lsec_pack_send(out, lse, N)


def unpack_combine(recv: torch.Tensor, D: int, base_e: bool = True, return_lse: bool = False):
    """The receive side under its plain name, with the head dimension D stated
    (as the page's ``_dcp_a2a_unpack_combine`` takes it): recv [N,B,Hl,D+P]."""
    if recv.dim() != 4 or recv.shape[-1] != D + lsec_pack_dim(recv.dtype):
        raise ValueError(f"recv {tuple(recv.shape)} does not hold rows of D={D} plus the LSE")
    return lsec_unpack_combine(recv, base_e=base_e, return_lse=return_lse)


# ---------------------------------------------------------------- measurement aids
# (include/lsec_floor.h: not operations of the combine; the reference points
# its kernels are timed against)

def lsec_floor_empty(device=None, stream=None) -> None:
    """Launch one wave that does nothing (the duration no launch goes below)."""
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None \
        else torch.device(device)
    _raise_on(load_library().lsec_floor_empty(_stream(dev, stream)), "lsec_floor_empty")


def lsec_floor_read(src: torch.Tensor, sink: torch.Tensor | None = None,
                    stream=None) -> torch.Tensor:
    """Read every byte of ``src`` once with the combine's 16-byte non-temporal
    loads (a plain streaming read). Returns the int32 ``sink``: one word per
    16 KiB of ``src``, the XOR of its 32-bit words."""
    lib = load_library()
    dev = _check_dev(src)
    nbytes = src.numel() * src.element_size()
    words = lib.lsec_floor_read_blocks(nbytes)
    if words < 0:
        raise ValueError(f"src holds {nbytes} bytes: a multiple of 16 is required")
    if sink is None:
        sink = torch.empty(max(words, 1), dtype=torch.int32, device=dev)
    elif sink.dtype != torch.int32 or sink.numel() < words or sink.device != dev or \
            not sink.is_contiguous():
        raise ValueError(f"sink must be a contiguous int32 tensor of >= {words} words on {dev}")
    _raise_on(lib.lsec_floor_read(_ptr(src), nbytes, _ptr(sink), _stream(dev, stream)),
              "lsec_floor_read")
    return sink


def lsec_floor_copy(src: torch.Tensor, dst: torch.Tensor, stream=None) -> None:
    """Copy every byte of ``src`` into ``dst`` (same byte size, no overlap) once,
    with the combine's 16-byte non-temporal loads and stores (a plain copy)."""
    dev = _check_dev(src, dst)
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes:
        raise ValueError("src and dst must hold the same number of bytes")
    if nbytes % 16:
        raise ValueError(f"src holds {nbytes} bytes: a multiple of 16 is required")
    _raise_on(load_library().lsec_floor_copy(_ptr(src), _ptr(dst), nbytes, _stream(dev, stream)),
              "lsec_floor_copy")


_hip = None


def _hip_runtime():
    """The HIP runtime this process already runs on (torch's; liblsec.so binds
    to the same copy by its soname), for the event calls of LaunchTimer."""
    global _hip
    if _hip is None:
        torch.cuda.init()
        path = None
        with open("/proc/self/maps") as f:
            for line in f:
                if "libamdhip64" in line:
                    path = line.split()[-1]
                    break
        hip = ctypes.CDLL(path or "libamdhip64.so.7")
        hip.hipEventCreate.restype = ctypes.c_int
        hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        hip.hipEventDestroy.restype = ctypes.c_int
        hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        hip.hipEventElapsedTime.restype = ctypes.c_int
        hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                            ctypes.c_void_p]
        _hip = hip
    return _hip


class LaunchTimer:
    """Times single launches of the library by the kernels' own dispatch
    (lsec_time_next_launch): ``arm(i)`` before a call times its kernel into
    pair i; after a synchronisation ``elapsed_ms(i)`` is that kernel's
    duration. Events are created on the current device."""

    def __init__(self, pairs: int):
        hip = _hip_runtime()
        self._ev = []
        for _ in range(2 * pairs):
            e = ctypes.c_void_p()
            if hip.hipEventCreate(ctypes.byref(e)) != 0:
                self.close()
                raise LsecError("hipEventCreate failed")
            self._ev.append(e)

    def arm(self, i: int) -> None:
        _raise_on(load_library().lsec_time_next_launch(self._ev[2 * i], self._ev[2 * i + 1]),
                  "lsec_time_next_launch")

    def disarm(self) -> None:
        load_library().lsec_time_next_launch(None, None)

    def elapsed_ms(self, i: int) -> float:
        ms = ctypes.c_float()
        rc = _hip_runtime().hipEventElapsedTime(ctypes.byref(ms), self._ev[2 * i],
                                                self._ev[2 * i + 1])
        if rc != 0:
            raise LsecError(f"hipEventElapsedTime failed ({rc}): was pair {i} timed?")
        return float(ms.value)

    def close(self) -> None:
        for e in self._ev:
            _hip_runtime().hipEventDestroy(e)
        self._ev = []

    def __del__(self):
        try:
            self.close()
        except Exception:  # noqa: BLE001 - interpreter shutdown
            pass


def _check_out(t: torch.Tensor, shape, dtype, dev) -> None:
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype or t.device != dev or \
            not t.is_contiguous():
        raise ValueError(f"output tensor must be contiguous {dtype} of shape {tuple(shape)} "
                         f"on {dev}, got {t.dtype} {tuple(t.shape)} on {t.device}")


__all__ = [
    "lsec_pack_dim", "lsec_combine", "lsec_pack_send", "lsec_unpack_combine", "lsec_unpack",
    "lsec_combine_path", "lsec_pack_path", "lsec_merge", "merge_dcp_outputs", "lsec_correct_partial",
    "lsec_combine_planes", "lse_combine", "pack_send", "unpack_combine", "dcp_a2a_lse_reduce",
    "lse_weighted_combine", "load_library", "status_string", "LsecError", "LIB_PATH",
    "lsec_floor_empty", "lsec_floor_read", "lsec_floor_copy", "dcp_a2a_send_recv_buffers",
    "LaunchTimer",
]
