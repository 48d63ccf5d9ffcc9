"""Host-side checks of the C ABI (no GPU needed, nothing is launched).

The library must load, export every function ``include/*.h`` declares (the
combine's ABI in lsec.h, the measurement aids in lsec_floor.h), and reject bad
arguments with the documented status before touching the GPU.
"""
import ctypes
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lsec.h")
HEADERS = sorted(os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include"))
                 if f.endswith(".h"))


@pytest.fixture(scope="module")
def lib():
    import lse_weighted_merge_combine_amd as lsec
    if not os.path.exists(lsec.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return lsec.load_library()


def _declared(headers=None):
    names = set()
    for h in headers or HEADERS:
        src = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names.update(re.findall(r"\b(lsec_[a-z_0-9]+)\s*\(", src))
    return sorted(names)


def test_header_declares_expected_entry_points():
    names = _declared()
    for n in ("lsec_combine", "lsec_merge", "lsec_pack_send", "lsec_unpack_combine",
              "lsec_unpack", "lsec_pack_dim", "lsec_status_string", "lsec_version",
              "lsec_combine_planes", "lsec_combine_planes_valid", "lsec_correct_partial",
              "lsec_combine_path", "lsec_pack_path"):
        assert n in _declared([HEADER])
    for n in ("lsec_floor_empty", "lsec_floor_read", "lsec_floor_read_blocks", "lsec_floor_copy",
              "lsec_time_next_launch"):
        assert n in names


def _prototypes(headers=None):
    """{name: (return type, [parameter types])} of every function include/*.h
    declares (parameter names dropped)."""
    protos = {}
    for h in headers or HEADERS:
        src = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        for m in re.finditer(r"^([A-Za-z_][\w \t\*]*?)\b(lsec_\w+)\s*\(([^)]*)\)\s*;", src,
                             flags=re.M):
            params = " ".join(m.group(3).split())
            decls = [] if params in ("", "void") else [d.strip() for d in params.split(",")]
            types = [re.sub(r"\s*\b\w+$", "", d) if re.search(r"[\w*]\s+\**\w+$", d) else d
                     for d in decls]
            protos[m.group(2)] = (" ".join(m.group(1).split()), types)
    return protos


def _ctype(c_type, is_return=False):
    t = c_type.replace(" ", "")
    if is_return and t == "constchar*":
        return ctypes.c_char_p
    if "*" in t:
        return ctypes.c_void_p
    return {"int": ctypes.c_int, "int64_t": ctypes.c_int64}[t]


def test_binding_signatures_match_the_headers(lib):
    """Every declared function has ctypes argtypes / restype in the binding,
    and they match the header's parameter list one for one (a pointer is
    c_void_p, int64_t c_int64, int c_int; const char* returns c_char_p)."""
    protos = _prototypes()
    assert len(protos) == len(_declared())
    for name, (ret, params) in protos.items():
        fn = getattr(lib, name)
        assert fn.argtypes is not None, f"{name}: the binding sets no argtypes"
        assert list(fn.argtypes) == [_ctype(p) for p in params], \
            f"{name}: argtypes {fn.argtypes} against the header's ({', '.join(params)})"
        assert fn.restype == _ctype(ret, is_return=True), f"{name}: restype {fn.restype} against {ret}"


def test_library_exports_every_declared_symbol(lib):
    for name in _declared():
        assert hasattr(lib, name), f"{name} declared in include/ but not exported"


def test_constants_match_header(lib):
    import lse_weighted_merge_combine_amd as lsec
    src = open(HEADER).read()
    for name in ("LSEC_OK", "LSEC_ERR_NULL", "LSEC_ERR_SHAPE", "LSEC_ERR_DIVISIBILITY",
                 "LSEC_ERR_DTYPE", "LSEC_ERR_ALIGNMENT", "LSEC_ERR_BASE", "LSEC_ERR_LAUNCH",
                 "LSEC_ERR_TOKEN_DIM", "LSEC_ERR_RANK",
                 "LSEC_BF16", "LSEC_FP16", "LSEC_FP32", "LSEC_OUT_FP32", "LSEC_BASE_E",
                 "LSEC_BASE_2"):
        m = re.search(rf"\b{name}\s*=\s*(\d+)", src)
        assert m and int(m.group(1)) == getattr(lsec, name), name


def test_pack_dim_and_strings(lib):
    assert lib.lsec_pack_dim(0) == 2 and lib.lsec_pack_dim(1) == 2 and lib.lsec_pack_dim(2) == 1
    assert lib.lsec_pack_dim(7) == -1 and lib.lsec_pack_dim(0 | 256) == -1
    assert lib.lsec_version() >= 100
    for s in range(0, 11):
        assert lib.lsec_status_string(s)


FAKE = 0x100000  # a 16-byte aligned non-null address; never dereferenced (calls fail validation)


@pytest.mark.parametrize("args,want", [
    ((FAKE, FAKE, 0, 1, 1, 8, 0, 0, FAKE, None, None), 2),      # N < 1
    ((FAKE, FAKE, 2, -1, 1, 8, 0, 0, FAKE, None, None), 2),     # B < 0
    ((FAKE, FAKE, 2, 1, 0, 8, 0, 0, FAKE, None, None), 2),      # H < 1
    ((FAKE, FAKE, 2, 1, 1, 0, 0, 0, FAKE, None, None), 2),      # D < 1
    ((FAKE, FAKE, 2, 1 << 40, 1 << 20, 1 << 10, 0, 0, FAKE, None, None), 2),  # overflow
    ((FAKE, FAKE, 2, 1, 1, 8, 5, 0, FAKE, None, None), 4),      # dtype
    ((FAKE, FAKE, 2, 1, 1, 8, 3 | 256, 0, FAKE, None, None), 4),  # flag on an unknown dtype
    ((FAKE, FAKE, 2, 1, 1, 8, 512, 0, FAKE, None, None), 4),    # unknown flag bit
    ((FAKE + 2, FAKE, 2, 1, 1, 8, 2, 0, FAKE, None, None), 5),  # fp32 outputs not 4-aligned
    ((FAKE, FAKE, 2, 1, 1, 8, 2, 0, FAKE + 2, None, None), 5),  # fp32 out not 4-aligned
    ((FAKE, FAKE, 2, 1, 1, 8, 0 | 256, 0, FAKE + 2, None, None), 5),  # fp32 result, out 2-aligned
    ((FAKE, FAKE, 2, 1 << 40, 1 << 20, 1 << 9, 2, 0, FAKE, None, None), 2),  # fp32 overflow
    ((FAKE, FAKE, 2, 1, 1, 8, 0, 3, FAKE, None, None), 6),      # base
    ((None, FAKE, 2, 1, 1, 8, 0, 0, FAKE, None, None), 1),      # NULL outputs
    ((FAKE, None, 2, 1, 1, 8, 0, 0, FAKE, None, None), 1),      # NULL lses
    ((FAKE, FAKE, 2, 1, 1, 8, 0, 0, None, None, None), 1),      # NULL out
    ((FAKE + 1, FAKE, 2, 1, 1, 8, 0, 0, FAKE, None, None), 5),  # odd address
    ((FAKE, FAKE + 2, 2, 1, 1, 8, 0, 0, FAKE, None, None), 5),  # lse not 4-aligned
    ((FAKE, FAKE, 2, 1, 1, 8, 0, 0, FAKE, FAKE + 2, None), 5),  # out_lse not 4-aligned
    ((None, None, 2, 0, 1, 8, 0, 0, None, None, None), 0),      # empty: nothing to do
])
def test_combine_validation(lib, args, want):
    assert lib.lsec_combine(*args) == want


def test_pack_send_validation(lib):
    f = lib.lsec_pack_send
    assert f(FAKE, FAKE, 3, 2, 8, 16, 0, FAKE, None) == 3   # 8 % 3 != 0
    assert f(FAKE, FAKE, 0, 2, 8, 16, 0, FAKE, None) == 2
    assert f(FAKE, FAKE, 2, 2, 8, 16, 9, FAKE, None) == 4
    assert f(FAKE, FAKE, 2, 2, 8, 16, 0 | 256, FAKE, None) == 4  # no fp32 result on a layout call
    assert f(FAKE, FAKE, 2, 2, 8, 16, 2, FAKE + 2, None) == 5    # fp32 send 2-aligned
    assert f(None, FAKE, 2, 2, 8, 16, 0, FAKE, None) == 1
    assert f(FAKE, FAKE, 2, 2, 8, 16, 0, FAKE + 1, None) == 5
    assert f(None, None, 2, 0, 8, 16, 0, None, None) == 0


def test_unpack_validation(lib):
    uc = lib.lsec_unpack_combine
    assert uc(FAKE, 0, 2, 2, 16, 0, 0, FAKE, None, None) == 2
    assert uc(FAKE, 2, 2, 2, 16, 3, 0, FAKE, None, None) == 4
    assert uc(FAKE, 2, 2, 2, 16, 0, 9, FAKE, None, None) == 6
    assert uc(None, 2, 2, 2, 16, 0, 0, FAKE, None, None) == 1
    assert uc(FAKE, 2, 2, 2, 16, 0, 0, FAKE, FAKE + 2, None) == 5
    u = lib.lsec_unpack
    assert u(FAKE, 2, 2, 0, 16, 0, FAKE, FAKE, None) == 2
    assert u(FAKE, 2, 2, 2, 16, 0, FAKE, None, None) == 1
    assert u(FAKE, 2, 2, 2, 16, 1 | 256, FAKE, FAKE, None) == 4
    assert u(FAKE + 2, 2, 2, 2, 16, 2, FAKE, FAKE, None) == 5
    assert uc(FAKE + 2, 2, 2, 2, 16, 2, 0, FAKE, None, None) == 5
    assert uc(FAKE, 2, 2, 2, 16, 1 | 256, 0, FAKE + 2, None, None) == 5
    assert u(FAKE, 2, 2, 2, 16, 0, FAKE, FAKE + 2, None) == 5
    assert u(None, 2, 0, 2, 16, 0, None, None, None) == 0


def test_python_binding_rejects_bad_tensors():
    import torch
    import lse_weighted_merge_combine_amd as lsec
    with pytest.raises(ValueError):
        lsec.lsec_combine(torch.zeros(2, 1, 1, 8, dtype=torch.bfloat16),
                          torch.zeros(2, 1, 1), base_e=True)  # CPU tensors
    with pytest.raises(ValueError):
        lsec.lsec_combine(torch.zeros(2, 1, 8, dtype=torch.bfloat16), torch.zeros(2, 1))
    with pytest.raises(ValueError):
        lsec.lsec_pack_dim(torch.float64)
    assert lsec.lsec_pack_dim(torch.float32) == 1
    with pytest.raises(ValueError):
        lsec.lsec_pack_send(torch.zeros(1, 6, 8, dtype=torch.float16), torch.zeros(1, 6), 4)


@pytest.mark.parametrize("args,want", [
    # N, B, H, D, dtype, packed, aligned
    ((16, 16384, 32, 128, 0, 0, 1), "combine_tiled_kernel S=16"),
    ((8, 4096, 16, 512, 0, 0, 1), "combine_tiled_kernel S=8"),
    ((4, 256, 32, 128, 0, 0, 1), "combine_tiled_kernel S=1"),
    ((8, 2048, 8, 128, 0, 1, 1), "combine_span_kernel"),          # packed, 16-bit, rows % 4 == 0
    ((16, 64, 4, 128, 1, 1, 1), "combine_span_kernel"),           # packed fp16, N = 16
    ((8, 2047, 1, 128, 0, 1, 1), "combine_tiled_kernel S=1"),    # packed, rows % 4 != 0
    ((5, 2048, 8, 128, 0, 1, 1), "combine_tiled_kernel S=1"),    # packed, N at run time
    ((8, 2048, 8, 256, 0, 1, 1), "combine_tiled_kernel S=1"),    # packed, D != 128
    ((8, 2048, 8, 128, 0, 1, 0), "combine_elems_kernel"),        # packed, unaligned buffers
    ((8, 2048, 8, 128, 256, 1, 1), "combine_tiled_kernel S=1"),  # packed, fp32 result
    ((8, 2048, 8, 128, 2, 1, 1), "combine_span32_kernel"),      # fp32 packed rows, whole spans
    ((8, 2047, 2, 128, 2, 1, 1), "combine_tiled_kernel S=1"),    # fp32 packed rows, not whole spans
    ((8, 2048, 8, 256, 2, 1, 1), "combine_tiled_kernel S=2"),    # fp32 packed rows, D != 128
    ((17, 2048, 8, 128, 0, 1, 1), "combine_rows_kernel"),        # packed, N > 16
    ((16, 16384, 32, 128, 0, 0, 0), "combine_elems_kernel"),   # buffers not 16-byte aligned
    ((1, 50, 3, 512, 0, 0, 1), "combine_rows_kernel"),          # N = 1
    ((32, 6, 4, 128, 0, 0, 1), "combine_rows_kernel"),          # N > 16
    ((3, 16384, 32, 128, 0, 0, 1), "combine_tiled_kernel S=16"),  # N at run time
    ((12, 8192, 16, 256, 0, 0, 1), "combine_tiled_kernel S=8"),
    ((4, 10, 3, 64, 0, 0, 1), "combine_rows_kernel"),           # D outside {128, 256, 512}
    ((3, 5, 2, 3, 0, 0, 1), "combine_elems_kernel"),            # D % 8 != 0
    ((2, 2, 2, 4096, 0, 0, 1), "combine_elems_kernel"),         # D > 2048
    ((4, 0, 8, 128, 0, 0, 1), "none"),
    ((4, 8, 8, 128, 7, 0, 1), "none"),                          # unknown dtype
    ((16, 16384, 32, 128, 256, 0, 1), "combine_tiled_kernel S=16"),  # bf16 -> fp32 result
    ((2, 8197, 32, 128, 2, 0, 1), "combine_tiled_kernel S=16"),  # fp32: 262304 rows of 32 lanes
    ((4, 3001, 33, 256, 2, 0, 1), "combine_tiled_kernel S=8"),
    ((2, 2, 2, 1024, 2, 0, 1), "combine_rows_kernel"),          # fp32: 256 lanes per row
    ((2, 2, 2, 2048, 2, 0, 1), "combine_elems_kernel"),         # fp32: D > 1024
    ((3, 5, 2, 6, 2, 0, 1), "combine_elems_kernel"),            # fp32: D % 4 != 0
])
def test_combine_path(lib, args, want):
    assert lib.lsec_combine_path(*args).decode() == want


@pytest.mark.parametrize("args,want", [
    # N, B, H, D, dtype, in_aligned, send_align
    ((8, 2048, 64, 128, 0, 1, 16), "pack_pipe_kernel"),      # the packed workload
    ((8, 2048, 64, 128, 1, 1, 16), "pack_pipe_kernel"),      # fp16
    ((1, 3, 4, 128, 0, 1, 64), "pack_pipe_kernel"),          # N = 1, odd B
    ((8, 2048, 64, 128, 2, 1, 16), "pack_pipe_kernel"),      # fp32 rows
    ((8, 2048, 48, 128, 0, 1, 16), "pack_pipe_kernel"),      # Hl = 6
    ((8, 2048, 64, 256, 0, 1, 16), "pack_pipe_kernel"),      # D = 256
    ((2, 4, 4, 1024, 2, 1, 16), "pack_pipe_kernel"),         # fp32: 256 lanes per row
    ((2, 4, 4, 2048, 2, 1, 16), "pack_elems_kernel"),       # fp32: D > 1024
    ((8, 2048, 64, 128, 0, 1, 4), "pack_rows_kernel"),      # send buffer 4-byte aligned
    ((8, 2048, 64, 128, 0, 1, 8), "pack_rows_kernel"),
    ((8, 2048, 64, 128, 0, 0, 16), "pack_elems_kernel"),    # attn_out not 16-byte aligned
    ((8, 2048, 64, 128, 0, 1, 2), "pack_elems_kernel"),     # send buffer 2-byte aligned
    ((8, 16, 64, 12, 0, 1, 16), "pack_elems_kernel"),       # D % 8 != 0
    ((8, 16, 60, 128, 0, 1, 16), "none"),                   # H % N != 0
    ((8, 0, 64, 128, 0, 1, 16), "none"),                    # B = 0
    ((8, 16, 64, 128, 256, 1, 16), "none"),                 # no fp32-result flag on a pack
    ((8, 16, 64, 128, 7, 1, 16), "none"),                   # unknown dtype
])
def test_pack_path(lib, args, want):
    assert lib.lsec_pack_path(*args).decode() == want


def test_merge_validation(lib):
    m = lib.lsec_merge
    assert m(FAKE, FAKE, 2, 3, 4, 8, 0, 0, 0, FAKE, None, None) == 8   # token_dim 0
    assert m(FAKE, FAKE, 2, 3, 4, 8, 3, 0, 0, FAKE, None, None) == 8   # token_dim 3
    assert m(FAKE, FAKE, 0, 3, 4, 8, 2, 0, 0, FAKE, None, None) == 2   # N < 1
    assert m(FAKE, FAKE, 2, 3, 4, 8, 2, 7, 0, FAKE, None, None) == 4   # dtype
    assert m(None, FAKE, 2, 3, 4, 8, 2, 0, 0, FAKE, None, None) == 1   # NULL outputs
    assert m(FAKE, FAKE, 2, 3, 4, 8, 2, 0, 0, FAKE + 1, None, None) == 5  # out alignment
    assert m(None, None, 2, 0, 4, 8, 2, 0, 0, None, None, None) == 0   # empty
    import torch
    import lse_weighted_merge_combine_amd as lsec
    with pytest.raises(RuntimeError):
        lsec.lsec_merge(torch.zeros(2, 3, 4, 8, dtype=torch.bfloat16), torch.zeros(2, 3, 4), 3)
    with pytest.raises(RuntimeError):
        lsec.lsec_merge(torch.zeros(2, 3, 4, 8, dtype=torch.bfloat16), torch.zeros(2, 3, 5), 2)


def test_correct_partial_validation(lib):
    c = lib.lsec_correct_partial
    assert c(FAKE, 4, 4, FAKE, 2, 3, 8, 0, 0, FAKE, None, None) == 9    # rank == N
    assert c(FAKE, 4, -1, FAKE, 2, 3, 8, 0, 0, FAKE, None, None) == 9   # rank < 0
    assert c(FAKE, 0, 0, FAKE, 2, 3, 8, 0, 0, FAKE, None, None) == 2    # N < 1
    assert c(FAKE, 4, 1, FAKE, 2, 3, 8, 3, 0, FAKE, None, None) == 4    # dtype
    assert c(FAKE, 4, 1, FAKE, 2, 3, 8, 0, 5, FAKE, None, None) == 6    # base
    assert c(None, 4, 1, FAKE, 2, 3, 8, 0, 0, FAKE, None, None) == 1    # NULL lses
    assert c(FAKE, 4, 1, FAKE + 1, 2, 3, 8, 0, 0, FAKE, None, None) == 5  # odd partial
    assert c(None, 4, 1, None, 0, 3, 8, 0, 0, None, None, None) == 0    # empty


def test_combine_planes_validation(lib):
    c = lib.lsec_combine_planes
    # outputs, plane_stride, lses, lse_plane_stride, N, T, H, D, dtype, base, out, out_lse, stream
    assert c(FAKE, 2 * 3 * 8 - 1, FAKE, 6, 2, 2, 3, 8, 0, 0, FAKE, None, None) == 2  # stride < plane
    assert c(FAKE, 48, FAKE, 5, 2, 2, 3, 8, 0, 0, FAKE, None, None) == 2      # lse stride < plane
    assert c(FAKE, 1 << 62, FAKE, 6, 3, 2, 3, 8, 0, 0, FAKE, None, None) == 2  # span overflows
    assert c(FAKE, 48, FAKE, 1 << 62, 3, 2, 3, 8, 0, 0, FAKE, None, None) == 2  # lse span overflows
    assert c(None, 64, FAKE, 8, 2, 2, 3, 8, 0, 0, FAKE, None, None) == 1
    assert c(FAKE, 64, FAKE, 8, 2, 2, 3, 8, 9, 0, FAKE, None, None) == 4
    assert c(FAKE, 64, FAKE, 8, 2, 2, 3, 8, 0, 7, FAKE, None, None) == 6
    assert c(FAKE + 1, 64, FAKE, 8, 2, 2, 3, 8, 0, 0, FAKE, None, None) == 5
    assert c(FAKE, 64, FAKE + 2, 8, 2, 2, 3, 8, 0, 0, FAKE, None, None) == 5
    assert c(None, 64, None, 8, 2, 0, 3, 8, 0, 0, None, None, None) == 0      # T = 0
    assert c(FAKE, 64, FAKE, 8, 0, 2, 3, 8, 0, 0, FAKE, None, None) == 2      # N < 1


def test_combine_planes_valid_validation(lib):
    c = lib.lsec_combine_planes_valid
    # outputs, plane_stride, lses, lse_plane_stride, N, T, H, D, dtype, base,
    # query_start_loc, num_reqs, out, out_lse, stream
    assert c(FAKE, 64, FAKE, 8, 2, 2, 3, 8, 0, 0, None, 1, FAKE, None, None) == 1   # NULL offsets
    assert c(FAKE, 64, FAKE, 8, 2, 2, 3, 8, 0, 0, FAKE + 2, 1, FAKE, None, None) == 5  # misaligned
    assert c(FAKE, 64, FAKE, 8, 2, 2, 3, 8, 0, 0, FAKE, -1, FAKE, None, None) == 2  # num_reqs < 0
    assert c(FAKE, 1 << 40, FAKE, 1 << 34, 2, 1, 1 << 32, 8, 0, 0, FAKE, 1, FAKE, None,
             None) == 2                                                              # H >= 2^32
    assert c(FAKE, 47, FAKE, 6, 2, 2, 3, 8, 0, 0, FAKE, 1, FAKE, None, None) == 2   # stride < plane
    assert c(FAKE, 64, FAKE, 8, 2, 2, 3, 8, 9, 0, FAKE, 1, FAKE, None, None) == 4   # dtype
    assert c(FAKE, 64, FAKE, 8, 2, 2, 3, 8, 0, 7, FAKE, 1, FAKE, None, None) == 6   # base
    assert c(None, 64, None, 8, 2, 0, 3, 8, 0, 0, None, 1, None, None, None) == 0   # T = 0


def test_header_and_c_consumer_compile_as_c99():
    """include/lsec.h is a plain C header: the C consumer of the library
    compiles as C99 with warnings as errors (nothing is linked or run)."""
    src = os.path.join(ROOT, "tests", "c_abi", "c_abi_check.c")
    cmd = ["gcc", "-std=c99", "-fsyntax-only", "-Wall", "-Wextra", "-Werror",
           "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
           "-I", "/opt/rocm/include", src]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr


def test_dcp_a2a_lse_reduce_host_contract():
    """The page's dcp_a2a_lse_reduce contract before any kernel runs: world
    size 1 returns the inputs themselves, H % world_size != 0 raises
    ValueError, and a multi-rank call needs an exchange."""
    import torch

    import lse_weighted_merge_combine_amd as lsec
    out = torch.zeros((3, 8, 16), dtype=torch.bfloat16)
    lse = torch.zeros((3, 8), dtype=torch.float32)
    assert lsec.dcp_a2a_lse_reduce(out, lse, 1) is out
    o2, l2 = lsec.dcp_a2a_lse_reduce(out, lse, 1, return_lse=True)
    assert o2 is out and l2 is lse
    with pytest.raises(ValueError, match="divisible"):
        lsec.dcp_a2a_lse_reduce(out, lse, 3)
    with pytest.raises(ValueError, match="exchange"):
        lsec.dcp_a2a_lse_reduce(out, lse, 4)


def test_send_recv_buffers_are_kept_per_shape():
    """dcp_a2a_send_recv_buffers hands out one send and one receive buffer
    per (shape, device, dtype) and the same ones on every later call."""
    import torch

    import lse_weighted_merge_combine_amd as lsec
    s1, r1 = lsec.dcp_a2a_send_recv_buffers((4, 3, 2, 130), "cpu", torch.bfloat16)
    assert tuple(s1.shape) == (4, 3, 2, 130) and s1.dtype == torch.bfloat16
    assert s1.data_ptr() != r1.data_ptr()
    s2, r2 = lsec.dcp_a2a_send_recv_buffers([4, 3, 2, 130], torch.device("cpu"), torch.bfloat16)
    assert s2 is s1 and r2 is r1
    s3, _ = lsec.dcp_a2a_send_recv_buffers((4, 3, 2, 130), "cpu", torch.float16)
    assert s3 is not s1
    s4, _ = lsec.dcp_a2a_send_recv_buffers((4, 3, 4, 130), "cpu", torch.bfloat16)
    assert s4 is not s1
    with pytest.raises(ValueError):
        lsec.dcp_a2a_send_recv_buffers((4, 3, 130), "cpu", torch.bfloat16)
    with pytest.raises(ValueError):
        lsec.dcp_a2a_send_recv_buffers((4, 3, 2, 130), "cpu", torch.int8)


def test_floor_read_validation(lib):
    """The measurement aids check their arguments before launching."""
    assert lib.lsec_floor_read_blocks(0) == 0
    assert lib.lsec_floor_read_blocks(16) == 1
    assert lib.lsec_floor_read_blocks(16384) == 1
    assert lib.lsec_floor_read_blocks(16400) == 2
    assert lib.lsec_floor_read_blocks(-16) == -1
    assert lib.lsec_floor_read_blocks(24) == -1
    fake = ctypes.c_void_p(1 << 20)
    assert lib.lsec_floor_read(fake, 24, fake, None) == 2       # SHAPE: not a multiple of 16
    assert lib.lsec_floor_read(fake, -16, fake, None) == 2      # SHAPE
    assert lib.lsec_floor_read(None, 0, None, None) == 0        # nothing to read, nothing launched
    assert lib.lsec_floor_read(None, 32, fake, None) == 1       # NULL
    assert lib.lsec_floor_read(fake, 32, None, None) == 1       # NULL
    assert lib.lsec_floor_read(ctypes.c_void_p((1 << 20) + 4), 32, fake, None) == 5  # ALIGNMENT
    assert lib.lsec_floor_read(fake, 32, ctypes.c_void_p((1 << 20) + 2), None) == 5  # ALIGNMENT
    other = ctypes.c_void_p(1 << 21)
    assert lib.lsec_floor_copy(fake, other, 24, None) == 2      # SHAPE
    assert lib.lsec_floor_copy(None, None, 0, None) == 0        # nothing to copy
    assert lib.lsec_floor_copy(None, other, 32, None) == 1      # NULL
    assert lib.lsec_floor_copy(fake, None, 32, None) == 1       # NULL
    assert lib.lsec_floor_copy(fake, ctypes.c_void_p((1 << 21) + 8), 32, None) == 5  # ALIGNMENT


def test_time_next_launch_arms_and_disarms(lib):
    """Arming and disarming touch no GPU state; exactly one NULL is an error."""
    lib.lsec_time_next_launch.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    fake = ctypes.c_void_p(1 << 20)
    assert lib.lsec_time_next_launch(fake, None) == 1           # NULL
    assert lib.lsec_time_next_launch(None, fake) == 1           # NULL
    assert lib.lsec_time_next_launch(None, None) == 0           # disarm (nothing armed)
    assert lib.lsec_time_next_launch(fake, fake) == 0           # armed ...
    assert lib.lsec_time_next_launch(None, None) == 0           # ... and disarmed unused


def test_floor_header_compiles_as_c99(tmp_path):
    src = tmp_path / "use_floor.c"
    src.write_text('#include "lsec_floor.h"\n#include "lsec.h"\n'
                   'int main(void) { return lsec_floor_read_blocks(16) == 1 ? 0 : 1; }\n')
    res = subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-fsyntax-only",
                          "-I", os.path.join(ROOT, "include"), str(src)],
                         capture_output=True, text=True)
    assert res.returncode == 0, res.stderr


def test_binding_fails_loudly_without_the_library(tmp_path):
    """With liblsec.so absent, every hot-path entry point of the binding
    raises instead of computing anything: there is no CPU fallback, and the
    oracle is never imported."""
    import shutil
    pkg = os.path.join(ROOT, "lse_weighted_merge_combine_amd")
    shutil.copytree(pkg, tmp_path / "lse_weighted_merge_combine_amd",
                    ignore=shutil.ignore_patterns("*.so", "__pycache__"))
    code = f"""
import sys, torch
sys.path.insert(0, {str(tmp_path)!r})
import lse_weighted_merge_combine_amd as m
assert m.__file__.startswith({str(tmp_path)!r}), m.__file__
o = torch.zeros(2, 3, 4, 128, dtype=torch.bfloat16)
l = torch.zeros(2, 3, 4)
calls = [(m.lse_combine, (o, l)), (m.lsec_combine, (o, l)), (m.pack_send, (o[0], l[0], 2)),
         (m.unpack_combine, (torch.zeros(2, 3, 2, 130, dtype=torch.bfloat16), 128)),
         (m.lse_weighted_combine, (o, l)), (m.load_library, ())]
for fn, args in calls:
    try:
        fn(*args)
    except (ImportError, ValueError) as e:
        pass
    else:
        raise SystemExit(f"{{fn.__name__}} returned without the library")
try:
    m.load_library()
except ImportError as e:
    assert "missing" in str(e), e
assert "oracle" not in sys.modules
print("ok")
"""
    res = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    assert res.returncode == 0 and res.stdout.strip().endswith("ok"), res.stdout + res.stderr
