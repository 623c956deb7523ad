"""C ABI contract of libbitlinear.so, checked without a GPU.

The library must load, export every function include/bitlinear.h declares, and return
each validation status synchronously, before anything is launched (fake, never
dereferenced device addresses are passed; a call that passed validation would need a
GPU, so only failing calls are made here).
"""
import ctypes

import numpy as np
import math
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bitlinear.h")
LIB = os.path.join(ROOT, "ternary_quantized_linear_amd", "libbitlinear.so")

BL_OK, BL_ERR_NULL, BL_ERR_DIM, BL_ERR_K_TOO_LARGE, BL_ERR_WORKSPACE, BL_ERR_ALIGN, \
    BL_ERR_HIP, BL_ERR_ARG = range(8)
MAX_K = 132104

P = ctypes.c_void_p
I64 = ctypes.c_int64
A = P(0x100000)      # 16-byte aligned fake device addresses
B = P(0x200000)
C = P(0x300000)
D = P(0x400000)
E = P(0x500000)
MIS = P(0x100004)    # misaligned


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        import __graft_entry__  # noqa: F401  (the library is not built yet: build it)
        __graft_entry__.build()
    return ctypes.CDLL(LIB)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"\b(bitlinear_\w+)\s*\(", text)
    return sorted(set(names))


def test_header_declares_the_abi():
    names = declared_functions()
    for n in ["bitlinear_quantize_weights", "bitlinear_quantize_acts", "bitlinear_forward",
              "bitlinear_forward_ex", "bitlinear_forward_grouped",
              "bitlinear_quantize_acts_grouped", "bitlinear_weight_workspace_bytes",
              "bitlinear_status_str", "bitlinear_last_hip_error", "bitlinear_abi_version",
              "bitlinear_forward_choice", "bitlinear_quantize_weights_sign",
              "bitlinear_forward_sign", "bitlinear_forward_sign_grouped",
              "bitlinear_quantize_weights_scale_groups", "bitlinear_forward_scale_groups",
              "bitlinear_forward_grouped_scale_groups", "bitlinear_warmup_lambda",
              "bitlinear_fake_quant_weights", "bitlinear_fake_quant_acts",
              "bitlinear_rmsnorm_backward", "bitlinear_bitdelta_compress",
              "bitlinear_bitdelta_forward", "bitlinear_forward_workspace_bytes",
              "bitlinear_forward_ws", "bitlinear_forward_grouped_ws",
              "bitlinear_forward_choice_ws"]:
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for n in declared_functions():
        assert hasattr(lib, n), "missing export " + n


def test_abi_version_and_strings(lib):
    lib.bitlinear_abi_version.restype = ctypes.c_int
    assert lib.bitlinear_abi_version() == 1
    lib.bitlinear_status_str.restype = ctypes.c_char_p
    lib.bitlinear_status_str.argtypes = [ctypes.c_int]
    for s in range(8):
        assert lib.bitlinear_status_str(s)
    assert lib.bitlinear_status_str(0) == b"ok"
    lib.bitlinear_last_hip_error.restype = ctypes.c_char_p
    assert lib.bitlinear_last_hip_error() == b""


def _qw(lib):
    f = lib.bitlinear_quantize_weights
    f.argtypes = [P, I64, I64, P, P, P, P, ctypes.c_size_t, P]
    f.restype = ctypes.c_int
    lib.bitlinear_weight_workspace_bytes.argtypes = [I64, I64]
    lib.bitlinear_weight_workspace_bytes.restype = ctypes.c_size_t
    return f


def test_quantize_weights_validation(lib):
    f = _qw(lib)
    ws = lib.bitlinear_weight_workspace_bytes(256, 1024)
    assert ws > 0
    assert f(None, 256, 1024, B, C, None, D, ws, None) == BL_ERR_NULL
    assert f(A, 256, 1024, None, C, None, D, ws, None) == BL_ERR_NULL
    assert f(A, 256, 1024, B, None, None, D, ws, None) == BL_ERR_NULL
    assert f(A, 0, 1024, B, C, None, D, ws, None) == BL_ERR_DIM
    assert f(A, 256, -4, B, C, None, D, ws, None) == BL_ERR_DIM
    assert f(A, 256, 1022, B, C, None, D, ws, None) == BL_ERR_DIM
    assert f(A, 1 << 20, 1 << 12, B, C, None, D, ws, None) == BL_ERR_DIM  # > 2^31 weights
    assert f(A, 256, 1024, B, C, None, None, ws, None) == BL_ERR_WORKSPACE
    assert f(A, 256, 1024, B, C, None, D, ws - 1, None) == BL_ERR_WORKSPACE
    assert f(MIS, 256, 1024, B, C, None, D, ws, None) == BL_ERR_ALIGN
    assert f(A, 256, 1024, B, C, P(0x300004), D, ws, None) == BL_ERR_ALIGN  # gamma not 8-aligned


def _qa(lib):
    f = lib.bitlinear_quantize_acts
    f.argtypes = [P, P, I64, I64, ctypes.c_float, ctypes.c_uint32, P, P, P]
    f.restype = ctypes.c_int
    return f


def test_quantize_acts_validation(lib):
    f = _qa(lib)
    assert f(None, None, 8, 1024, 1e-6, 0, B, C, None) == BL_ERR_NULL
    assert f(A, None, 8, 1024, 1e-6, 0, None, C, None) == BL_ERR_NULL
    assert f(A, None, 8, 1024, 1e-6, 0, B, None, None) == BL_ERR_NULL
    assert f(A, None, 0, 1024, 1e-6, 0, B, C, None) == BL_ERR_DIM
    assert f(A, None, 8, 1026, 1e-6, 0, B, C, None) == BL_ERR_DIM
    assert f(A, None, 70000, 1024, 1e-6, 0, B, C, None) == BL_ERR_DIM
    assert f(A, None, 8, MAX_K + 4, 1e-6, 0, B, C, None) == BL_ERR_K_TOO_LARGE
    assert f(A, None, 8, 1024, -1.0, 0, B, C, None) == BL_ERR_ARG
    assert f(A, None, 8, 1024, math.nan, 0, B, C, None) == BL_ERR_ARG
    assert f(A, None, 8, 1024, math.inf, 0, B, C, None) == BL_ERR_ARG
    assert f(A, None, 8, 1024, 1e-6, 2, B, C, None) == BL_ERR_ARG
    assert f(MIS, None, 8, 1024, 1e-6, 0, B, C, None) == BL_ERR_ALIGN
    assert f(A, None, 8, 1024, 1e-6, 0, MIS, C, None) == BL_ERR_ALIGN
    assert f(A, MIS, 8, 1024, 1e-6, 0, B, C, None) == BL_ERR_ALIGN  # gain


class ActDesc(ctypes.Structure):
    _fields_ = [("X", P), ("gain", P), ("Xq", P), ("x_scale", P), ("K", I64)]


class ProjDesc(ctypes.Structure):
    _fields_ = [("Xq", P), ("x_scale", P), ("W_packed", P), ("w_scale", P), ("Y", P),
                ("acc", P), ("N", I64), ("K", I64)]


def test_grouped_validation(lib):
    fa = lib.bitlinear_quantize_acts_grouped
    fa.argtypes = [ctypes.POINTER(ActDesc), ctypes.c_int, I64, ctypes.c_float, ctypes.c_uint32, P]
    fa.restype = ctypes.c_int
    arr = (ActDesc * 9)(*[ActDesc(A.value, None, B.value, C.value, 1024) for _ in range(9)])
    assert fa(None, 1, 8, 1e-6, 0, None) == BL_ERR_NULL
    assert fa(arr, 0, 8, 1e-6, 0, None) == BL_ERR_ARG
    assert fa(arr, 9, 8, 1e-6, 0, None) == BL_ERR_ARG
    arr[3].K = 1030
    assert fa(arr, 4, 8, 1e-6, 0, None) == BL_ERR_DIM
    fp = lib.bitlinear_forward_grouped
    fp.argtypes = [ctypes.POINTER(ProjDesc), ctypes.c_int, I64, P]
    fp.restype = ctypes.c_int
    pa = (ProjDesc * 9)(*[ProjDesc(A.value, B.value, C.value, D.value, E.value, None, 64, 1024)
                          for _ in range(9)])
    assert fp(None, 1, 1, None) == BL_ERR_NULL
    assert fp(pa, 0, 1, None) == BL_ERR_ARG
    assert fp(pa, 9, 1, None) == BL_ERR_ARG
    pa[2].Y = None
    assert fp(pa, 3, 1, None) == BL_ERR_NULL


def _fw(lib):
    f = lib.bitlinear_forward_ex
    f.argtypes = [P, P, I64, I64, P, P, I64, P, P, ctypes.c_int, P]
    f.restype = ctypes.c_int
    return f


def test_forward_validation(lib):
    f = _fw(lib)
    g = lib.bitlinear_forward
    g.argtypes = [P, P, I64, I64, P, P, I64, P, P, P]
    g.restype = ctypes.c_int
    assert g(None, B, 1, 4096, C, D, 4096, E, None, None) == BL_ERR_NULL
    assert g(A, B, 1, 4096, C, D, 4096, None, None, None) == BL_ERR_NULL
    assert g(A, B, 1, 4096, None, D, 4096, E, None, None) == BL_ERR_NULL
    assert g(A, B, 0, 4096, C, D, 4096, E, None, None) == BL_ERR_DIM
    assert g(A, B, 1, 4098, C, D, 4096, E, None, None) == BL_ERR_DIM
    assert g(A, B, 1, 4096, C, D, 0, E, None, None) == BL_ERR_DIM
    assert g(A, B, 1, MAX_K + 4, C, D, 4096, E, None, None) == BL_ERR_K_TOO_LARGE
    assert g(A, B, 1, 4096, MIS, D, 4096, E, None, None) == BL_ERR_ALIGN
    assert g(A, B, 1, 4096, C, D, 4096, MIS, None, None) == BL_ERR_ALIGN
    assert g(A, B, 1, 4096, C, D, 4096, E, MIS, None) == BL_ERR_ALIGN
    # explicit kernels outside their shapes
    assert f(A, B, 2, 4096, C, D, 4096, E, None, 1, None) == BL_ERR_ARG  # gemv: T == 1
    assert f(A, B, 1, 4128, C, D, 4096, E, None, 1, None) == BL_ERR_ARG  # gemv: K % 64
    assert f(A, B, 1, 4160, C, D, 4096, E, None, 2, None) == BL_ERR_ARG  # skinny: K % 256
    assert f(A, B, 129, 4096, C, D, 4096, E, None, 2, None) == BL_ERR_ARG  # skinny: T <= 128
    assert f(A, B, 8, 4160, C, D, 4096, E, None, 3, None) == BL_ERR_ARG  # prefill: K % 128
    assert f(A, B, 1, 4096, C, D, 4096, E, None, 7, None) == BL_ERR_ARG  # no such kernel


def test_dispatch_choice(lib):
    f = lib.bitlinear_forward_choice
    f.argtypes = [I64, I64, I64]
    f.restype = ctypes.c_int
    assert f(1, 4096, 4096) == 1
    assert f(1, 4096, 14336) == 1
    assert f(2, 4096, 4096) == 2
    assert f(16, 4096, 4096) == 2
    # without a workspace the tiled GEMM cannot split K: the streaming kernel up to 95
    assert f(32, 8192, 28672) == 2
    assert f(64, 8192, 28672) == 2
    assert f(64, 14336, 4096) == 2
    assert f(96, 4096, 4096) == 3
    assert f(128, 28672, 8192) == 3
    assert f(129, 28672, 8192) == 3
    assert f(128, 65536, 4096) == 3   # 512 GEMM tiles
    assert f(2048, 14336, 4096) == 3
    assert f(8, 256, 1028) == 4


def test_split_k_workspace_query_and_validation(lib):
    # split-K workspace: one int32 plane [T, N] per K slice, slices chosen so that the
    # 256-row tiles fill 256 CUs with at least 8 k-tiles of 128 codes each
    q = lib.bitlinear_forward_workspace_bytes
    q.argtypes = [I64, I64, I64]
    q.restype = ctypes.c_size_t
    assert q(40, 12288, 4096) == 4 * 40 * 12288 * 4     # 48 tiles, 4 slices (32 k-tiles)
    assert q(64, 8192, 28672) == 8 * 64 * 8192 * 4      # 32 tiles, 8 slices
    assert q(64, 65536, 4096) == 0                      # 256 tiles: no split
    assert q(129, 8192, 28672) == 0                     # beyond 128 tokens
    assert q(0, 8192, 28672) == 0 and q(8, 8192, 4098) == 0
    c = lib.bitlinear_forward_choice_ws
    c.argtypes = [I64, I64, I64, ctypes.c_size_t]
    c.restype = ctypes.c_int
    for T, N, K, k in [(16, 8192, 28672, 2), (17, 8192, 28672, 3), (64, 8192, 28672, 3),
                       (32, 28672, 8192, 2), (64, 28672, 8192, 2), (65, 28672, 8192, 3),
                       (64, 4096, 4096, 2)]:
        # beyond 16 tokens at K >= 16384, beyond 64 (a second streaming pass) when the
        # slices fill the device (112 row tiles x 3 slices, 32 x 8); 16 row tiles x 4
        # slices do not
        assert c(T, N, K, q(T, N, K)) == k, (T, N, K)
    need = q(80, 14336, 4096)
    assert c(80, 14336, 4096, need) == 3 and c(80, 14336, 4096, need - 4) == 2
    plain = lib.bitlinear_forward_choice
    plain.argtypes = [I64, I64, I64]
    plain.restype = ctypes.c_int
    assert c(80, 14336, 4096, 0) == plain(80, 14336, 4096) == 2
    f = lib.bitlinear_forward_ws
    f.argtypes = [P, P, I64, I64, P, P, I64, P, P, ctypes.c_int, P, ctypes.c_size_t, P]
    f.restype = ctypes.c_int
    A, B, C, D, E = 1 << 20, 2 << 20, 3 << 20, 4 << 20, 5 << 20   # aligned, never touched
    assert f(A, B, 40, 4096, C, D, 12288, E, None, 3, (6 << 20) + 8, 1 << 24, None) == BL_ERR_ALIGN
    g = lib.bitlinear_forward_grouped_ws
    g.argtypes = [P, ctypes.c_int, I64, P, ctypes.c_size_t, P]
    g.restype = ctypes.c_int
    assert g(None, 1, 40, None, 0, None) == BL_ERR_NULL


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    # the package must raise, not fall back, when its shared library is missing
    import importlib.util
    src = os.path.join(ROOT, "ternary_quantized_linear_amd", "__init__.py")
    pkg = tmp_path / "ternary_quantized_linear_amd"
    pkg.mkdir()
    (pkg / "__init__.py").write_text(open(src).read())
    spec = importlib.util.spec_from_file_location("tql_nolib", str(pkg / "__init__.py"))
    mod = importlib.util.module_from_spec(spec)
    with pytest.raises(ImportError):
        spec.loader.exec_module(mod)


def test_sign_variant_validation(lib):
    f = lib.bitlinear_quantize_weights_sign
    f.argtypes = [P, I64, I64, P, P, P, P, ctypes.c_size_t, P]
    f.restype = ctypes.c_int
    lib.bitlinear_weight_workspace_bytes.argtypes = [I64, I64]
    lib.bitlinear_weight_workspace_bytes.restype = ctypes.c_size_t
    ws = lib.bitlinear_weight_workspace_bytes(256, 1024)
    assert f(None, 256, 1024, B, C, None, D, ws, None) == BL_ERR_NULL
    assert f(A, 256, 1024, None, C, None, D, ws, None) == BL_ERR_NULL
    assert f(A, 256, 1020, B, C, None, D, ws, None) == BL_ERR_DIM  # K % 8
    assert f(A, 256, 1024, B, C, None, D, ws - 1, None) == BL_ERR_WORKSPACE
    assert f(A, 256, 1024, MIS, C, None, D, ws, None) == BL_ERR_ALIGN
    assert f(A, 256, 1024, B, C, P(0x300004), D, ws, None) == BL_ERR_ALIGN  # alpha
    g = lib.bitlinear_forward_sign
    g.argtypes = [P, P, I64, I64, P, P, I64, P, P, P]
    g.restype = ctypes.c_int
    assert g(None, B, 1, 4096, C, D, 4096, E, None, None) == BL_ERR_NULL
    assert g(A, B, 1, 4100, C, D, 4096, E, None, None) == BL_ERR_DIM  # K % 8
    assert g(A, B, 1, 4096, C, D, 4096, MIS, None, None) == BL_ERR_ALIGN
    fg = lib.bitlinear_forward_sign_grouped
    fg.argtypes = [ctypes.POINTER(ProjDesc), ctypes.c_int, I64, P]
    fg.restype = ctypes.c_int
    pa = (ProjDesc * 9)(*[ProjDesc(A.value, B.value, C.value, D.value, E.value, None, 64, 1024)
                          for _ in range(9)])
    assert fg(None, 1, 1, None) == BL_ERR_NULL
    assert fg(pa, 9, 1, None) == BL_ERR_ARG
    pa[1].K = 1028
    assert fg(pa, 2, 1, None) == BL_ERR_DIM


def test_scale_groups_validation(lib):
    f = lib.bitlinear_quantize_weights_scale_groups
    f.argtypes = [P, I64, I64, I64, P, P, P, P, ctypes.c_size_t, P]
    f.restype = ctypes.c_int
    lib.bitlinear_weight_workspace_bytes.argtypes = [I64, I64]
    lib.bitlinear_weight_workspace_bytes.restype = ctypes.c_size_t
    ws = lib.bitlinear_weight_workspace_bytes(256, 1024)
    assert f(A, 256, 1024, 0, B, C, None, D, ws, None) == BL_ERR_ARG
    assert f(A, 256, 1024, 3, B, C, None, D, ws, None) == BL_ERR_ARG   # 3 does not divide 256
    assert f(A, 256, 1024, 8, None, C, None, D, ws, None) == BL_ERR_NULL
    assert f(A, 256, 1024, 8, B, C, None, D, ws - 1, None) == BL_ERR_WORKSPACE
    g = lib.bitlinear_forward_scale_groups
    g.argtypes = [P, P, I64, I64, P, P, I64, I64, P, P, ctypes.c_int, P]
    g.restype = ctypes.c_int
    assert g(A, B, 1, 4096, C, D, 4096, 0, E, None, 0, None) == BL_ERR_ARG
    assert g(A, B, 1, 4096, C, D, 4096, 3, E, None, 0, None) == BL_ERR_ARG
    assert g(A, B, 2, 4096, C, D, 4096, 8, E, None, 1, None) == BL_ERR_ARG  # gemv: T == 1
    assert g(None, B, 1, 4096, C, D, 4096, 8, E, None, 0, None) == BL_ERR_NULL
    fg = lib.bitlinear_forward_grouped_scale_groups
    fg.argtypes = [ctypes.POINTER(ProjDesc), ctypes.POINTER(I64), ctypes.c_int, I64, P]
    fg.restype = ctypes.c_int
    pa = (ProjDesc * 2)(*[ProjDesc(A.value, B.value, C.value, D.value, E.value, None, 64, 1024)
                          for _ in range(2)])
    gr = (I64 * 2)(4, 3)
    assert fg(pa, None, 2, 1, None) == BL_ERR_NULL
    assert fg(pa, gr, 2, 1, None) == BL_ERR_ARG  # 3 does not divide 64


def test_training_side_validation_and_lambda(lib):
    lam = lib.bitlinear_warmup_lambda
    lam.argtypes = [I64, I64]
    lam.restype = ctypes.c_float
    assert [lam(t, 1000) for t in (-5, 0, 250, 999, 1000, 5000)] == \
        [0.0, 0.0, 0.25, np.float32(0.999), 1.0, 1.0]
    assert lam(3, 0) == 1.0
    f = lib.bitlinear_fake_quant_weights
    f.argtypes = [P, I64, I64, P, ctypes.c_float, P, P]
    f.restype = ctypes.c_int
    assert f(None, 4, 8, B, 0.5, C, None) == BL_ERR_NULL
    assert f(A, 4, 6, B, 0.5, C, None) == BL_ERR_DIM
    assert f(A, 4, 8, B, 1.5, C, None) == BL_ERR_ARG
    assert f(A, 4, 8, B, -0.1, C, None) == BL_ERR_ARG
    assert f(A, 4, 8, B, math.nan, C, None) == BL_ERR_ARG
    assert f(A, 4, 8, B, 0.5, MIS, None) == BL_ERR_ALIGN
    g = lib.bitlinear_fake_quant_acts
    g.argtypes = [P, P, I64, I64, ctypes.c_float, ctypes.c_uint32, ctypes.c_float, P, P, P, P, P]
    g.restype = ctypes.c_int
    assert g(A, None, 8, 1024, 1e-6, 0, 0.5, B, C, None, None, None) == BL_ERR_NULL
    assert g(A, None, 8, 1024, 1e-6, 0, 2.0, B, C, D, None, None) == BL_ERR_ARG
    assert g(A, None, 8, 1024, 1e-6, 0, 0.5, B, C, MIS, None, None) == BL_ERR_ALIGN
    assert g(A, None, 8, 1024, 1e-6, 0, 0.5, B, C, D, P(0x300004), None) == BL_ERR_ALIGN
    h = lib.bitlinear_rmsnorm_backward
    h.argtypes = [P, P, P, P, I64, I64, P, P, P]
    h.restype = ctypes.c_int
    assert h(A, None, None, B, 8, 1024, C, None, None) == BL_ERR_NULL
    assert h(A, None, D, B, 0, 1024, C, None, None) == BL_ERR_DIM
    assert h(A, None, P(0x300004), B, 8, 1024, C, None, None) == BL_ERR_ALIGN


def test_bitdelta_validation(lib):
    c = lib.bitlinear_bitdelta_compress
    c.argtypes = [P, P, I64, I64, ctypes.c_int, ctypes.c_int, P, P, P, ctypes.c_size_t, P]
    c.restype = ctypes.c_int
    lib.bitlinear_weight_workspace_bytes.argtypes = [I64, I64]
    lib.bitlinear_weight_workspace_bytes.restype = ctypes.c_size_t
    ws = lib.bitlinear_weight_workspace_bytes(64, 1024)
    assert c(None, B, 64, 1024, 8, 0, C, D, E, ws, None) == BL_ERR_NULL
    assert c(A, B, 64, 1000, 8, 0, C, D, E, ws, None) == BL_ERR_DIM     # M % 16
    assert c(A, B, 64, 16384, 8, 0, C, D, E, ws, None) == BL_ERR_DIM    # M <= 8192
    assert c(A, B, 64, 1024, 9, 0, C, D, E, ws, None) == BL_ERR_DIM     # B <= 8
    assert c(A, B, 64, 1024, 8, 8, C, D, E, ws, None) == BL_ERR_ARG     # model < B
    assert c(A, B, 64, 1024, 8, 0, C, D, E, ws - 1, None) == BL_ERR_WORKSPACE
    assert c(A, B, 64, 1024, 8, 0, MIS, D, E, ws, None) == BL_ERR_ALIGN
    f = lib.bitlinear_bitdelta_forward
    f.argtypes = [P, P, P, P, I64, I64, ctypes.c_int, P, P]
    f.restype = ctypes.c_int
    assert f(A, B, C, None, 64, 1024, 8, E, None) == BL_ERR_NULL
    assert f(A, B, C, D, 64, 1024, 0, E, None) == BL_ERR_DIM
    assert f(A, B, C, MIS, 64, 1024, 8, E, None) == BL_ERR_ALIGN
