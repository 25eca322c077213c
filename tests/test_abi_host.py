"""Host-side checks of the C ABI (no GPU needed).

- libnvfp4.so and its checked build libnvfp4_checked.so load and export
  every function include/nvfp4.h declares and no self-test hook;
  libnvfp4_selftest.so exports those include/nvfp4_selftest.h declares; the
  device-side precondition checks exist only in the checked build;
- in both builds, argument errors return the documented status before any
  HIP call (null pointers, negative sizes, k % 16 != 0, misaligned
  pointers, zero groups), and empty problems return success without
  launching.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nvfp4.h")
SELFTEST_HEADER = os.path.join(ROOT, "include", "nvfp4_selftest.h")

OK, INVALID, SHAPE, MISALIGNED = 0, 1, 2, 3


@pytest.fixture(scope="module", params=["product", "checked"])
def L(request):
    import nvfp4_token_quantization_amd as nv
    return nv.load(nv.PRODUCT_LIB_PATH if request.param == "product" else nv.CHECKED_LIB_PATH)


@pytest.fixture(scope="module")
def S():
    import nvfp4_token_quantization_amd.selftest as st
    return st.lib()


def declared_functions(header=HEADER):
    txt = open(header).read()
    return re.findall(r"^(?:int|const char\*)\s+(nvfp4_\w+)\(", txt, re.M)


def test_header_declares_the_boundary():
    names = set(declared_functions())
    for n in ("nvfp4_quantize_rows", "nvfp4_quantize_weight", "nvfp4_gemm", "nvfp4_grouped_gemm",
              "nvfp4_status_string", "nvfp4_version"):
        assert n in names


def test_library_exports_every_declared_symbol(L):
    for name in declared_functions():
        assert hasattr(L, name), name


def test_selftest_hooks_live_outside_the_product_library(L, S):
    hooks = declared_functions(SELFTEST_HEADER)
    assert sorted(hooks) == ["nvfp4_debug_block_scale", "nvfp4_debug_encode_e2m1",
                             "nvfp4_debug_encode_e4m3", "nvfp4_debug_encode_fp8",
                             "nvfp4_debug_quantize_weight_onepass"]
    assert not set(hooks) & set(declared_functions())
    for name in hooks:
        assert hasattr(S, name), name
        assert not hasattr(L, name), name


def test_status_strings_and_version(L):
    assert L.nvfp4_version() == 100
    for st in range(7):
        assert L.nvfp4_status_string(st) != b"unknown status"
    assert b"precondition" in L.nvfp4_status_string(6)
    assert L.nvfp4_status_string(99) == b"unknown status"


def test_precondition_checks_only_in_the_checked_build():
    import nvfp4_token_quantization_amd as nv
    check_symbol = "_ZN10nvfp4check6Checks6resultEv"  # nvfp4check::Checks::result()
    assert hasattr(nv.load(nv.CHECKED_LIB_PATH), check_symbol)
    assert not hasattr(nv.load(nv.PRODUCT_LIB_PATH), check_symbol)
    assert nv.LIB_PATH == nv.PRODUCT_LIB_PATH or os.environ.get("NVFP4_CHECKED")


FAKE = 0x10000          # 16-byte aligned, never dereferenced (errors return first)
FAKE_ODD = 0x10001


def P(v):
    return ctypes.c_void_p(v)


def test_quantize_rows_argument_errors(L):
    f = L.nvfp4_quantize_rows
    assert f(P(FAKE), -1, 16, None, P(FAKE), P(FAKE), P(FAKE), None) == INVALID
    assert f(P(FAKE), 4, -16, None, P(FAKE), P(FAKE), P(FAKE), None) == INVALID
    assert f(P(FAKE), 4, 24, None, P(FAKE), P(FAKE), P(FAKE), None) == SHAPE
    assert f(None, 4, 16, None, P(FAKE), P(FAKE), P(FAKE), None) == INVALID
    assert f(P(FAKE), 4, 16, None, None, P(FAKE), P(FAKE), None) == INVALID
    assert f(P(FAKE), 4, 16, None, P(FAKE), None, P(FAKE), None) == INVALID
    assert f(P(FAKE), 4, 16, None, P(FAKE), P(FAKE), None, None) == INVALID
    assert f(P(FAKE_ODD), 4, 16, None, P(FAKE), P(FAKE), P(FAKE), None) == MISALIGNED
    assert f(P(FAKE), 4, 16, None, P(FAKE + 8), P(FAKE), P(FAKE), None) == MISALIGNED
    # nothing to do: success without touching the device
    assert f(None, 0, 16, None, None, None, None, None) == OK


def test_quantize_weight_argument_errors(L):
    f = L.nvfp4_quantize_weight
    a = P(FAKE)
    assert f(a, 0, 4, 16, None, a, a, a, a, None) == INVALID        # zero groups
    assert f(a, 2, -1, 16, None, a, a, a, a, None) == INVALID
    assert f(a, 2, 4, 40, None, a, a, a, a, None) == SHAPE
    assert f(a, 2, 4, 16, None, None, a, a, a, None) == INVALID     # no amax target
    assert f(a, 2, 4, 16, None, a, a, a, None, None) == INVALID     # no s
    assert f(None, 2, 4, 16, None, a, a, a, a, None) == INVALID
    assert f(P(FAKE_ODD), 2, 4, 16, None, a, a, a, a, None) == MISALIGNED
    # amax_out and s overlapping (the same array, or shifted by one entry)
    assert f(a, 2, 4, 16, None, a, a, a, a, None) == INVALID
    assert f(a, 2, 4, 16, None, P(FAKE + 4), a, a, a, None) == INVALID


def test_onepass_hook_argument_errors(S):
    f = S.nvfp4_debug_quantize_weight_onepass
    a, ms = P(FAKE), ctypes.c_double(10.0)
    assert f(a, 0, 4, 16, a, a, a, a, ms, None) == INVALID                     # zero groups
    assert f(a, 2, 0, 16, a, a, a, a, ms, None) == INVALID                     # no rows
    assert f(a, 2, 4, 16, a, a, a, a, ctypes.c_double(-1.0), None) == INVALID  # negative limit
    assert f(a, 2, 4, 40, a, a, a, a, ms, None) == SHAPE
    assert f(a, 2, 4, 16, None, a, a, a, ms, None) == INVALID                  # no amax target
    assert f(a, 2, 4, 16, a, a, a, None, ms, None) == INVALID                  # no s
    assert f(P(FAKE_ODD), 2, 4, 16, a, a, a, a, ms, None) == MISALIGNED


def test_gemm_argument_errors(L):
    f = L.nvfp4_gemm
    a = P(FAKE)
    assert f(a, a, a, -1, a, a, a, 8, 16, a, None) == INVALID
    assert f(a, a, a, 8, a, a, a, 8, 20, a, None) == SHAPE
    assert f(a, a, a, 8, a, a, a, 8, 16, None, None) == INVALID
    assert f(None, a, a, 8, a, a, a, 8, 16, a, None) == INVALID
    assert f(a, a, a, 8, a, P(FAKE + 4), a, 8, 16, a, None) == MISALIGNED
    assert f(None, None, None, 0, None, None, None, 8, 16, None, None) == OK  # m == 0


def test_grouped_gemm_argument_errors(L):
    f = L.nvfp4_grouped_gemm
    a = P(FAKE)
    assert f(a, a, a, 8, None, 8, a, 0, a, a, a, 8, 16, a, None) == INVALID    # groups 0
    assert f(a, a, a, 8, None, 8, a, 2000, a, a, a, 8, 16, a, None) == SHAPE   # > 1024 groups
    assert f(a, a, a, 8, None, 8, a, 2, a, a, a, 8, 24, a, None) == SHAPE
    assert f(a, a, a, 8, None, 8, None, 2, a, a, a, 8, 16, a, None) == INVALID  # no offsets
    assert f(a, a, a, 4, None, 8, a, 2, a, a, a, 8, 16, a, None) == INVALID     # a_rows < m_total
    assert f(a, a, a, 8, P(FAKE + 2), 8, a, 2, a, a, a, 8, 16, a, None) == MISALIGNED
    assert f(None, None, None, 0, None, 0, None, 2, None, None, None, 8, 16, None, None) == OK


def test_gemm_grids_past_the_tile_limit(L):
    """Outputs whose tile grid would pass 2^28 tiles (far beyond device
    memory) are rejected as UNSUPPORTED_SHAPE before any HIP call, in every
    tiled GEMM entry point; the largest sizes each argument allows on its
    own still pass the other checks."""
    a = P(FAKE)
    big = 1 << 31
    assert L.nvfp4_gemm(a, a, a, big, a, a, a, big, 16, a, None) == SHAPE
    assert L.nvfp4_grouped_gemm(a, a, a, big, a, big, a, 4, a, a, a, big, 16, a, None) == SHAPE
    assert L.nvfp4_grouped_gemm_swiglu(a, a, a, 64, a, big, a, 4, a, a, a, (1 << 21) - 16, 256,
                                       a, a, None) == SHAPE
    assert L.nvfp4_mxfp8_gemm(a, a, big, a, a, big, 32, a, None) == SHAPE
    assert L.nvfp4_mxfp8_grouped_gemm(a, a, big, a, big, a, 4, a, a, big, 32, a, None) == SHAPE


def test_swiglu_quantize_argument_errors(L):
    f = L.nvfp4_swiglu_quantize_rows
    a = P(FAKE)
    assert f(a, -1, 16, None, None, a, a, a, None) == INVALID
    assert f(a, 4, 24, None, None, a, a, a, None) == SHAPE            # f % 16
    assert f(a, 4, 12304, None, None, a, a, a, None) == SHAPE         # f > 12288
    assert f(a, 4, 16, None, None, None, None, None, None) == INVALID  # no output
    assert f(a, 4, 16, None, None, a, None, a, None) == INVALID       # partial q/sb/s
    assert f(a, 4, 16, None, None, a, a, None, None) == INVALID       # q, sb without s
    assert f(None, 4, 16, None, None, a, a, a, None) == INVALID
    assert f(P(FAKE + 4), 4, 16, None, None, a, a, a, None) == MISALIGNED
    assert f(a, 4, 16, P(FAKE + 8), None, a, a, a, None) == MISALIGNED
    assert f(a, 4, 16, None, P(FAKE + 2), None, None, None, None) == MISALIGNED
    assert f(None, 0, 16, None, None, None, None, None, None) == OK     # no rows: nothing to do


def test_moe_route_argument_errors(L):
    f = L.nvfp4_moe_route
    a = P(FAKE)
    assert f(a, -1, 128, 8, a, a, a, a, None) == INVALID
    assert f(a, 4, 128, 0, a, a, a, a, None) == INVALID            # topk < 1
    assert f(a, 4, 8, 9, a, a, a, a, None) == INVALID              # topk > experts
    assert f(a, 4, 2048, 8, a, a, a, a, None) == SHAPE             # > 1024 experts
    assert f(a, 4, 128, 65, a, a, a, a, None) == SHAPE             # topk > 64
    assert f(a, 1 << 28, 128, 8, a, a, a, a, None) == SHAPE        # >= 2^31 routed rows
    assert f(a, 4, 128, 8, a, None, a, a, None) == INVALID         # offsets always needed
    assert f(None, 4, 128, 8, a, a, a, a, None) == INVALID
    assert f(a, 4, 128, 8, a, a, P(FAKE + 2), a, None) == MISALIGNED


def test_dequantize_argument_errors(L):
    f = L.nvfp4_dequantize_rows
    a = P(FAKE)
    assert f(a, a, a, -1, 16, 1, a, None) == INVALID
    assert f(a, a, a, 4, 16, 0, a, None) == INVALID              # rows_per_scale < 1
    assert f(a, a, a, 4, 24, 1, a, None) == SHAPE
    assert f(None, a, a, 4, 16, 1, a, None) == INVALID
    assert f(a, a, a, 4, 16, 1, None, None) == INVALID
    assert f(P(FAKE + 8), a, a, 4, 16, 1, a, None) == MISALIGNED
    assert f(a, a, a, 4, 16, 1, P(FAKE + 2), None) == MISALIGNED
    assert f(None, None, None, 0, 16, 1, None, None) == OK


def test_debug_hooks_argument_errors(S):
    assert S.nvfp4_debug_encode_e2m1(None, 4, P(FAKE), None) == INVALID
    assert S.nvfp4_debug_encode_e4m3(P(FAKE), -1, P(FAKE), None) == INVALID
    assert S.nvfp4_debug_encode_e4m3(P(FAKE + 1), 4, P(FAKE), None) == MISALIGNED
    assert S.nvfp4_debug_encode_e2m1(None, 0, None, None) == OK
    assert S.nvfp4_debug_encode_fp8(None, 4, P(FAKE), None) == INVALID
    assert S.nvfp4_debug_block_scale(P(FAKE), P(FAKE), 4, None, P(FAKE), None) == INVALID


def test_binding_fails_loudly_without_gpu_tensors():
    import torch

    import nvfp4_token_quantization_amd as nv
    with pytest.raises(ValueError):
        nv.nvfp4_quantize_rows(torch.zeros((4, 16), dtype=torch.bfloat16))  # CPU tensor
