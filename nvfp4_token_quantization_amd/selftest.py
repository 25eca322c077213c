"""Self-test hooks (test-only) over ``libnvfp4_selftest.so``, declared in
``include/nvfp4_selftest.h``: the quantizers' device rounding functions
applied to arbitrary float32 inputs, so tests can sweep every bit pattern, and
the one-pass weight quantizer on any group size with a chosen bound on its
wait.  Not part of the product boundary; raises if the library is not built."""
import ctypes
import os

import torch

import nvfp4_token_quantization_amd as nv

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libnvfp4_selftest.so")
_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libnvfp4_selftest.so is not built: run __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        P, I64 = ctypes.c_void_p, ctypes.c_int64
        for f in ("nvfp4_debug_encode_fp8", "nvfp4_debug_encode_e2m1", "nvfp4_debug_encode_e4m3"):
            getattr(L, f).argtypes = [P, I64, P, P]
            getattr(L, f).restype = ctypes.c_int
        L.nvfp4_debug_block_scale.argtypes = [P, P, I64, P, P, P]
        L.nvfp4_debug_block_scale.restype = ctypes.c_int
        L.nvfp4_debug_quantize_weight_onepass.argtypes = [P, I64, I64, I64, P, P, P, P, ctypes.c_double, P]
        L.nvfp4_debug_quantize_weight_onepass.restype = ctypes.c_int
        _lib = L
    return _lib


def nvfp4_debug_encode_e2m1(v):
    """Device E2M1 code (sign | RNE_SAT magnitude) of each float32 in v."""
    nv._dev(v, "v", (torch.float32,))
    out = torch.empty(v.shape, dtype=torch.uint8, device=v.device)
    nv._check("nvfp4_debug_encode_e2m1",
           lib().nvfp4_debug_encode_e2m1(nv._ptr(v), v.numel(), nv._ptr(out), nv._stream(v.device)))
    return out


def nvfp4_debug_encode_e4m3(v):
    """Device RNE_SAT E4M3 code of each non-negative float32 in v."""
    nv._dev(v, "v", (torch.float32,))
    out = torch.empty(v.shape, dtype=torch.uint8, device=v.device)
    nv._check("nvfp4_debug_encode_e4m3",
           lib().nvfp4_debug_encode_e4m3(nv._ptr(v), v.numel(), nv._ptr(out), nv._stream(v.device)))
    return out


def nvfp4_debug_block_scale(block_amax, amax):
    """The quantizer's block-scale step on arbitrary inputs: block_amax int16
    (bf16 bits of a block's largest magnitude) and amax float32 (the row's
    amax), same shape.  Returns (code uint8, inv float32)."""
    nv._dev(block_amax, "block_amax", (torch.int16,))
    nv._dev(amax, "amax", (torch.float32,))
    if block_amax.shape != amax.shape:
        raise ValueError("block_amax and amax differ in shape")
    code = torch.empty(amax.shape, dtype=torch.uint8, device=amax.device)
    inv = torch.empty(amax.shape, dtype=torch.float32, device=amax.device)
    nv._check("nvfp4_debug_block_scale",
           lib().nvfp4_debug_block_scale(nv._ptr(block_amax), nv._ptr(amax), amax.numel(), nv._ptr(code),
                                         nv._ptr(inv), nv._stream(amax.device)))
    return code, inv


def nvfp4_debug_encode_fp8(v):
    """E4M3 code (sign | RNE_SAT magnitude) of each float32 in v through the
    pack-convert the MXFP8 quantizer uses (specified for |v| <= 448)."""
    nv._dev(v, "v", (torch.float32,))
    out = torch.empty(v.shape, dtype=torch.uint8, device=v.device)
    nv._check("nvfp4_debug_encode_fp8",
           lib().nvfp4_debug_encode_fp8(nv._ptr(v), v.numel(), nv._ptr(out), nv._stream(v.device)))
    return out


def nvfp4_debug_quantize_weight_onepass(w, limit_ms=10.0):
    """nvfp4_quantize_weight of a bf16 [groups, rows, k] weight (group amax
    computed) forced onto the one-pass kernel, each workgroup's wait for its
    team bounded by limit_ms (0: workgroups that do not find the team complete
    read the whole group themselves).  Returns (q, sb, s, amax) shaped as
    nvfp4_quantize_weight's; raises NVFP4Error (UNSUPPORTED_SHAPE) when the
    kernel cannot hold a group."""
    nv._dev(w, "w", nv._BF16, 3)
    groups, rows, k = w.shape
    d = w.device
    q = torch.empty((groups, rows, k // 2), dtype=torch.uint8, device=d)
    sb = torch.empty((groups, rows, k // 16), dtype=torch.uint8, device=d)
    s = torch.empty(groups, dtype=torch.float32, device=d)
    amax = torch.empty(groups, dtype=torch.float32, device=d)
    nv._check("nvfp4_debug_quantize_weight_onepass",
              lib().nvfp4_debug_quantize_weight_onepass(nv._ptr(w), groups, rows, k, nv._ptr(amax), nv._ptr(q),
                                                        nv._ptr(sb), nv._ptr(s), float(limit_ms), nv._stream(d)))
    return q, sb, s, amax
