"""CPU oracle for the per-token NVFP4 path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product library
(``nvfp4_token_quantization_amd``) never imports it, and the two share no code.

The arithmetic lives in ``nvfp4_oracle.c`` (plain C, built with
``-ffp-contract=off`` and without fast-math so every fp32 step is one IEEE
operation).  This module only marshals numpy arrays.

Sources: the pages "miniTE报告：原生NVFP4训RL后期为何失稳，8×B300上提速1.37倍"
(section NVFP4格式、两级缩放与转换误差), "Towards Blackwell-Native 8-bit and 4-bit
RL: End-to-End MXFP8 and NVFP4 RL in Miles" (sections 速读, NVFP4格式背景,
位级精确的量化器契约) and "TRIAGE: Direction-Aware Mismatch Stabilization of
Native NVFP4 Reinforcement Learning" (section 前置知识, the decode formula
x_hat = S * s_b * Q_E2M1(x / (S * s_b))).

Every function here is pinned by the ``-m "not gpu"`` tests in
``tests/test_oracle_*.py`` against library routines, closed forms, invariants
and brute force.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "nvfp4_oracle.c")
_LIB = os.path.join(_HERE, "libnvfp4_oracle.so")
# an alternative build (the mutation tests load builds of patched copies of
# the source, each with one planted mistake); used as given, never rebuilt here
_LIB_OVERRIDE = os.environ.get("NVFP4_ORACLE_LIB")

GCC_FLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
             "-fno-fast-math", "-fexcess-precision=standard", "-Wall"]
SOURCE = _SRC


def build(force=False, src=None, path=None, extra_flags=()):
    """Compile the oracle with gcc (plain C, IEEE fp32, OpenMP).  `src` and
    `path` build another copy of the source into another library (the
    mutation tests and the sanitizer build use them)."""
    if src or path:
        out = path or (_LIB + ".alt")
        subprocess.check_call(["gcc"] + GCC_FLAGS + list(extra_flags) + [src or _SRC, "-o", out, "-lm"])
        return out
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc"] + GCC_FLAGS + [_SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if _LIB_OVERRIDE:
            L = ctypes.CDLL(_LIB_OVERRIDE)
        else:
            build()
            L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        L.oracle_threads.restype = ctypes.c_int
        L.oracle_set_threads.argtypes = [ctypes.c_int]
        L.oracle_set_threads.restype = None
        L.oracle_e2m1_value.argtypes = [ctypes.c_int]
        L.oracle_e2m1_value.restype = ctypes.c_double
        L.oracle_e4m3_value.argtypes = [ctypes.c_int]
        L.oracle_e4m3_value.restype = ctypes.c_double
        L.oracle_rne_sat_e2m1.argtypes = [ctypes.c_float]
        L.oracle_rne_sat_e2m1.restype = ctypes.c_int
        L.oracle_rne_sat_e4m3.argtypes = [ctypes.c_float]
        L.oracle_rne_sat_e4m3.restype = ctypes.c_int
        L.oracle_rne_sat_e2m1_array.argtypes = [P, I64, P]
        L.oracle_rne_sat_e4m3_array.argtypes = [P, I64, P]
        L.oracle_quantize_rows.argtypes = [P, I64, I64, P, P, P, P]
        L.oracle_quantize_rows.restype = ctypes.c_int
        L.oracle_quantize_weight.argtypes = [P, I64, I64, I64, P, P, P, P, P]
        L.oracle_quantize_weight.restype = ctypes.c_int
        L.oracle_dequantize.argtypes = [P, P, P, P, I64, I64, P]
        L.oracle_f32_to_bf16_array.argtypes = [P, I64, P]
        L.oracle_f64_to_bf16_array.argtypes = [P, I64, P]
        L.oracle_dequantize_bf16.argtypes = [P, P, P, I64, I64, I64, P]
        L.oracle_swiglu_rows.argtypes = [P, I64, I64, P]
        L.oracle_swiglu_rows.restype = ctypes.c_int
        L.oracle_route.argtypes = [P, I64, I64, I64, P, P, P, P]
        L.oracle_mxfp8_quantize_rows.argtypes = [P, I64, I64, P, P]
        L.oracle_mxfp8_quantize_rows.restype = ctypes.c_int
        L.oracle_mxfp8_gemm.argtypes = [P, P, I64, P, P, I64, I64, P, P]
        L.oracle_route.restype = ctypes.c_int
        L.oracle_gemm_entries.argtypes = [P, P, P, P, P, P, I64, P, P, P, I64, P, P]
        L.oracle_gemm.argtypes = [P, P, P, I64, P, P, P, I64, I64, P, P]
        L.oracle_grouped_gemm.argtypes = [P, P, P, P, P, I64, P, P, P, I64, I64, P, P]
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def threads():
    """OpenMP threads the oracle's parallel loops use."""
    return lib().oracle_threads()


def set_threads(n):
    """Set the OpenMP thread count of the oracle's parallel loops."""
    lib().oracle_set_threads(int(n))


# ------------------------------------------------------------------ codecs --
def e2m1_value(code):
    """Value of a 4-bit E2M1 code (sign, 2 exponent bits, 1 mantissa bit)."""
    return lib().oracle_e2m1_value(int(code))


def e4m3_value(code):
    """Value of an 8-bit E4M3 (OCP FN) code; NaN for 0x7F / 0xFF."""
    return lib().oracle_e4m3_value(int(code))


def e2m1_table():
    return np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)


def e4m3_table():
    return np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


def rne_sat_e2m1(v):
    """Non-negative E2M1 magnitude code (0..7) nearest to each fp32 v >= 0."""
    v = _c(np.atleast_1d(v), np.float32)
    out = np.empty(v.shape, np.uint8)
    lib().oracle_rne_sat_e2m1_array(_p(v), v.size, _p(out))
    return out


def rne_sat_e4m3(v):
    """Non-negative E4M3 code (0..0x7E) nearest to each fp32 v >= 0."""
    v = _c(np.atleast_1d(v), np.float32)
    out = np.empty(v.shape, np.uint8)
    lib().oracle_rne_sat_e4m3_array(_p(v), v.size, _p(out))
    return out


# --------------------------------------------------------------- quantizer --
def quantize_rows(x_bf16, amax_in=None):
    """Per-token NVFP4: x_bf16 is uint16 bf16 bits [rows, k], k % 16 == 0.

    Returns (q uint8 [rows, k/2], sb uint8 [rows, k/16], s float32 [rows]).
    """
    x = _c(x_bf16, np.uint16)
    rows, k = x.shape
    q = np.empty((rows, k // 2), np.uint8)
    sb = np.empty((rows, k // 16), np.uint8)
    s = np.empty((rows,), np.float32)
    a = None if amax_in is None else _c(amax_in, np.float32)
    rc = lib().oracle_quantize_rows(_p(x), rows, k, _p(a), _p(q), _p(sb), _p(s))
    if rc != 0:
        raise ValueError("oracle_quantize_rows: bad shape or non-finite input")
    return q, sb, s


def quantize_weight(w_bf16, amax_in=None):
    """Per-tensor / per-expert NVFP4: w_bf16 uint16 [groups, rows, k].

    Returns (q [groups, rows, k/2], sb [groups, rows, k/16], s float32 [groups],
    amax float32 [groups]).
    """
    w = _c(w_bf16, np.uint16)
    g, r, k = w.shape
    q = np.empty((g, r, k // 2), np.uint8)
    sb = np.empty((g, r, k // 16), np.uint8)
    s = np.empty((g,), np.float32)
    amax = np.empty((g,), np.float32)
    a = None if amax_in is None else _c(amax_in, np.float32)
    rc = lib().oracle_quantize_weight(_p(w), g, r, k, _p(a), _p(amax), _p(q), _p(sb), _p(s))
    if rc != 0:
        raise ValueError("oracle_quantize_weight: bad shape or non-finite input")
    return q, sb, s, amax


def dequantize(q, sb, s, s_index=None):
    """x_hat = S * s_b * e2m1(q) in fp64; q [rows, k/2], sb [rows, k/16]."""
    q = _c(q, np.uint8)
    sb = _c(sb, np.uint8)
    s = _c(s, np.float32)
    rows = q.shape[0]
    k = q.shape[1] * 2
    si = None if s_index is None else _c(s_index, np.int64)
    out = np.empty((rows, k), np.float64)
    lib().oracle_dequantize(_p(q), _p(sb), _p(s), _p(si), rows, k, _p(out))
    return out


# ------------------------------------------------------------ bf16, SwiGLU --
def f32_to_bf16(v):
    """bf16 bit patterns nearest to fp32 values (ties to even; not NaN)."""
    v = _c(v, np.float32)
    out = np.empty(v.shape, np.uint16)
    lib().oracle_f32_to_bf16_array(_p(v), v.size, _p(out))
    return out


def f64_to_bf16(v):
    """bf16 bit patterns nearest to float64 values (one rounding, ties to even)."""
    v = _c(v, np.float64)
    out = np.empty(v.shape, np.uint16)
    lib().oracle_f64_to_bf16_array(_p(v), v.size, _p(out))
    return out


def dequantize_bf16(q, sb, s, rows_per_scale=1):
    """bf16(S * s_b * e2m1(q)) rounded once; q [rows, k/2], sb [rows, k/16],
    s [rows / rows_per_scale].  Returns uint16 bf16 bits [rows, k]."""
    q = _c(q, np.uint8)
    sb = _c(sb, np.uint8)
    s = _c(np.atleast_1d(s), np.float32)
    rows = q.shape[0]
    k = q.shape[1] * 2
    out = np.empty((rows, k), np.uint16)
    lib().oracle_dequantize_bf16(_p(q), _p(sb), _p(s), rows, k, int(rows_per_scale), _p(out))
    return out


def swiglu_rows(gate_up):
    """h = bf16(fl32(silu(g) * u)) for a fused fp32 [rows, 2f] gate|up block
    (gate in columns [0, f), up in [f, 2f)).  Returns uint16 bf16 [rows, f]."""
    gu = _c(gate_up, np.float32)
    rows, f2 = gu.shape
    if f2 % 2:
        raise ValueError("gate_up must have an even number of columns")
    f = f2 // 2
    h = np.empty((rows, f), np.uint16)
    if lib().oracle_swiglu_rows(_p(gu), rows, f, _p(h)) != 0:
        raise ValueError("oracle_swiglu_rows: non-finite input or result")
    return h


def swiglu_quantize_rows(gate_up):
    """The fused SwiGLU -> per-token quantize chain: H = swiglu_rows(gate_up),
    its exact row amax, and quantize_rows(H) (which equals quantize_rows(H,
    amax_in=amax): amax reuse).  Returns (h, amax, q, sb, s)."""
    h = swiglu_rows(gate_up)
    amax = (np.abs((h.astype(np.uint32) << 16).view(np.float32)).max(axis=1)
            if h.shape[1] else np.zeros((h.shape[0],), np.float32)).astype(np.float32)
    q, sb, s = quantize_rows(h)
    return h, amax, q, sb, s


# ----------------------------------------------------------------- routing --
def route(logits, topk=8):
    """Top-k routing of fp32 logits [T, E] into the contiguous per-expert
    layout.  Returns dict(experts int32 [T, topk] (descending logit, lower id
    first on ties), offsets int32 [E+1], row_index int32 [T*topk] (token of
    each routed row, ordered by expert then token), slot_of int32 [T, topk]
    (routed row of each choice), counts int64 [E])."""
    lg = _c(logits, np.float32)
    T, E = lg.shape
    experts = np.empty((T, topk), np.int32)
    offsets = np.empty((E + 1,), np.int32)
    row_index = np.empty((T * topk,), np.int32)
    slot_of = np.empty((T, topk), np.int32)
    if lib().oracle_route(_p(lg), T, E, topk, _p(experts), _p(offsets), _p(row_index),
                          _p(slot_of)) != 0:
        raise ValueError("oracle_route: bad shape or non-finite logit")
    return dict(experts=experts, offsets=offsets, row_index=row_index, slot_of=slot_of,
                counts=np.diff(offsets).astype(np.int64))


# ------------------------------------------------------------------- MXFP8 --
def mxfp8_quantize_rows(x_bf16):
    """MXFP8 of bf16 rows [rows, k] (k % 32 == 0): E4M3 codes [rows, k] and
    E8M0 scale codes [rows, k/32] (2^(code - 127), rounded up)."""
    x = _c(x_bf16, np.uint16)
    rows, k = x.shape
    q = np.empty((rows, k), np.uint8)
    sc = np.empty((rows, k // 32), np.uint8)
    if lib().oracle_mxfp8_quantize_rows(_p(x), rows, k, _p(q), _p(sc)) != 0:
        raise ValueError("oracle_mxfp8_quantize_rows: bad shape or non-finite input")
    return q, sc


def mxfp8_dequantize(q, sc):
    """fp64 values of MXFP8 rows (exact)."""
    q = _c(q, np.uint8)
    sc = _c(sc, np.uint8)
    mag = e4m3_table()[q & 0x7F]
    v = np.where(q & 0x80, -mag, mag)
    return v * np.repeat(np.ldexp(1.0, sc.astype(np.int64) - 127), 32, axis=1)


def mxfp8_gemm(a, b):
    """(y_ref, bound) for Y = deq(A) . deq(B)^T, a = (q [m, k], sc [m, k/32]),
    b = (q [n, k], sc [n, k/32])."""
    aq, asc = _c(a[0], np.uint8), _c(a[1], np.uint8)
    bq, bsc = _c(b[0], np.uint8), _c(b[1], np.uint8)
    m, k = aq.shape
    n = bq.shape[0]
    y = np.empty((m, n), np.float64)
    bound = np.empty((m, n), np.float64)
    lib().oracle_mxfp8_gemm(_p(aq), _p(asc), m, _p(bq), _p(bsc), n, k, _p(y), _p(bound))
    return y, bound


# -------------------------------------------------------------------- GEMM --
def gemm(a, b):
    """Exact Y_ref and error bound for Y = deq(A) . deq(B)^T.

    a = (q [m, k/2], sb [m, k/16], s [m]); b = (q [n, k/2], sb [n, k/16], s [1]).
    Returns (y_ref fp64 [m, n], bound fp64 [m, n]) where bound = sum_k |a_k b_k|.
    """
    aq, asb, as_ = (_c(a[0], np.uint8), _c(a[1], np.uint8), _c(a[2], np.float32))
    bq, bsb, bs = (_c(b[0], np.uint8), _c(b[1], np.uint8), _c(np.atleast_1d(b[2]), np.float32))
    m, n, k = aq.shape[0], bq.shape[0], aq.shape[1] * 2
    y = np.empty((m, n), np.float64)
    bound = np.empty((m, n), np.float64)
    lib().oracle_gemm(_p(aq), _p(asb), _p(as_), m, _p(bq), _p(bsb), _p(bs), n, k, _p(y), _p(bound))
    return y, bound


def gemm_entries(a, b, a_row, b_row, b_scale):
    """Exact (y_ref, bound) for a list of entries: A row a_row[i] against B row
    b_row[i] (B flattened to [groups*n, k]) with B outer scale b_s[b_scale[i]]."""
    aq, asb, as_ = (_c(a[0], np.uint8), _c(a[1], np.uint8), _c(a[2], np.float32))
    bq, bsb, bs = (_c(b[0], np.uint8), _c(b[1], np.uint8), _c(np.atleast_1d(b[2]), np.float32))
    k = aq.shape[-1] * 2
    ar, br, bsi = _c(a_row, np.int64), _c(b_row, np.int64), _c(b_scale, np.int64)
    cnt = ar.size
    y = np.empty((cnt,), np.float64)
    bound = np.empty((cnt,), np.float64)
    lib().oracle_gemm_entries(_p(aq), _p(asb), _p(as_), _p(bq), _p(bsb), _p(bs), k,
                              _p(ar), _p(br), _p(bsi), cnt, _p(y), _p(bound))
    return y, bound


def grouped_gemm(a, offsets, b, row_index=None, m_total=None):
    """Exact (y_ref, bound) for the grouped GEMM over a contiguous per-expert
    layout.  b = (q [g, n, k/2], sb [g, n, k/16], s [g]).  Rows at or past
    offsets[g] are NaN in the returned arrays (not part of the product)."""
    aq, asb, as_ = (_c(a[0], np.uint8), _c(a[1], np.uint8), _c(a[2], np.float32))
    bq, bsb, bs = (_c(b[0], np.uint8), _c(b[1], np.uint8), _c(b[2], np.float32))
    off = _c(offsets, np.int32)
    groups, n, k = bq.shape[0], bq.shape[1], bq.shape[2] * 2
    if m_total is None:
        m_total = int(off[-1])
    ri = None if row_index is None else _c(row_index, np.int32)
    # preconditions of this reference (the library's handling of bad
    # metadata, clamped offsets and zero rows for indices outside A, is
    # checked against expected values built separately): non-decreasing
    # offsets within the output, and every row read inside A
    if off.size != groups + 1 or off[0] < 0 or np.any(np.diff(off) < 0) or off[-1] > m_total:
        raise ValueError("offsets must be non-decreasing, start at >= 0 and end at <= m_total")
    used = int(off[-1])
    if ri is None:
        if used > aq.shape[0]:
            raise ValueError("without row_index, A must hold offsets[groups] rows")
    elif ri.size < used or (used and (ri[:used].min() < 0 or ri[:used].max() >= aq.shape[0])):
        raise ValueError("row_index must hold offsets[groups] indices inside A")
    y = np.full((m_total, n), np.nan, np.float64)
    bound = np.full((m_total, n), np.nan, np.float64)
    lib().oracle_grouped_gemm(_p(aq), _p(asb), _p(as_), _p(ri), _p(off), groups, _p(bq), _p(bsb),
                              _p(bs), n, k, _p(y), _p(bound))
    return y, bound


def gemm_within_bound(y, y_ref, bound, rel=1e-5):
    """Acceptance: |Y - Y_ref| <= rel * sum_k |a_k b_k|, and Y is +-0 where the
    bound is 0.  Returns a boolean mask of passing entries."""
    y = np.asarray(y, np.float64)
    return np.abs(y - y_ref) <= rel * bound
