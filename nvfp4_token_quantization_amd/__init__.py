"""Per-token NVFP4 quantization and block-scaled W4A4 GEMM on MI355X (gfx950).

Thin Python binding over the C ABI of ``libnvfp4.so`` (declared in
``include/nvfp4.h``).  Every step of the path runs in the library's HIP
kernels; this module only checks tensor metadata, allocates outputs with
torch and passes device pointers plus torch's current stream.  There is no
CPU fallback: if the library is missing or the device is not gfx950 the
calls raise.

Functions keep the C names:

  nvfp4_quantize_rows(x, amax_in=None)            -> (q, sb, s)
  nvfp4_quantize_weight(w, amax_in=None)          -> (q, sb, s, amax)
  nvfp4_gemm(a, b)                                -> y
  nvfp4_grouped_gemm(a, offsets, b, row_index=None, m_total=None) -> y
  nvfp4_grouped_gemm_swiglu(a, offsets, b, row_index=None, m_total=None) -> (h, amax)

(The codec self-test hooks live in the test-only ``selftest`` submodule over
``libnvfp4_selftest.so``.)

Layouts (all row-major): x bf16 [rows, k]; q uint8 [rows, k/2] with element
2i in the low nibble; sb uint8 [rows, k/16] (E4M3 codes); s float32 [rows]
(per-token) or [groups] (weights); a GEMM operand is the tuple (q, sb, s).
"""
import ctypes
import os

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
PRODUCT_LIB_PATH = os.path.join(_HERE, "libnvfp4.so")
# the checked build: the same library with device-side preconditions
# (finite inputs and scales, no NaN scale codes, non-decreasing offsets)
# validated before every call's work; it synchronizes the host on each call
CHECKED_LIB_PATH = os.path.join(_HERE, "libnvfp4_checked.so")
# NVFP4_CHECKED=1 in the environment makes the binding load the checked build
LIB_PATH = CHECKED_LIB_PATH if os.environ.get("NVFP4_CHECKED", "0") not in ("", "0") else PRODUCT_LIB_PATH

SUCCESS = 0
ERROR_PRECONDITION = 6
_lib = None
_loaded = {}


class NVFP4Error(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__("%s failed: %s (status %d)" % (fn, status_string(status), status))


def load(path):
    """Load one build of the library (libnvfp4.so or libnvfp4_checked.so,
    built in-tree by ``__graft_entry__.build()``) with its C signatures."""
    if path in _loaded:
        return _loaded[path]
    if not os.path.exists(path):
        raise RuntimeError("%s is not built: run __graft_entry__.build() "
                           "(or python -m nvfp4_token_quantization_amd.build)" % os.path.basename(path))
    L = ctypes.CDLL(path)
    P, I64 = ctypes.c_void_p, ctypes.c_int64
    L.nvfp4_version.restype = ctypes.c_int
    L.nvfp4_status_string.argtypes = [ctypes.c_int]
    L.nvfp4_status_string.restype = ctypes.c_char_p
    L.nvfp4_quantize_rows.argtypes = [P, I64, I64, P, P, P, P, P]
    L.nvfp4_quantize_weight.argtypes = [P, I64, I64, I64, P, P, P, P, P, P]
    L.nvfp4_gemm.argtypes = [P, P, P, I64, P, P, P, I64, I64, P, P]
    L.nvfp4_grouped_gemm.argtypes = [P, P, P, I64, P, I64, P, I64, P, P, P, I64, I64, P, P]
    L.nvfp4_grouped_gemm_swiglu.argtypes = [P, P, P, I64, P, I64, P, I64, P, P, P, I64, I64,
                                            P, P, P]
    L.nvfp4_swiglu_quantize_rows.argtypes = [P, I64, I64, P, P, P, P, P, P]
    L.nvfp4_moe_route.argtypes = [P, I64, I64, I64, P, P, P, P, P]
    L.nvfp4_dequantize_rows.argtypes = [P, P, P, I64, I64, I64, P, P]
    L.nvfp4_mxfp8_quantize_rows.argtypes = [P, I64, I64, P, P, P]
    L.nvfp4_mxfp8_gemm.argtypes = [P, P, I64, P, P, I64, I64, P, P]
    L.nvfp4_mxfp8_grouped_gemm.argtypes = [P, P, I64, P, I64, P, I64, P, P, I64, I64, P, P]
    for f in ("nvfp4_quantize_rows", "nvfp4_quantize_weight", "nvfp4_gemm",
              "nvfp4_swiglu_quantize_rows", "nvfp4_moe_route", "nvfp4_dequantize_rows",
              "nvfp4_mxfp8_quantize_rows", "nvfp4_mxfp8_gemm", "nvfp4_mxfp8_grouped_gemm",
              "nvfp4_grouped_gemm", "nvfp4_grouped_gemm_swiglu"):
        getattr(L, f).restype = ctypes.c_int
    _loaded[path] = L
    return L


def lib():
    """The library every call goes through: LIB_PATH (the product build
    unless NVFP4_CHECKED is set)."""
    global _lib
    if _lib is None:
        _lib = load(LIB_PATH)
    return _lib


def version():
    return lib().nvfp4_version()


def status_string(status):
    return lib().nvfp4_status_string(int(status)).decode()


def _check(fn, status):
    if status != SUCCESS:
        raise NVFP4Error(fn, status)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _dev(t, name, dtypes, ndim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if not t.is_cuda:
        raise ValueError("%s must be on a GPU (got %s)" % (name, t.device))
    if t.dtype not in dtypes:
        raise TypeError("%s must have dtype in %s (got %s)" % (name, dtypes, t.dtype))
    if ndim is not None and t.dim() != ndim:
        raise ValueError("%s must have %d dims (got %s)" % (name, ndim, tuple(t.shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t


_BF16 = (torch.bfloat16, torch.int16, torch.uint16)


def _out(t, name, shape, dtype, device):
    """Check a caller-supplied output tensor: the kernels write exactly
    `shape` elements of `dtype` through its pointer, so anything else (a
    smaller or strided buffer, another device) is refused."""
    _dev(t, name, (dtype,))
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s (got %s)" % (name, tuple(shape), tuple(t.shape)))
    if t.device != device:
        raise ValueError("%s must be on %s (got %s)" % (name, device, t.device))
    return t


def _out_rows(t, name, min_rows, cols, dtype, device):
    """Output of a grouped GEMM: [rows >= min_rows, cols]; the kernels write
    only rows below offsets[groups] <= min_rows, so a taller buffer is fine."""
    _dev(t, name, (dtype,), 2)
    if t.shape[0] < min_rows or t.shape[1] != cols:
        raise ValueError("%s must have shape (>= %d, %d) (got %s)" % (name, min_rows, cols, tuple(t.shape)))
    if t.device != device:
        raise ValueError("%s must be on %s (got %s)" % (name, device, t.device))
    return t


def _same_device(device, *named):
    for name, t in named:
        if t is not None and t.device != device:
            raise ValueError("%s must be on %s (got %s)" % (name, device, t.device))


def nvfp4_quantize_rows(x, amax_in=None, out=None):
    """Per-token NVFP4 of bf16 rows x [rows, k] (k % 16 == 0).

    amax_in: optional float32 [rows], the producer's row amax (amax reuse).
    out: optional preallocated (q, sb, s).  Returns (q, sb, s).
    """
    _dev(x, "x", _BF16, 2)
    rows, k = x.shape
    dev = x.device
    if out is None:
        q = torch.empty((rows, k // 2), dtype=torch.uint8, device=dev)
        sb = torch.empty((rows, k // 16), dtype=torch.uint8, device=dev)
        s = torch.empty((rows,), dtype=torch.float32, device=dev)
    else:
        q, sb, s = out
        _out(q, "out q", (rows, k // 2), torch.uint8, dev)
        _out(sb, "out sb", (rows, k // 16), torch.uint8, dev)
        _out(s, "out s", (rows,), torch.float32, dev)
    if amax_in is not None:
        _dev(amax_in, "amax_in", (torch.float32,), 1)
        if amax_in.numel() != rows:
            raise ValueError("amax_in must have one entry per row")
        _same_device(dev, ("amax_in", amax_in))
    st = lib().nvfp4_quantize_rows(_ptr(x), rows, k, _ptr(amax_in), _ptr(q), _ptr(sb), _ptr(s),
                                   _stream(dev))
    _check("nvfp4_quantize_rows", st)
    return q, sb, s


def nvfp4_swiglu_quantize_rows(gate_up, want_h=False, want_amax=False, quantize=True, out=None):
    """SwiGLU of a fused fp32 gate|up block [rows, 2f] (gate in columns
    [0, f), up in [f, 2f)) fused with per-token NVFP4 of its bf16 output.

    Returns a dict with the requested outputs: "h" (bf16 [rows, f]), "amax"
    (float32 [rows]) and "q", "sb", "s" when quantize is true.  `out` may hold
    preallocated tensors under the same keys.
    """
    _dev(gate_up, "gate_up", (torch.float32,), 2)
    rows, f2 = gate_up.shape
    if f2 % 2:
        raise ValueError("gate_up must have an even number of columns")
    f = f2 // 2
    dev = gate_up.device
    out = dict(out or {})
    res = {}
    want = []
    if want_h:
        want.append(("h", (rows, f), torch.bfloat16))
    if want_amax:
        want.append(("amax", (rows,), torch.float32))
    if quantize:
        want += [("q", (rows, f // 2), torch.uint8), ("sb", (rows, f // 16), torch.uint8),
                 ("s", (rows,), torch.float32)]
    for key, shape, dt in want:
        t = out.get(key, None)
        res[key] = torch.empty(shape, dtype=dt, device=dev) if t is None else \
            _out(t, "out " + key, shape, dt, dev)
    st = lib().nvfp4_swiglu_quantize_rows(_ptr(gate_up), rows, f, _ptr(res.get("h")),
                                          _ptr(res.get("amax")), _ptr(res.get("q")),
                                          _ptr(res.get("sb")), _ptr(res.get("s")), _stream(dev))
    _check("nvfp4_swiglu_quantize_rows", st)
    return res


def nvfp4_dequantize_rows(q, sb, s, rows_per_scale=1, out=None):
    """bf16 dequantization of NVFP4 rows: q [rows, k/2] (or [groups, rows,
    k/2]), sb matching, s float32 with one entry per rows_per_scale rows.
    Returns bf16 [rows, k] (same leading shape as q)."""
    _dev(q, "q", (torch.uint8,))
    _dev(sb, "sb", (torch.uint8,))
    _dev(s, "s", (torch.float32,))
    k = q.shape[-1] * 2
    rows = q.numel() // max(q.shape[-1], 1) if q.shape[-1] else int(np.prod(q.shape[:-1]))
    if sb.numel() != rows * (k // 16):
        raise ValueError("sb must hold k/16 scale codes per row")
    if s.numel() * rows_per_scale < rows:
        raise ValueError("s must hold one outer scale per rows_per_scale rows")
    _same_device(q.device, ("sb", sb), ("s", s))
    shape = tuple(q.shape[:-1]) + (k,)
    if out is None:
        out = torch.empty(shape, dtype=torch.bfloat16, device=q.device)
    else:
        _out(out, "out", shape, torch.bfloat16, q.device)
    st = lib().nvfp4_dequantize_rows(_ptr(q), _ptr(sb), _ptr(s), rows, k, int(rows_per_scale),
                                     _ptr(out), _stream(q.device))
    _check("nvfp4_dequantize_rows", st)
    return out


def nvfp4_mxfp8_quantize_rows(x, out=None):
    """MXFP8 of bf16 rows x [rows, k] (k % 32 == 0): returns (q uint8 [rows,
    k] E4M3 codes, sc uint8 [rows, k/32] E8M0 codes)."""
    _dev(x, "x", _BF16, 2)
    rows, k = x.shape
    if out is None:
        q = torch.empty((rows, k), dtype=torch.uint8, device=x.device)
        sc = torch.empty((rows, k // 32), dtype=torch.uint8, device=x.device)
    else:
        q, sc = out
        _out(q, "out q", (rows, k), torch.uint8, x.device)
        _out(sc, "out sc", (rows, k // 32), torch.uint8, x.device)
    st = lib().nvfp4_mxfp8_quantize_rows(_ptr(x), rows, k, _ptr(q), _ptr(sc), _stream(x.device))
    _check("nvfp4_mxfp8_quantize_rows", st)
    return q, sc


def nvfp4_mxfp8_gemm(a, b, out=None):
    """Y = deq(A) . deq(B)^T for MXFP8 operands a = (q [m, k], sc [m, k/32]),
    b = (q [n, k], sc [n, k/32]); fp32 [m, n]."""
    aq, asc = _mx_operand(a, "a", 2)
    bq, bsc = _mx_operand(b, "b", 2)
    m, k = aq.shape
    n = bq.shape[0]
    if bq.shape[1] != k:
        raise ValueError("A and B must have the same k")
    _same_device(aq.device, ("b.q", bq))
    y = _out(out, "out", (m, n), torch.float32, aq.device) if out is not None else \
        torch.empty((m, n), dtype=torch.float32, device=aq.device)
    st = lib().nvfp4_mxfp8_gemm(_ptr(aq), _ptr(asc), m, _ptr(bq), _ptr(bsc), n, k, _ptr(y),
                                _stream(aq.device))
    _check("nvfp4_mxfp8_gemm", st)
    return y


def nvfp4_mxfp8_grouped_gemm(a, offsets, b, row_index=None, m_total=None, out=None):
    """Grouped MXFP8 GEMM: a = (q [a_rows, k], sc [a_rows, k/32]); offsets
    int32 [groups+1] on the device; b = (q [groups, n, k], sc [groups, n,
    k/32]); row_index optional int32 [m_total]."""
    aq, asc = _mx_operand(a, "a", 2)
    bq, bsc = _mx_operand(b, "b", 3)
    _dev(offsets, "offsets", (torch.int32,), 1)
    groups, n, k = bq.shape[0], bq.shape[1], bq.shape[2]
    if aq.shape[1] != k:
        raise ValueError("A and B must have the same k")
    if offsets.numel() != groups + 1:
        raise ValueError("offsets must have groups + 1 entries")
    m_total = _grouped_rows(aq.shape[0], row_index, m_total)
    _same_device(aq.device, ("b.q", bq), ("offsets", offsets), ("row_index", row_index))
    y = _out_rows(out, "out", m_total, n, torch.float32, aq.device) if out is not None else \
        torch.empty((m_total, n), dtype=torch.float32, device=aq.device)
    st = lib().nvfp4_mxfp8_grouped_gemm(_ptr(aq), _ptr(asc), aq.shape[0], _ptr(row_index), m_total,
                                        _ptr(offsets), groups, _ptr(bq), _ptr(bsc), n, k, _ptr(y),
                                        _stream(aq.device))
    _check("nvfp4_mxfp8_grouped_gemm", st)
    return y


def nvfp4_moe_route(logits, topk, out=None):
    """Top-k routing of fp32 logits [tokens, experts] into the contiguous
    per-expert layout on the device.  Returns a dict of int32 tensors:
    experts [tokens, topk], offsets [experts+1], row_index [tokens*topk],
    slot_of [tokens, topk]."""
    _dev(logits, "logits", (torch.float32,), 2)
    T, E = logits.shape
    dev = logits.device
    out = dict(out or {})
    i32 = torch.int32
    res = {}
    for key, shape in (("experts", (T, topk)), ("offsets", (E + 1,)), ("row_index", (T * topk,)),
                       ("slot_of", (T, topk))):
        t = out.get(key, None)
        res[key] = torch.empty(shape, dtype=i32, device=dev) if t is None else \
            _out(t, "out " + key, shape, i32, dev)
    st = lib().nvfp4_moe_route(_ptr(logits), T, E, int(topk), _ptr(res["experts"]),
                               _ptr(res["offsets"]), _ptr(res["row_index"]), _ptr(res["slot_of"]),
                               _stream(dev))
    _check("nvfp4_moe_route", st)
    return res


def nvfp4_quantize_weight(w, amax_in=None, out=None):
    """Per-tensor (groups == 1) or per-expert NVFP4 of bf16 w [groups, rows, k].

    Returns (q [groups, rows, k/2], sb [groups, rows, k/16], s [groups],
    amax [groups]).
    """
    _dev(w, "w", _BF16, 3)
    g, r, k = w.shape
    dev = w.device
    if out is None:
        q = torch.empty((g, r, k // 2), dtype=torch.uint8, device=dev)
        sb = torch.empty((g, r, k // 16), dtype=torch.uint8, device=dev)
        s = torch.empty((g,), dtype=torch.float32, device=dev)
        amax = torch.empty((g,), dtype=torch.float32, device=dev)
    else:
        q, sb, s, amax = out
        _out(q, "out q", (g, r, k // 2), torch.uint8, dev)
        _out(sb, "out sb", (g, r, k // 16), torch.uint8, dev)
        _out(s, "out s", (g,), torch.float32, dev)
        _out(amax, "out amax", (g,), torch.float32, dev)
    if amax_in is not None:
        _dev(amax_in, "amax_in", (torch.float32,), 1)
        if amax_in.numel() != g:
            raise ValueError("amax_in must have one entry per group")
        _same_device(dev, ("amax_in", amax_in))
    st = lib().nvfp4_quantize_weight(_ptr(w), g, r, k, _ptr(amax_in), _ptr(amax), _ptr(q),
                                     _ptr(sb), _ptr(s), _stream(dev))
    _check("nvfp4_quantize_weight", st)
    return q, sb, s, amax


def _operand(t, name, ndim, scales):
    """Check an NVFP4 operand (q, sb, s): q [..., k/2] and sb [..., k/16]
    with the same leading shape (ndim dims), s with `scales` entries, all on
    one device."""
    q, sb, s = t
    _dev(q, name + ".q", (torch.uint8,), ndim)
    _dev(sb, name + ".sb", (torch.uint8,), ndim)
    _dev(s, name + ".s", (torch.float32,))
    if tuple(sb.shape[:-1]) != tuple(q.shape[:-1]) or sb.shape[-1] * 8 != q.shape[-1]:
        raise ValueError("%s.sb must be %s + [k/16] for %s.q of shape %s (got %s)" % (
            name, tuple(q.shape[:-1]), name, tuple(q.shape), tuple(sb.shape)))
    if s.numel() != scales:
        raise ValueError("%s.s must have %d entries (got %d)" % (name, scales, s.numel()))
    _same_device(q.device, (name + ".sb", sb), (name + ".s", s))
    return q, sb, s


def _mx_operand(t, name, ndim):
    """Check an MXFP8 operand (q [..., k], sc [..., k/32])."""
    q, sc = t
    _dev(q, name + ".q", (torch.uint8,), ndim)
    _dev(sc, name + ".sc", (torch.uint8,), ndim)
    if tuple(sc.shape[:-1]) != tuple(q.shape[:-1]) or sc.shape[-1] * 32 != q.shape[-1]:
        raise ValueError("%s.sc must be %s + [k/32] for %s.q of shape %s (got %s)" % (
            name, tuple(q.shape[:-1]), name, tuple(q.shape), tuple(sc.shape)))
    _same_device(q.device, (name + ".sc", sc))
    return q, sc


def _grouped_rows(a_rows, row_index, m_total):
    """Output rows of a grouped GEMM: m_total, else len(row_index), else
    a_rows; checks row_index covers them (or, without it, that A does)."""
    if row_index is not None:
        _dev(row_index, "row_index", (torch.int32,), 1)
        if m_total is None:
            m_total = row_index.numel()
        elif row_index.numel() < m_total:
            raise ValueError("row_index must have m_total entries")
    elif m_total is None:
        m_total = a_rows
    elif m_total > a_rows:
        raise ValueError("without row_index, A must have at least m_total rows")
    return int(m_total)


def nvfp4_gemm(a, b, out=None):
    """Y = deq(A) . deq(B)^T, fp32 [m, n].  a = (q [m, k/2], sb [m, k/16],
    s [m]); b = (q [n, k/2], sb [n, k/16], s [1])."""
    aq = a[0]
    m = aq.shape[0]
    aq, asb, as_ = _operand(a, "a", 2, m)
    bq = b[0]
    if bq.dim() == 3 and bq.shape[0] == 1:  # a per-tensor weight from nvfp4_quantize_weight
        b = (bq[0], b[1][0] if b[1].dim() == 3 else b[1], b[2])
    bq, bsb, bs = _operand(b, "b", 2, 1)
    n = bq.shape[0]
    k = aq.shape[-1] * 2
    if bq.shape[-1] * 2 != k:
        raise ValueError("A and B must have the same k")
    dev = aq.device
    _same_device(dev, ("b.q", bq))
    y = torch.empty((m, n), dtype=torch.float32, device=dev) if out is None else \
        _out(out, "out", (m, n), torch.float32, dev)
    st = lib().nvfp4_gemm(_ptr(aq), _ptr(asb), _ptr(as_), m, _ptr(bq), _ptr(bsb), _ptr(bs), n, k,
                          _ptr(y), _stream(dev))
    _check("nvfp4_gemm", st)
    return y


def nvfp4_grouped_gemm(a, offsets, b, row_index=None, m_total=None, out=None):
    """Grouped GEMM over a contiguous per-expert layout.

    a = (q [a_rows, k/2], sb [a_rows, k/16], s [a_rows]);
    offsets int32 [groups+1] (device); b = (q [groups, n, k/2],
    sb [groups, n, k/16], s [groups]); row_index optional int32 [m_total].
    m_total defaults to len(row_index) or a_rows (the host never reads
    offsets).  Rows at or past offsets[groups] of the output are not written.
    """
    aq, asb, as_ = _operand(a, "a", 2, a[0].shape[0] if a[0].dim() == 2 else -1)
    if b[0].dim() != 3:
        raise ValueError("b.q must be [groups, n, k/2]")
    bq, bsb, bs = _operand(b, "b", 3, b[0].shape[0])
    _dev(offsets, "offsets", (torch.int32,), 1)
    groups, n, k = bq.shape[0], bq.shape[1], bq.shape[2] * 2
    if aq.shape[1] * 2 != k:
        raise ValueError("A and B must have the same k")
    if offsets.numel() != groups + 1:
        raise ValueError("offsets must have groups + 1 entries")
    a_rows = aq.shape[0]
    m_total = _grouped_rows(a_rows, row_index, m_total)
    dev = aq.device
    _same_device(dev, ("b.q", bq), ("offsets", offsets), ("row_index", row_index))
    y = torch.empty((m_total, n), dtype=torch.float32, device=dev) if out is None else \
        _out_rows(out, "out", m_total, n, torch.float32, dev)
    st = lib().nvfp4_grouped_gemm(_ptr(aq), _ptr(asb), _ptr(as_), a_rows, _ptr(row_index),
                                  m_total, _ptr(offsets), groups, _ptr(bq), _ptr(bsb), _ptr(bs),
                                  n, k, _ptr(y), _stream(dev))
    _check("nvfp4_grouped_gemm", st)
    return y


def nvfp4_grouped_gemm_swiglu(a, offsets, b, row_index=None, m_total=None, out=None):
    """Grouped up-projection with SwiGLU in the epilogue.

    a, offsets, row_index, m_total as nvfp4_grouped_gemm; b = the fused
    gate|up weight (q [groups, 2f, k/2], sb [groups, 2f, k/16], s [groups]),
    gate rows first.  Returns (h bf16 [m_total, f], amax float32 [m_total]):
    H = silu(gate) * up of the GEMM output and its row amax (the amax_in of
    the requantize).  out: optional preallocated (h, amax).  k must be a
    positive multiple of 256.
    """
    aq, asb, as_ = _operand(a, "a", 2, a[0].shape[0] if a[0].dim() == 2 else -1)
    if b[0].dim() != 3:
        raise ValueError("b.q must be [groups, 2f, k/2]")
    bq, bsb, bs = _operand(b, "b", 3, b[0].shape[0])
    _dev(offsets, "offsets", (torch.int32,), 1)
    groups, n2, k = bq.shape[0], bq.shape[1], bq.shape[2] * 2
    if n2 % 2:
        raise ValueError("b must have an even number of rows per expert (gate, then up)")
    f = n2 // 2
    if aq.shape[1] * 2 != k:
        raise ValueError("A and B must have the same k")
    if offsets.numel() != groups + 1:
        raise ValueError("offsets must have groups + 1 entries")
    a_rows = aq.shape[0]
    m_total = _grouped_rows(a_rows, row_index, m_total)
    dev = aq.device
    _same_device(dev, ("b.q", bq), ("offsets", offsets), ("row_index", row_index))
    if out is None:
        h = torch.empty((m_total, f), dtype=torch.bfloat16, device=dev)
        amax = torch.empty((m_total,), dtype=torch.float32, device=dev)
    else:
        h = _out_rows(out[0], "out.h", m_total, f, torch.bfloat16, dev)
        amax = out[1]
        _dev(amax, "out.amax", (torch.float32,), 1)
        if amax.numel() < m_total or amax.device != dev:
            raise ValueError("out.amax must have at least m_total entries on %s" % dev)
    st = lib().nvfp4_grouped_gemm_swiglu(_ptr(aq), _ptr(asb), _ptr(as_), a_rows, _ptr(row_index),
                                         m_total, _ptr(offsets), groups, _ptr(bq), _ptr(bsb),
                                         _ptr(bs), f, k, _ptr(h), _ptr(amax), _stream(dev))
    _check("nvfp4_grouped_gemm_swiglu", st)
    return h, amax
