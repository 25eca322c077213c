"""GPU edge cases of the block-scaled GEMMs, each against the oracle:

- the largest expert count the ABI accepts (1024 groups), NVFP4 and MXFP8:
  the per-expert tile prefix then needs its entry 1024 (the total);
- expert counts on both sides of the schedule's 64-expert scan segments and
  of its 256-expert switch from registers to LDS (1 to 513 experts), in
  the few-rows and the tiled kernels;
- an output whose address has bit 31 of its low 32-bit word set, through
  every branch of the LDS kernel's epilogue (n % 4 == 0 through LDS, whole
  tiles, per element): the epilogue's buffer resource takes the tile's base
  address from two 32-bit halves, so the low half must be zero-extended;
  the bytes around the output must stay untouched;
- long contractions (K = 8192 and 16384) with every product of one sign, the
  case where fp32 accumulation error relative to sum |a b| is largest;
- the binding's argument checks (wrong output shapes, mismatched operands):
  they raise before anything is launched.
"""
import numpy as np
import pytest
import torch

import nvfp4_token_quantization_amd as nv
import oracle
import synthgen as sg
from gpu_helpers import check_gemm, dev, to_dev, to_np

pytestmark = pytest.mark.gpu


def dev_op(t):
    return tuple(to_dev(np.ascontiguousarray(v)) for v in t)


# ------------------------------------------------------------ 1024 groups --
def _counts_1024(seed):
    # mostly empty or tiny experts, a few with several tiles, and the last
    # expert non-empty so the final prefix entry matters
    u = sg.uniform(seed, 1, 1024)
    counts = np.where(u < 0.55, 0, np.where(u < 0.9, 1 + (u * 97).astype(np.int64) % 4,
                                              (u * 1000).astype(np.int64) % 300))
    counts[-1] = 37
    counts[512] = 129
    return counts.astype(np.int64)


def test_grouped_1024_groups():
    counts = _counts_1024(501)
    groups, n, k, tokens = 1024, 64, 256, 333
    x = sg.student_t3_bf16(502, 1, (tokens, k))
    a = oracle.quantize_rows(x)
    w = sg.normal_bf16(503, 2, (groups, n, k), 0.0, 0.02)
    b = oracle.quantize_weight(w)[:3]
    offsets = np.zeros(groups + 1, np.int32)
    offsets[1:] = np.cumsum(counts)
    m_total = int(offsets[-1])
    ri = ((np.arange(m_total) * 7919) % tokens).astype(np.int32)
    y = torch.full((m_total + 5, n), float("nan"), device=dev())
    nv.nvfp4_grouped_gemm(dev_op(a), to_dev(offsets), dev_op(b), row_index=to_dev(ri),
                          m_total=m_total, out=y)
    y = to_np(y)
    y_ref, bound = oracle.grouped_gemm(a, offsets, b, row_index=ri)
    check_gemm(y[:m_total], y_ref, bound, "1024 groups, %d rows" % m_total)
    assert np.all(np.isnan(y[m_total:])), "rows past offsets[groups] must not be written"


def test_grouped_1024_groups_tiled_kernel():
    """The same expert pattern with every count times 4 (more than 16 rows per
    expert on average): the tiled kernel's schedule, whose expert prefix
    reads the offsets in 64-expert segments, over all 1024 experts."""
    counts = 4 * _counts_1024(504)
    groups, n, k, tokens = 1024, 64, 256, 501
    assert counts.sum() > 16 * groups
    x = sg.student_t3_bf16(505, 1, (tokens, k))
    a = oracle.quantize_rows(x)
    w = sg.normal_bf16(506, 2, (groups, n, k), 0.0, 0.02)
    b = oracle.quantize_weight(w)[:3]
    offsets = np.zeros(groups + 1, np.int32)
    offsets[1:] = np.cumsum(counts)
    m_total = int(offsets[-1])
    ri = ((np.arange(m_total) * 7919) % tokens).astype(np.int32)
    y = to_np(nv.nvfp4_grouped_gemm(dev_op(a), to_dev(offsets), dev_op(b), row_index=to_dev(ri)))
    y_ref, bound = oracle.grouped_gemm(a, offsets, b, row_index=ri)
    check_gemm(y, y_ref, bound, "1024 groups, tiled, %d rows" % m_total)


def _counts_any(seed, groups, scale):
    # empty, tiny and a few larger experts; the last expert non-empty, the
    # middle one over one 128-row tile (one expert: 9 or 72 rows)
    if groups == 1:
        return np.array([9 * scale], np.int64)
    u = sg.uniform(seed, 1, groups)
    counts = np.where(u < 0.5, 0, np.where(u < 0.9, 1 + (u * 97).astype(np.int64) % 4,
                                             (u * 1000).astype(np.int64) % 80))
    counts = counts * scale
    counts[-1] = 37
    counts[groups // 2] = 129
    return counts.astype(np.int64)


@pytest.mark.parametrize("groups", [1, 63, 64, 65, 255, 256, 257, 300, 513])
@pytest.mark.parametrize("scale", [1, 8])
def test_grouped_expert_counts_across_scan_segments(groups, scale):
    """scale 1: few rows per expert (the few-rows kernel, whose workgroups scan
    the offsets into LDS); scale 8: more than 16 rows per expert on average
    (the tiled kernel: the expert prefix in registers up to 256 experts, in
    LDS above).  Segment boundaries at 64, 256 and the partial last segment
    of the second round at 300 and 513."""
    counts = _counts_any(520 + groups, groups, scale)
    n, k, tokens = 64, 256, 211
    if scale > 1:
        assert counts.sum() > 16 * groups
    else:
        assert counts.sum() <= 16 * groups
    x = sg.student_t3_bf16(521, 1, (tokens, k))
    a = oracle.quantize_rows(x)
    w = sg.normal_bf16(522 + groups, 2, (groups, n, k), 0.0, 0.02)
    b = oracle.quantize_weight(w)[:3]
    offsets = np.zeros(groups + 1, np.int32)
    offsets[1:] = np.cumsum(counts)
    m_total = int(offsets[-1])
    ri = ((np.arange(m_total) * 7919) % tokens).astype(np.int32)
    y = torch.full((m_total + 3, n), float("nan"), device=dev())
    nv.nvfp4_grouped_gemm(dev_op(a), to_dev(offsets), dev_op(b), row_index=to_dev(ri),
                          m_total=m_total, out=y)
    y = to_np(y)
    y_ref, bound = oracle.grouped_gemm(a, offsets, b, row_index=ri)
    check_gemm(y[:m_total], y_ref, bound, "%d groups x%d, %d rows" % (groups, scale, m_total))
    assert np.all(np.isnan(y[m_total:])), "rows past offsets[groups] must not be written"


def test_mxfp8_grouped_1024_groups():
    from test_gpu_mxfp8 import check_mx_gemm, grouped_reference
    counts = _counts_1024(511)
    groups, n, k, tokens = 1024, 64, 128, 257
    aq, asc = oracle.mxfp8_quantize_rows(sg.student_t3_bf16(512, sg.S_X, (tokens, k)))
    wq, wsc = oracle.mxfp8_quantize_rows(sg.normal_bf16(513, sg.S_W, (groups * n, k), 0.0, 0.02))
    wq, wsc = wq.reshape(groups, n, k), wsc.reshape(groups, n, k // 32)
    offsets = np.zeros(groups + 1, np.int32)
    offsets[1:] = np.cumsum(counts)
    m_total = int(offsets[-1])
    ri = ((np.arange(m_total) * 7919) % tokens).astype(np.int32)
    y = torch.full((m_total + 5, n), float("nan"), device=dev())
    nv.nvfp4_mxfp8_grouped_gemm((to_dev(aq), to_dev(asc)), to_dev(offsets), (to_dev(wq), to_dev(wsc)),
                                row_index=to_dev(ri), m_total=m_total, out=y)
    y = to_np(y)
    y_ref, bound = grouped_reference(aq, asc, {"offsets": offsets, "row_index": ri}, wq, wsc)
    check_mx_gemm(y[:m_total], y_ref, bound, "MXFP8, 1024 groups")
    assert np.all(np.isnan(y[m_total:]))


@pytest.mark.parametrize("groups", [65, 257, 300])
def test_mxfp8_grouped_expert_counts_across_scan_segments(groups):
    from test_gpu_mxfp8 import check_mx_gemm, grouped_reference
    counts = _counts_any(530 + groups, groups, 8)
    n, k, tokens = 64, 128, 199
    aq, asc = oracle.mxfp8_quantize_rows(sg.student_t3_bf16(531, sg.S_X, (tokens, k)))
    wq, wsc = oracle.mxfp8_quantize_rows(sg.normal_bf16(532 + groups, sg.S_W, (groups * n, k), 0.0, 0.02))
    wq, wsc = wq.reshape(groups, n, k), wsc.reshape(groups, n, k // 32)
    offsets = np.zeros(groups + 1, np.int32)
    offsets[1:] = np.cumsum(counts)
    m_total = int(offsets[-1])
    ri = ((np.arange(m_total) * 7919) % tokens).astype(np.int32)
    y = to_np(nv.nvfp4_mxfp8_grouped_gemm((to_dev(aq), to_dev(asc)), to_dev(offsets),
                                          (to_dev(wq), to_dev(wsc)), row_index=to_dev(ri)))
    y_ref, bound = grouped_reference(aq, asc, {"offsets": offsets, "row_index": ri}, wq, wsc)
    check_mx_gemm(y, y_ref, bound, "MXFP8, %d groups" % groups)


# -------------------------------------------- output address, bit 31 set --
_BIG = None


def _bit31_view(rows, cols):
    """A [rows, cols] fp32 view into a larger buffer whose address has bit 31
    of its low 32-bit word set (16-byte aligned), with a guard band of NaN
    before and after it.  Returns (view, region, guard): region is the view
    plus `guard` elements on each side."""
    global _BIG
    guard = 4096
    need = rows * cols + 2 * guard
    # 4 GiB plus 2 MiB plus the view: some offset below 2^32 + 2^21 bytes puts
    # the view's low address word at 2^31 + 2^20 or 2^31 + 2^21
    size = (1 << 30) + (1 << 19) + need
    if _BIG is None or _BIG.numel() < size:
        _BIG = None
        torch.cuda.empty_cache()
        _BIG = torch.empty((size,), dtype=torch.float32, device=dev())
    base = _BIG.data_ptr()
    off_bytes = ((1 << 31) + (1 << 20) - (base & 0xFFFFFFFF)) % (1 << 32)
    if off_bytes < 4 * guard:
        off_bytes += 1 << 20
    assert off_bytes % 16 == 0
    off = off_bytes // 4
    assert off - guard >= 0 and off + rows * cols + guard <= _BIG.numel()
    region = _BIG[off - guard: off + rows * cols + guard]
    region.fill_(float("nan"))
    v = _BIG[off: off + rows * cols].view(rows, cols)
    addr = v.data_ptr()
    assert addr & 0x80000000 and addr % 16 == 0
    return v, region, guard


def _check_sampled(y, a, b, seed, what):
    """Compare seeded entries of y plus its first and last rows and columns
    (tile borders included) with the oracle."""
    m, n = y.shape
    cnt = 100000
    ii = np.concatenate([(sg.uniform(seed, 1, cnt) * m).astype(np.int64),
                         np.repeat([0, 127, 128, m - 1], n), np.tile(np.arange(m), 4)])
    jj = np.concatenate([(sg.uniform(seed, 2, cnt) * n).astype(np.int64),
                         np.tile(np.arange(n), 4), np.repeat([0, 127, 128, n - 1], m)])
    y_ref, bound = oracle.gemm_entries(a, b, ii, jj, np.zeros_like(ii))
    check_gemm(y[ii, jj], y_ref, bound, what)


# Small problems issue every tile as a 64-row half tile (their last round is
# their only round), which takes the per-element stores when n % 4 != 0; a
# region needs more than half an XCD's worth of 128 x 128 tiles (2048 x 4098:
# 528 tiles, about 66 per XCD) for whole tiles.
@pytest.mark.parametrize("m,n,k", [
    (200, 384, 512),    # n % 4 == 0: values transposed through LDS, 16-byte stores
    (2048, 4098, 256),  # n % 4 != 0: whole 128 x 128 tiles, scalar-offset stores
    (200, 131, 768),    # n % 4 != 0, half and ragged tiles: per-element stores
])
def test_output_address_with_bit31_set(m, n, k):
    a = oracle.quantize_rows(sg.student_t3_bf16(600 + n, 1, (m, k)))
    b = oracle.quantize_weight(sg.normal_bf16(601 + n, 2, (1, n, k), 0.0, 0.02))
    b2 = (b[0][0], b[1][0], b[2])
    y, region, guard = _bit31_view(m, n)
    nv.nvfp4_gemm(dev_op(a), dev_op(b2), out=y)
    torch.cuda.synchronize()
    what = "dense %dx%dx%d at a high output address" % (m, n, k)
    if m * n <= 1 << 18:
        y_ref, bound = oracle.gemm(a, b2)
        check_gemm(to_np(y), y_ref, bound, what)
    else:
        _check_sampled(to_np(y), a, b2, 603 + n, what)
    r = to_np(region)
    assert np.all(np.isnan(r[:guard])) and np.all(np.isnan(r[-guard:])), \
        "bytes around the output were written"
    # grouped: two experts over the same rows
    offsets = np.array([0, m // 3, m], np.int32)
    bg = oracle.quantize_weight(sg.normal_bf16(602 + n, 2, (2, n, k), 0.0, 0.02))[:3]
    y, region, guard = _bit31_view(m, n)
    nv.nvfp4_grouped_gemm(dev_op(a), to_dev(offsets), dev_op(bg), out=y)
    torch.cuda.synchronize()
    what = "grouped %dx%dx%d at a high output address" % (m, n, k)
    if m * n <= 1 << 18:
        y_ref, bound = oracle.grouped_gemm(a, offsets, bg)
        check_gemm(to_np(y), y_ref, bound, what)
    else:
        yn = to_np(y)
        for g in range(2):
            lo, hi = int(offsets[g]), int(offsets[g + 1])
            a_g = tuple(v[lo:hi] for v in a)
            _check_sampled(yn[lo:hi], a_g, (bg[0][g], bg[1][g], bg[2][g:g + 1]), 604 + g, what)
    r = to_np(region)
    assert np.all(np.isnan(r[:guard])) and np.all(np.isnan(r[-guard:]))


def test_release_big_buffer():
    global _BIG
    _BIG = None
    torch.cuda.empty_cache()


# ------------------------------------------------------ long contractions --
def _same_sign_operands(seed, m, n, k, groups=1):
    """Every element non-negative, so every product a_k b_k >= 0 and
    |sum a b| = sum |a b|: fp32 rounding errors of the accumulation all count
    against the bound, with no cancellation to hide them."""
    # clearing the bf16 sign bit gives |x|
    x = sg.student_t3_bf16(seed, 1, (m, k)).view(np.uint16) & np.uint16(0x7FFF)
    w = sg.normal_bf16(seed, 2, (groups, n, k), 0.0, 0.02).view(np.uint16) & np.uint16(0x7FFF)
    return oracle.quantize_rows(x), oracle.quantize_weight(w)[:3]


@pytest.mark.parametrize("k", [8192, 16384])
def test_dense_long_k_same_sign(k):
    m, n = 160, 200
    a, b = _same_sign_operands(700 + k // 1024, m, n, k)
    y = nv.nvfp4_gemm(dev_op(a), (to_dev(b[0][0]), to_dev(b[1][0]), to_dev(b[2])))
    y_ref, bound = oracle.gemm(a, (b[0][0], b[1][0], b[2]))
    y = to_np(y)
    check_gemm(y, y_ref, bound, "dense k=%d, same-sign operands" % k)
    rel = np.max(np.abs(y - y_ref) / bound)
    print("dense k=%d: max |dY| / sum|ab| = %.3g" % (k, rel))


@pytest.mark.parametrize("k", [8192, 16384])
def test_grouped_long_k_same_sign(k):
    counts = [70, 0, 130, 33]
    n, tokens = 96, 150
    a, b = _same_sign_operands(710 + k // 1024, tokens, n, k, groups=len(counts))
    offsets = np.zeros(len(counts) + 1, np.int32)
    offsets[1:] = np.cumsum(counts)
    ri = ((np.arange(int(offsets[-1])) * 31) % tokens).astype(np.int32)
    y = to_np(nv.nvfp4_grouped_gemm(dev_op(a), to_dev(offsets), dev_op(b), row_index=to_dev(ri)))
    y_ref, bound = oracle.grouped_gemm(a, offsets, b, row_index=ri)
    check_gemm(y, y_ref, bound, "grouped k=%d, same-sign operands" % k)


# ------------------------------------------------------- binding checks --
def test_binding_rejects_bad_outputs_and_operands():
    d = dev()
    x = torch.zeros((8, 64), dtype=torch.bfloat16, device=d)
    u8, f32 = torch.uint8, torch.float32
    good = (torch.empty((8, 32), dtype=u8, device=d), torch.empty((8, 4), dtype=u8, device=d),
            torch.empty((8,), dtype=f32, device=d))
    nv.nvfp4_quantize_rows(x, out=good)
    for bad in ((torch.empty((7, 32), dtype=u8, device=d), good[1], good[2]),
                (good[0], torch.empty((8, 3), dtype=u8, device=d), good[2]),
                (good[0], good[1], torch.empty((4,), dtype=f32, device=d)),
                (torch.empty((8, 64), dtype=u8, device=d)[:, ::2], good[1], good[2])):
        with pytest.raises(ValueError):
            nv.nvfp4_quantize_rows(x, out=bad)
    with pytest.raises(TypeError):
        nv.nvfp4_quantize_rows(x, out=(good[0].to(torch.int8), good[1], good[2]))
    a = nv.nvfp4_quantize_rows(x)
    w = nv.nvfp4_quantize_weight(torch.zeros((1, 16, 64), dtype=torch.bfloat16, device=d))
    b = (w[0][0], w[1][0], w[2])
    nv.nvfp4_gemm(a, b)
    with pytest.raises(ValueError):
        nv.nvfp4_gemm(a, b, out=torch.empty((8, 15), dtype=f32, device=d))
    with pytest.raises(ValueError):   # block scales of another k
        nv.nvfp4_gemm((a[0], a[1][:, :2].contiguous(), a[2]), b)
    with pytest.raises(ValueError):   # one outer scale short
        nv.nvfp4_gemm((a[0], a[1], a[2][:7]), b)
    with pytest.raises(ValueError):   # k differs
        nv.nvfp4_gemm(a, (b[0][:, :16].contiguous(), b[1][:, :2].contiguous(), b[2]))
    off = torch.tensor([0, 8], dtype=torch.int32, device=d)
    nv.nvfp4_grouped_gemm(a, off, w[:3])
    with pytest.raises(ValueError):
        nv.nvfp4_grouped_gemm(a, off, w[:3], out=torch.empty((7, 16), dtype=f32, device=d))
    with pytest.raises(ValueError):   # per-expert scales of another group count
        nv.nvfp4_grouped_gemm(a, off, (w[0], w[1], torch.ones(2, device=d)))
    with pytest.raises(ValueError):   # without row_index A must cover m_total
        nv.nvfp4_grouped_gemm(a, off, w[:3], m_total=9)
    with pytest.raises(ValueError):
        nv.nvfp4_moe_route(torch.zeros((4, 8), device=d), 2,
                           out={"offsets": torch.empty(8, dtype=torch.int32, device=d)})
