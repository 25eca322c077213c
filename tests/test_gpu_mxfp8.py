"""GPU parity of MXFP8 (Miles page, section MXFP8格式背景: 32 E4M3 values per
E8M0 power-of-two scale, the scale rounded up so the block maximum is not
clipped) against the oracle: E4M3 codes and E8M0 codes bit-exact."""
import numpy as np
import pytest
import torch

import nvfp4_token_quantization_amd as nv
import nvfp4_token_quantization_amd.selftest as st
import oracle
import synthgen as sg
from gpu_helpers import dev, to_dev, to_np, workload
from test_gpu_quantize import _sweep

pytestmark = pytest.mark.gpu


def check_quant(x, what):
    q, sc = nv.nvfp4_mxfp8_quantize_rows(to_dev(x))
    torch.cuda.synchronize()
    wq, wsc = oracle.mxfp8_quantize_rows(x)
    for name, g, w in (("sc", to_np(sc), wsc), ("q", to_np(q), wq)):
        if not np.array_equal(g, w):
            bad = np.argwhere(g != w)
            i = tuple(bad[0])
            raise AssertionError("%s %s: %d mismatches, first at %s (got %#x want %#x)" % (
                what, name, len(bad), i, g[i], w[i]))


def test_fp8_convert_exhaustive():
    """Every fp32 pattern in [0, 448] through the pack-convert: non-decreasing,
    at most 0x7E, equal to the oracle at 0, at every E4M3 value and on both
    sides of every rounding boundary; negative inputs give the sign bit."""
    END = 0x43E00001  # through 448.0
    last = -1
    for a, codes in _sweep(st.nvfp4_debug_encode_fp8, 0, END):
        c = codes.to(torch.int16)
        assert int(c.max()) <= 0x7E
        assert bool(torch.all(c[1:] >= c[:-1])), "not monotone in chunk at %#x" % a
        assert int(c[0]) >= last
        last = int(c[-1])
        neg = st.nvfp4_debug_encode_fp8(
            (torch.arange(a, a + c.numel(), dtype=torch.int64, device=dev()) | 0x80000000)
            .to(torch.int32).view(torch.float32))
        assert bool(torch.all(neg.to(torch.int16) == (c | 0x80))), "sign handling at %#x" % a
    tab = oracle.e4m3_table()[:0x7F]
    pts = [0.0, np.float32(1e-45)]
    for m in (tab[:-1] + tab[1:]) / 2:
        f = np.float32(m)
        pts += [f, np.nextafter(f, np.float32(0)), np.nextafter(f, np.float32(np.inf))]
    pts += list(tab.astype(np.float32))
    v = np.array(pts, np.float32)
    got = to_np(st.nvfp4_debug_encode_fp8(to_dev(v)))
    assert np.array_equal(got, oracle.rne_sat_e4m3(v))


@pytest.mark.parametrize("rows,k", [(1, 32), (5, 96), (64, 2048), (300, 768), (17, 4128)])
def test_mxfp8_quantize_random(rows, k):
    x = sg.normal_outliers_bf16(900 + rows, sg.S_X, (rows, k), 1.0, 0.01, 80.0)
    check_quant(x, "rows=%d k=%d" % (rows, k))


def test_mxfp8_quantize_edges():
    """Zero blocks, bf16 maximum, subnormal blocks, -0, and amaxes on both
    sides of the scale's rounding point (mantissa 1.75 keeps e = E - 8, the
    next bf16 needs e = E - 7)."""
    rows, k = 12, 256
    x = sg.student_t3_bf16(31, sg.S_X, (rows, k))
    x[0] = 0
    x[1, :32] = 0x7F7F
    x[1, 32:64] = 0xFF7F
    x[2, :32] = 0x0001
    x[2, 32:64] = 0x807F
    x[3, :32] = 0x8000
    for r, e in zip(range(4, 12), (-130, -126, -20, -1, 0, 7, 60, 127)):
        for b, mant in enumerate((0x60, 0x61, 0x5F, 0x7F, 0x00, 0x01, 0x40, 0x3F)):
            ef = max(e + 127, 1)
            x[r, 32 * b] = np.uint16((ef << 7) | mant)
    check_quant(x, "edges")


def test_mxfp8_quantize_full_dense_activation_and_weight():
    x = workload(2, "x")["x"]
    check_quant(x, "X 4096x2560")
    w = workload(2, "w")["w"][0]
    check_quant(w, "W 9728x2560")


def test_mxfp8_quantize_errors_and_empty():
    d = dev()
    with pytest.raises(nv.NVFP4Error):
        nv.nvfp4_mxfp8_quantize_rows(torch.zeros((2, 48), dtype=torch.bfloat16, device=d))
    q, sc = nv.nvfp4_mxfp8_quantize_rows(torch.zeros((0, 64), dtype=torch.bfloat16, device=d))
    assert q.shape == (0, 64) and sc.shape == (0, 2)


# ----------------------------------------------------------------- GEMM --
# Tolerance: the GEMM decodes every element exactly to bf16 (an E4M3 value
# times its block's power of two; every block scale here is a bf16-normal
# one) and the products are exact in its fp32 accumulator, so the only error
# is the fp32 summation, at most (k/16 + 1) 2^-24 sum |a b| < 1e-5 sum |a b|
# for the k <= 2560 used here.  (gfx950's scaled fp8 MFMA, which sums a
# 32-block's products in a truncating fixed-point window, misses this bound
# by an order of magnitude on these inputs.)
MX_TOL = 1e-5


def check_mx_gemm(y, y_ref, bound, what):
    y = to_np(y) if isinstance(y, torch.Tensor) else y
    ok = np.abs(y - y_ref) <= MX_TOL * bound
    if not ok.all():
        bad = np.argwhere(~ok)
        i = tuple(bad[0])
        raise AssertionError("%s: %d of %d entries outside 1e-5*sum|ab|; first %s got %r want %r" % (
            what, len(bad), ok.size, i, y[i], y_ref[i]))
    assert np.all(y[bound == 0] == 0), what


def mx_dev(op):
    return to_dev(op[0]), to_dev(op[1])


@pytest.mark.parametrize("m,n,k", [(1, 1, 32), (37, 50, 64), (128, 128, 256), (200, 300, 2048),
                                   (64, 96, 96), (130, 33, 160), (5, 700, 512)])
def test_mxfp8_gemm_dense(m, n, k):
    a = oracle.mxfp8_quantize_rows(sg.student_t3_bf16(m + 3 * k, sg.S_X, (m, k)))
    b = oracle.mxfp8_quantize_rows(sg.normal_bf16(n + 5 * k, sg.S_W, (n, k), 0.0, 0.02))
    y = nv.nvfp4_mxfp8_gemm(mx_dev(a), mx_dev(b))
    torch.cuda.synchronize()
    y_ref, bound = oracle.mxfp8_gemm(a, b)
    check_mx_gemm(y, y_ref, bound, "m=%d n=%d k=%d" % (m, n, k))


def test_mxfp8_gemm_dense_full_size_sampled():
    """The dense layer shape (4096 x 2560 -> 9728) quantized and multiplied on
    the GPU; 64 rows x 256 columns recomputed by the oracle from the bf16
    inputs."""
    x = workload(2, "x")["x"]
    w = workload(2, "w")["w"][0]
    aq = nv.nvfp4_mxfp8_quantize_rows(to_dev(x))
    bq = nv.nvfp4_mxfp8_quantize_rows(to_dev(w))
    y = to_np(nv.nvfp4_mxfp8_gemm(aq, bq))
    rows = (np.arange(64) * 61 + 7) % x.shape[0]
    cols = (np.arange(256) * 37 + 3) % w.shape[0]
    y_ref, bound = oracle.mxfp8_gemm(oracle.mxfp8_quantize_rows(x[rows]),
                                     oracle.mxfp8_quantize_rows(w[cols]))
    check_mx_gemm(y[np.ix_(rows, cols)], y_ref, bound, "dense 4096x9728x2560 sampled")


def grouped_reference(aq, asc, route, wq, wsc, cols=None):
    off, ri = route["offsets"], route["row_index"]
    groups = wq.shape[0]
    n = wq.shape[1] if cols is None else len(cols)
    y = np.full((int(off[-1]), n), np.nan)
    bound = np.full_like(y, np.nan)
    for g in range(groups):
        lo, hi = int(off[g]), int(off[g + 1])
        if hi == lo:
            continue
        src = ri[lo:hi]
        bq = wq[g] if cols is None else wq[g][cols]
        bsc = wsc[g] if cols is None else wsc[g][cols]
        y[lo:hi], bound[lo:hi] = oracle.mxfp8_gemm((aq[src], asc[src]), (bq, bsc))
    return y, bound


def test_mxfp8_grouped_small():
    T, E, n, k = 300, 16, 96, 256
    lg = sg.router_logits(71, T, E)
    route = oracle.route(lg, 4)
    aq, asc = oracle.mxfp8_quantize_rows(sg.student_t3_bf16(72, sg.S_X, (T, k)))
    w = sg.normal_bf16(73, sg.S_W, (E * n, k), 0.0, 0.02)
    wq, wsc = oracle.mxfp8_quantize_rows(w)
    wq, wsc = wq.reshape(E, n, k), wsc.reshape(E, n, k // 32)
    y = nv.nvfp4_mxfp8_grouped_gemm((to_dev(aq), to_dev(asc)), to_dev(route["offsets"]),
                                    (to_dev(wq), to_dev(wsc)), row_index=to_dev(route["row_index"]))
    torch.cuda.synchronize()
    y_ref, bound = grouped_reference(aq, asc, route, wq, wsc)
    check_mx_gemm(y, y_ref, bound, "grouped 300 tokens, 16 experts, top-4")


def test_mxfp8_grouped_moe_up_full_size_sampled():
    """The MoE up-projection at full size (4096 tokens, top-8 of 128 experts,
    fused 1536 x 2048 expert weights) on the GPU; for every expert 8 output
    columns of all its routed rows recomputed by the oracle."""
    d = workload(3, "x,w")
    route = oracle.route(workload(3, "logits")["logits"], 8)
    x, w = d["x"], d["w"]
    E, n, k = w.shape
    a_dev = nv.nvfp4_mxfp8_quantize_rows(to_dev(x))
    w_dev = nv.nvfp4_mxfp8_quantize_rows(to_dev(w.reshape(E * n, k)))
    y = to_np(nv.nvfp4_mxfp8_grouped_gemm(
        a_dev, to_dev(route["offsets"]), (w_dev[0].view(E, n, k), w_dev[1].view(E, n, k // 32)),
        row_index=to_dev(route["row_index"])))
    cols = (np.arange(8) * 191 + 5) % n
    aq, asc = oracle.mxfp8_quantize_rows(x)
    wq = np.empty((E, len(cols), k), np.uint8)
    wsc = np.empty((E, len(cols), k // 32), np.uint8)
    for g in range(E):
        wq[g], wsc[g] = oracle.mxfp8_quantize_rows(w[g][cols])
    y_ref, bound = grouped_reference(aq, asc, route, wq, wsc)
    check_mx_gemm(y[:, cols], y_ref, bound, "grouped MoE up sampled")


def test_mxfp8_gemm_errors():
    d = dev()
    z = torch.zeros((4, 48), dtype=torch.uint8, device=d)
    zs = torch.zeros((4, 1), dtype=torch.uint8, device=d)
    # k = 48 is not a multiple of 32: the binding finds no scale shape for it,
    # and the library itself returns UNSUPPORTED_SHAPE
    with pytest.raises(ValueError):
        nv.nvfp4_mxfp8_gemm((z, zs), (z, zs))
    y = torch.empty((4, 4), dtype=torch.float32, device=d)
    sp = torch.cuda.current_stream(d).cuda_stream
    st = nv.lib().nvfp4_mxfp8_gemm(z.data_ptr(), zs.data_ptr(), 4, z.data_ptr(), zs.data_ptr(), 4, 48,
                                   y.data_ptr(), sp)
    assert st == 2


def test_mxfp8_gemm_small_products_beside_a_large_one():
    """Blocks whose largest product is 448^2 and whose other 31 products are
    1, 0.5 or 0.25 (same sign): exact decoding keeps every small product
    (the scaled fp8 MFMA's truncating window would drop them, an error of up
    to 31 against a bound of 2.0)."""
    k = 256
    rows = []
    for small in (1.0, 0.5, 0.25, 2.0):
        for nblocks in (1, 3, 8):
            r = np.zeros(k, np.float32)
            for b in range(nblocks):
                r[32 * b] = 448.0
                r[32 * b + 1:32 * b + 32] = small
            rows.append(r)
    x = np.stack(rows)
    xb = (x.view(np.uint32) >> 16).astype(np.uint16)   # exact in bf16
    a = oracle.mxfp8_quantize_rows(xb)
    y = nv.nvfp4_mxfp8_gemm(mx_dev(a), mx_dev(a))
    y_ref, bound = oracle.mxfp8_gemm(a, a)
    check_mx_gemm(y, y_ref, bound, "large and small products")


@pytest.mark.parametrize("k", [256, 96])
def test_mxfp8_grouped_invalid_rows_read_as_zero(k):
    """Gathered rows whose index lies outside [0, a_rows) are zero rows on
    both kernels (k = 256: the LDS tile kernel, whose stale LDS bytes must
    not leak into such rows; k = 96: the shared-tile kernel)."""
    groups, n, tokens = 4, 160, 12
    aq, asc = oracle.mxfp8_quantize_rows(sg.student_t3_bf16(81, sg.S_X, (tokens, k)))
    w = sg.normal_bf16(82, sg.S_W, (groups * n, k), 0.0, 0.02)
    wq, wsc = oracle.mxfp8_quantize_rows(w)
    wq, wsc = wq.reshape(groups, n, k), wsc.reshape(groups, n, k // 32)
    offsets = np.array([0, 3, 3, 8, 10], np.int32)
    ri = ((np.arange(10) * 5) % tokens).astype(np.int32)
    ri[1] = -4
    ri[6] = tokens
    dev_b = (to_dev(wq), to_dev(wsc))
    # a first call with valid indices everywhere leaves real operand bytes in
    # LDS for the second
    nv.nvfp4_mxfp8_grouped_gemm((to_dev(aq), to_dev(asc)), to_dev(offsets), dev_b,
                                row_index=to_dev((np.arange(10) % tokens).astype(np.int32)))
    y = to_np(nv.nvfp4_mxfp8_grouped_gemm((to_dev(aq), to_dev(asc)), to_dev(offsets), dev_b,
                                          row_index=to_dev(ri)))
    assert np.all(y[1] == 0) and np.all(y[6] == 0)
    ok = np.ones(10, bool)
    ok[[1, 6]] = False
    route = {"offsets": offsets, "row_index": np.where(ok, ri, 0).astype(np.int32)}
    y_ref, bound = grouped_reference(aq, asc, route, wq, wsc)
    check_mx_gemm(y[ok], y_ref[ok], bound[ok], "valid rows k=%d" % k)
