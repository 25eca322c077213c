"""GPU parity of the NVFP4 quantizers against the oracle: bit-exact codes,
block scales and outer scales.

Test classes follow the Miles page (section 位级精确的量化器契约): random data,
data on quantization boundaries, all-zero tensors and maximum values; plus
the pages' batch-invariance requirement for per-token scales (miniTE report,
section 激活精度、缩放粒度与KV Cache) and amax reuse (miniTE report, section
Transformer Engine路径优化).  Results are reported per case as N/N matches.
"""
import numpy as np
import pytest
import torch

import nvfp4_token_quantization_amd as nv
import nvfp4_token_quantization_amd.selftest as st
import oracle
import synthgen as sg
from gpu_helpers import assert_same_quant, dev, oracle_rows, oracle_weight, to_dev, to_np, workload

pytestmark = pytest.mark.gpu

E4M3 = None


def _e4m3():
    global E4M3
    if E4M3 is None:
        E4M3 = oracle.e4m3_table()
    return E4M3


def _bf16(vals):
    return sg.f32_to_bf16(np.asarray(vals, np.float32))


def boundary_rows(rows, k, seed):
    """Rows whose block amaxes and elements sit on E4M3 / E2M1 rounding
    boundaries: anchor block amax 2688 * 2^e (so S = 2^e exactly), then blocks
    with a chosen scale code c whose elements are E2M1 midpoints and grid
    points times d = 2^e * s_b(c), their bf16 neighbours, and blocks whose
    amax is the midpoint between two E4M3 values."""
    e4 = _e4m3()
    u = sg.uniform(seed, 1, rows * (k // 16 + 1) * 64)
    ui = iter(u)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 0.5, 1, 1.5, 2, 3, 4, 6, 0.0])
    out = np.zeros((rows, k), np.uint16)
    for r in range(rows):
        e = int(next(ui) * 40) - 20
        row = np.zeros(k, np.float64)
        row[0] = 2688.0 * 2.0 ** e
        for b in range(1, k // 16):
            kind = next(ui)
            c = 1 + int(next(ui) * 0x7D)
            d = 2.0 ** e * e4[c]
            if kind < 0.6:
                vals = [6.0 * d] + [mids[int(next(ui) * len(mids))] * d for _ in range(15)]
            else:
                top = 6.0 * 2.0 ** e * (e4[c] + e4[c + 1]) / 2.0
                vals = [top] + [top * next(ui) for _ in range(15)]
            vals = np.array(vals)
            signs = np.where(np.array([next(ui) for _ in range(16)]) < 0.5, -1.0, 1.0)
            row[16 * b:16 * b + 16] = vals * signs
        xb = _bf16(row)
        # nudge some elements to a bf16 neighbour (one ulp up or down)
        for j in range(16, k):
            t = next(ui)
            mag = int(xb[j]) & 0x7FFF
            if t < 0.15 and 1 < mag < 0x7F7F:
                xb[j] = np.uint16(int(xb[j]) + (1 if t < 0.075 else -1))
        out[r] = xb
    return out


def zero_rows(rows, k, seed):
    u = sg.uniform(seed, 2, rows * k).reshape(rows, k)
    x = sg.normal_bf16(seed, 3, (rows, k))
    x[u < 0.5] = 0
    x[(u >= 0.5) & (u < 0.6)] = 0x8000          # -0
    x[::3] = 0                                   # all-zero rows
    x[1::3, : k // 2] = 0                        # zero blocks in non-zero rows
    x[2::5] = 0x8000                             # all -0 rows
    return x


def max_rows(rows, k, seed):
    u = sg.uniform(seed, 4, rows * k).reshape(rows, k)
    x = sg.normal_bf16(seed, 5, (rows, k), 0.0, 1e-30)
    x[u < 0.3] = 0x7F7F                          # +max finite bf16
    x[(u >= 0.3) & (u < 0.5)] = 0xFF7F           # -max
    x[::4] = np.where(u[::4] < 0.5, 0x7F7F, 0xFF7F)   # whole rows of +-max
    x[1::4] = np.where(u[1::4] < 0.5, 0x0001, 0x8001)  # rows of +-smallest subnormal
    x[2::4, ::7] = 0x0080                        # smallest normal among maxes
    return x


K_LIST = [16, 48, 512, 768, 2048, 2560, 4112, 8208]


@pytest.mark.parametrize("k", K_LIST)
@pytest.mark.parametrize("cls", ["random", "boundary", "zeros", "maxes"])
def test_quantize_rows_classes(k, cls):
    rows = 37 if k <= 4112 else 9
    seed = 1000 + k
    if cls == "random":
        x = sg.student_t3_bf16(seed, 1, (rows, k))
    elif cls == "boundary":
        x = boundary_rows(rows, k, seed)
    elif cls == "zeros":
        x = zero_rows(rows, k, seed)
    else:
        x = max_rows(rows, k, seed)
    got = nv.nvfp4_quantize_rows(to_dev(x))
    want = oracle.quantize_rows(x)
    assert_same_quant(got, want, "%s k=%d" % (cls, k))


@pytest.mark.parametrize("rows", [1, 2, 3, 5, 63, 64, 65, 1000])
def test_quantize_rows_ragged_counts(rows):
    for k in (512, 768, 2560):
        x = sg.student_t3_bf16(77 + rows, 1, (rows, k))
        assert_same_quant(nv.nvfp4_quantize_rows(to_dev(x)), oracle.quantize_rows(x),
                          "rows=%d k=%d" % (rows, k))


# The smallest and largest K (at most 8192) of every row layout the row
# kernels select (L lanes per row x U half-blocks per lane: L = 16 for K up
# to 240 and 384..1920 when the half-blocks divide by 16 only, L = 32 when
# they divide by 32 only, L = 64 otherwise; U from 1 to 16), and two K past
# 8192 (the long-row kernel).
LAYOUT_K = [16, 128, 144, 240, 384, 640, 896, 1152, 1408, 1664, 1920,
            256, 272, 496, 768, 1280, 1792, 2304, 2816, 3328, 3840,
            512, 528, 1024, 1040, 1536, 1552, 2048, 2064, 2560, 2576, 3072, 3088, 4096,
            4112, 5120, 5136, 6144, 6160, 8192, 8208, 9456]


def _spread_rows(seed, rows, k):
    """Student-t rows, each scaled by its own power of two from 2^-40 to
    2^40 (exact in bf16), so the outer scales span many exponents."""
    x = sg.bf16_to_f32(sg.student_t3_bf16(seed, 1, (rows, k)))
    e = (sg.uniform(seed, 2, rows) * 81).astype(np.int64) - 40
    return sg.f32_to_bf16(x * np.exp2(e.astype(np.float32))[:, None])


@pytest.mark.parametrize("k", LAYOUT_K)
def test_every_row_layout_all_modes(k):
    """Each layout in the three modes: row amax, supplied amax (the exact row
    amax, as a producer would reuse it) and weights (one group of all rows,
    and groups of one row each); 257 rows, so the last block's row groups
    are partial."""
    rows = 257
    x = _spread_rows(4000 + k, rows, k)
    xd = to_dev(x)
    assert_same_quant(nv.nvfp4_quantize_rows(xd), oracle.quantize_rows(x), "rows k=%d" % k)
    amax = np.abs(sg.bf16_to_f32(x)).max(axis=1).astype(np.float32)
    assert_same_quant(nv.nvfp4_quantize_rows(xd, amax_in=to_dev(amax)),
                      oracle.quantize_rows(x, amax_in=amax), "amax_in k=%d" % k)
    for shape in ((1, rows, k), (rows, 1, k)):
        w = x.reshape(shape)
        assert_same_quant(nv.nvfp4_quantize_weight(to_dev(w)), oracle.quantize_weight(w),
                          "weight %s" % (shape,))


def test_quantize_rows_k0_and_empty():
    x = torch.empty((5, 0), dtype=torch.int16, device=dev())
    q, sb, s = nv.nvfp4_quantize_rows(x)
    assert q.numel() == 0 and sb.numel() == 0 and torch.all(s == 0)
    a = torch.tensor([2688.0, 0.0, 1.0, 5376.0, 3.0], device=dev())
    q, sb, s = nv.nvfp4_quantize_rows(x, amax_in=a)
    assert np.array_equal(to_np(s), (a.cpu().numpy() / np.float32(2688.0)).astype(np.float32))
    q, sb, s = nv.nvfp4_quantize_rows(torch.empty((0, 64), dtype=torch.int16, device=dev()))
    assert q.shape == (0, 32)


@pytest.mark.parametrize("cfg,name", [(1, "x"), (2, "x"), (3, "x"), (4, "h"), (5, "x"), (5, "h"),
                                      (5, "xd")])
def test_quantize_rows_workloads(cfg, name):
    d = workload(cfg, name)
    x = d[name]
    got = nv.nvfp4_quantize_rows(to_dev(x))
    assert_same_quant(got, oracle_rows(cfg, name), "config %d %s" % (cfg, name))
    if name + "_amax" in d:
        got2 = nv.nvfp4_quantize_rows(to_dev(x), amax_in=to_dev(d[name + "_amax"]))
        assert_same_quant(got2, oracle_rows(cfg, name, True), "config %d %s amax reuse" % (cfg, name))
        assert_same_quant(got2, [to_np(t) for t in got], "amax reuse == recompute")


def test_amax_in_other_than_row_max():
    """amax_in is taken as given (bits are a function of x and amax_in),
    including amax values below the true max (saturation) and above it."""
    x = sg.student_t3_bf16(91, 1, (64, 768))
    amax = sg.row_amax_bf16(x)
    fac = np.where(np.arange(64) % 2 == 0, 0.37, 3.0).astype(np.float32)
    a2 = (amax * fac).astype(np.float32)
    a2[5] = 0.0
    got = nv.nvfp4_quantize_rows(to_dev(x), amax_in=to_dev(a2))
    assert_same_quant(got, oracle.quantize_rows(x, amax_in=a2), "amax_in scaled")


def test_batch_invariance_config4():
    """Each token's bits are identical alone, in seeded random subsets and in
    the full 32768-row batch (with and without amax reuse)."""
    d = workload(4, "h")
    h, amax = d["h"], d["h_amax"]
    full = [to_np(t) for t in nv.nvfp4_quantize_rows(to_dev(h))]
    full_r = [to_np(t) for t in nv.nvfp4_quantize_rows(to_dev(h), amax_in=to_dev(amax))]
    assert_same_quant(full, oracle_rows(4, "h"), "config 4 full batch")
    n = h.shape[0]
    alone = (sg.uniform(4, 20, 16) * n).astype(np.int64)
    for t in alone:
        got = nv.nvfp4_quantize_rows(to_dev(h[t:t + 1]))
        assert_same_quant(got, [f[t:t + 1] for f in full], "token %d alone" % t)
    sizes = [2, 7, 64, 100, 1000, 4096, 10000, 20000]
    for i, sz in enumerate(sizes):
        idx = np.argsort(sg.uniform(4, 30 + i, n))[:sz]
        got = nv.nvfp4_quantize_rows(to_dev(h[idx]))
        assert_same_quant(got, [f[idx] for f in full], "subset %d of size %d" % (i, sz))
        got = nv.nvfp4_quantize_rows(to_dev(h[idx]), amax_in=to_dev(amax[idx]))
        assert_same_quant(got, [f[idx] for f in full_r], "subset %d (amax reuse)" % i)


def test_quantize_rows_deterministic():
    x = to_dev(workload(2, "x")["x"])
    ref = [to_np(t) for t in nv.nvfp4_quantize_rows(x)]
    for _ in range(10):
        assert_same_quant(nv.nvfp4_quantize_rows(x), ref, "repeat")


@pytest.mark.parametrize("cfg,name", [(1, "w"), (2, "w"), (3, "w"), (4, "w"), (5, "wd")])
def test_quantize_weight_workloads(cfg, name):
    w = workload(cfg, name)[name]
    got = nv.nvfp4_quantize_weight(to_dev(w))
    assert_same_quant(got, oracle_weight(cfg, name), "config %d %s" % (cfg, name))


def test_quantize_weight_groups_and_amax_in():
    w = sg.normal_bf16(55, 2, (6, 40, 272), 0.0, 0.02)
    w[2] = 0                                        # an all-zero expert
    w[4, :, :16] = 0x7F7F                           # an expert with max values
    assert_same_quant(nv.nvfp4_quantize_weight(to_dev(w)), oracle.quantize_weight(w), "groups")
    a = np.array([0.1, 0.2, 0.0, 1e-3, 3e38, 0.05], np.float32)
    got = nv.nvfp4_quantize_weight(to_dev(w), amax_in=to_dev(a))
    want = oracle.quantize_weight(w, amax_in=a)
    assert_same_quant(got, want, "groups amax_in")
    # fused gate/up as one group per expert shares one outer scale
    gate = sg.normal_bf16(56, 1, (3, 24, 256), 0.0, 0.02)
    up = sg.normal_bf16(56, 2, (3, 24, 256), 0.0, 0.05)
    fused = np.concatenate([gate, up], axis=1)
    got = nv.nvfp4_quantize_weight(to_dev(fused))
    assert_same_quant(got, oracle.quantize_weight(fused), "fused gate/up")
    # rows longer than 1024 half-blocks take the one-wave-per-row kernel,
    # which also stores each group's outer scale
    wl = sg.normal_bf16(57, 2, (3, 5, 8208), 0.0, 0.02)
    wl[1, 2, 8000:8016] = 0x7F7F
    assert_same_quant(nv.nvfp4_quantize_weight(to_dev(wl)), oracle.quantize_weight(wl), "long rows")
    # one group of one row equals per-token quantization of the row
    got1 = nv.nvfp4_quantize_weight(to_dev(w[:1, :1]))
    gotr = nv.nvfp4_quantize_rows(to_dev(w[0, :1]))
    assert_same_quant(got1[:3], [to_np(t) for t in gotr], "1-row weight == per-token")


# ---------------------------------------------------------------- codecs --
def _sweep(encode, lo, hi, chunk=1 << 27):
    """Device codes for every fp32 bit pattern in [lo, hi) (as uint32)."""
    for a in range(lo, hi, chunk):
        b = min(hi, a + chunk)
        bits_ = torch.arange(a, b, dtype=torch.int64, device=dev()).to(torch.int32)
        yield a, encode(bits_.view(torch.float32))


def test_e2m1_codec_exhaustive():
    """Every fp32 bit pattern through the device E2M1 rounding: for x >= 0 the
    codes must be non-decreasing in x and agree with the oracle on both sides
    of every rounding boundary and at 0 and +inf (together these pin every
    value); negative inputs must give the positive code with the sign bit."""
    POS_END = 0x7F800001   # through +inf
    last = -1
    for a, codes in _sweep(st.nvfp4_debug_encode_e2m1, 0, POS_END):
        c = codes.to(torch.int16)
        assert int(c.max()) <= 7
        assert bool(torch.all(c[1:] >= c[:-1])), "not monotone in chunk at %#x" % a
        assert int(c[0]) >= last
        last = int(c[-1])
        neg = st.nvfp4_debug_encode_e2m1(
            (torch.arange(a, a + c.numel(), dtype=torch.int64, device=dev()) | 0x80000000)
            .to(torch.int32).view(torch.float32))
        assert bool(torch.all(neg.to(torch.int16) == (c | 8))), "sign handling at %#x" % a
    # boundary points: midpoints of the grid, their fp32 neighbours, grid points
    grid = oracle.e2m1_table()[:8]
    pts = [0.0, np.inf, np.float32(np.finfo(np.float32).max), np.float32(1e-45)]
    for m in (grid[:-1] + grid[1:]) / 2:
        f = np.float32(m)
        pts += [f, np.nextafter(f, np.float32(0)), np.nextafter(f, np.float32(np.inf))]
    pts += list(grid.astype(np.float32))
    v = np.array(pts, np.float32)
    got = to_np(st.nvfp4_debug_encode_e2m1(to_dev(v)))
    assert np.array_equal(got, oracle.rne_sat_e2m1(v)), list(zip(v, got, oracle.rne_sat_e2m1(v)))


def test_e4m3_codec_exhaustive():
    """Every non-negative fp32 bit pattern (through +inf) through the device
    E4M3 block-scale rounding: non-decreasing, and equal to the oracle on both
    sides of all 126 boundaries, at every code value, at 0 and at +inf."""
    last = -1
    for a, codes in _sweep(st.nvfp4_debug_encode_e4m3, 0, 0x7F800001):
        c = codes.to(torch.int16)
        assert int(c.max()) <= 0x7E
        assert bool(torch.all(c[1:] >= c[:-1])), "not monotone in chunk at %#x" % a
        assert int(c[0]) >= last
        last = int(c[-1])
    tab = oracle.e4m3_table()[:0x7F]
    pts = [0.0, np.inf, np.float32(1e-45), np.float32(3e38)]
    for m in (tab[:-1] + tab[1:]) / 2:
        f = np.float32(m)
        pts += [f, np.nextafter(f, np.float32(0)), np.nextafter(f, np.float32(np.inf))]
    pts += list(tab.astype(np.float32))
    pts += [np.float32(448.0), np.nextafter(np.float32(448.0), np.float32(np.inf)), np.float32(464.0),
            np.float32(480.0)]
    v = np.array(pts, np.float32)
    got = to_np(st.nvfp4_debug_encode_e4m3(to_dev(v)))
    assert np.array_equal(got, oracle.rne_sat_e4m3(v))


# ------------------------------------------------------------ block scale --
def _bf16_bits(v):
    """float32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(v, np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def _block_scale_expected(bbits, amax):
    """Steps Q2-Q4 of the quantizer in IEEE fp32 (numpy) with the oracle's
    E4M3 codec: S = amax / 2688, t = 6 S, code = RNE_SAT(a / t) (0 when S is
    0), inv = 1 / (S * e4m3(code)) (0 when that product is 0)."""
    S = amax / np.float32(2688.0)
    t = np.float32(6.0) * S
    a = (bbits.astype(np.uint32) << 16).view(np.float32)
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        v = a / t
        v = np.where(S == 0, np.float32(0.0), v).astype(np.float32)
        code = oracle.rne_sat_e4m3(v)
        d = S * oracle.e4m3_table()[code].astype(np.float32)
        inv = np.where(d == 0, np.float32(0.0), np.float32(1.0) / d).astype(np.float32)
    return code, inv


def _check_block_scale(bbits, amax, what):
    code, inv = st.nvfp4_debug_block_scale(to_dev(bbits.view(np.int16)), to_dev(amax))
    code, inv = to_np(code), to_np(inv)
    want_code, want_inv = _block_scale_expected(bbits, amax)
    bad = np.flatnonzero((code != want_code) | (inv.view(np.uint32) != want_inv.view(np.uint32)))
    if bad.size:
        i = bad[0]
        raise AssertionError("%s: %d mismatches; first a=%#06x amax=%r: code %#x/%#x inv %r/%r" % (
            what, bad.size, bbits[i], amax[i], code[i], want_code[i], inv[i], want_inv[i]))


def test_block_scale_reciprocal_sweep():
    """The block scale's reciprocal 1 / (S * s_b) over 99% of all fp32
    significands of the product: every row amax of one binade, with a block
    amax chosen so the block scale is 1, 1.125, 1.25 or 1.375."""
    amax = (np.arange(1 << 23, dtype=np.uint32) | np.uint32(127 << 23)).view(np.float32)
    S = amax / np.float32(2688.0)
    for m in (1.0, 1.125, 1.25, 1.375):
        bbits = _bf16_bits(np.float32(m) * (np.float32(6.0) * S))
        _check_block_scale(bbits, amax, "s_b = %g" % m)


def test_block_scale_quotients_and_edges():
    """Block amax over the full bf16 range against row amaxes spread over
    fp32's range (so a_b / 6S covers every code, saturation and underflow),
    plus edge rows: S = 0, subnormal and huge amax (the exact-division
    fallbacks), block amax above the row amax (amax reuse with a smaller
    amax_in), subnormal and largest bf16 blocks, and products S * s_b with a
    significand of all ones."""
    n = 1 << 22
    e = np.floor(sg.uniform(91, sg.S_MISC, n) * 250.0) - 125.0
    amax = np.ldexp(sg.uniform(92, sg.S_MISC, n) + 1.0, e.astype(np.int64)).astype(np.float32)
    ratio = sg.uniform(93, sg.S_MISC, n) * 1.1
    ratio = np.where(sg.uniform(94, sg.S_MISC, n) < 0.1, ratio * 1e-3, ratio)
    bbits = _bf16_bits((amax * ratio).astype(np.float32))
    _check_block_scale(bbits, amax, "random")

    edges_b, edges_a = [], []
    specials = [0.0, 1e-45, 1e-40, 1.2e-38, 1e-30, 1e-28, 1.0, 2688.0, 1e28, 1e30, 3e38,
                np.finfo(np.float32).max]
    blocks = [0x0000, 0x0001, 0x007F, 0x0080, 0x3F80, 0x43E0, 0x7F7F, 0x7F00, 0x0400]
    for a in specials:
        for b in blocks:
            edges_a.append(a)
            edges_b.append(b)
    # S * s_b with an all-ones significand (the reciprocal's fallback): found
    # among row amaxes in [1, 1.25) for s_b = 1.125 and 1.25, then scaled by
    # powers of two (which keep the significand)
    win = (np.arange(1 << 21, dtype=np.uint32) | np.uint32(127 << 23)).view(np.float32)
    Sw = win / np.float32(2688.0)
    found = 0
    for m in (1.125, 1.25):
        d = Sw * np.float32(m)
        for i in np.flatnonzero((d.view(np.uint32) & 0x7FFFFF) == 0x7FFFFF):
            for k in (-60, -20, 0, 20, 60):
                am = np.float32(np.ldexp(np.float64(win[i]), k))
                edges_a.append(am)
                Sk = am / np.float32(2688.0)
                edges_b.append(int(_bf16_bits(np.array([np.float32(m) * (np.float32(6.0) * Sk)]))[0]))
                found += 1
    assert found >= 10
    _check_block_scale(np.array(edges_b, np.uint16), np.array(edges_a, np.float32), "edges")
