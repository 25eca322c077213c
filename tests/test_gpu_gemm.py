"""GPU parity of the dense and grouped block-scaled GEMMs against the
oracle's exact result: |Y - Y_ref| <= 1e-5 * sum_k |a_k b_k| per entry (and
Y = +-0 where that sum is 0).  Operands are quantized by the oracle, so no
GEMM input comes from the GPU quantizer.

Small shapes span several tiles, ragged M/N tails and K tails (k % 256 == 0
takes the LDS-staged kernel, other multiples of 128 the register-direct one,
the rest its masked loader) and are compared in full; the workload shapes are
compared on seeded samples of entries plus whole rows and columns.
"""
import numpy as np
import pytest
import torch

import nvfp4_token_quantization_amd as nv
import oracle
import synthgen as sg
from gpu_helpers import check_gemm, dev, oracle_rows, oracle_weight, routing, to_dev, to_np, workload

pytestmark = pytest.mark.gpu


def quant_pair(seed, m, n, k, groups=None):
    x = sg.student_t3_bf16(seed, 1, (m, k))
    a = oracle.quantize_rows(x)
    w = sg.normal_bf16(seed, 2, (groups or 1, n, k), 0.0, 0.02)
    bq, bsb, bs, _ = oracle.quantize_weight(w)
    return a, (bq, bsb, bs)


def dev_op(t):
    return tuple(to_dev(np.ascontiguousarray(v)) for v in t)


@pytest.mark.parametrize("m,n,k", [(1, 1, 16), (3, 5, 32), (37, 53, 512), (128, 128, 128),
                                   (130, 260, 1040), (257, 129, 2048), (64, 384, 2560),
                                   (300, 200, 784), (65, 1100, 256), (96, 200, 384),
                                   (200, 136, 768)])
def test_dense_small(m, n, k):
    a, b = quant_pair(m * 1000 + n + k, m, n, k)
    y = nv.nvfp4_gemm(dev_op(a), (to_dev(b[0][0]), to_dev(b[1][0]), to_dev(b[2])))
    y_ref, bound = oracle.gemm(a, (b[0][0], b[1][0], b[2]))
    check_gemm(y, y_ref, bound, "dense %dx%dx%d" % (m, n, k))


def test_dense_all_scale_codes_random_codes():
    """Operands with every E4M3 scale code (subnormal ones included), every
    element code and a wide spread of outer scales."""
    m, n, k = 96, 160, 2048
    rnd = lambda s, shape, hi: (sg.uniform(s, 1, int(np.prod(shape))) * hi).astype(np.int64).reshape(shape)
    aq = rnd(1, (m, k // 2), 256).astype(np.uint8)
    bq = rnd(2, (n, k // 2), 256).astype(np.uint8)
    asb = rnd(3, (m, k // 16), 0x7F).astype(np.uint8)
    bsb = rnd(4, (n, k // 16), 0x7F).astype(np.uint8)
    asb[:, :8] = np.arange(8, dtype=np.uint8)[None, :]      # subnormal E4M3 scales
    as_ = (2.0 ** (rnd(5, (m,), 60) - 30)).astype(np.float32) * np.float32(1.2345)
    bs = np.array([0.0123], np.float32)
    y = nv.nvfp4_gemm((to_dev(aq), to_dev(asb), to_dev(as_)), (to_dev(bq), to_dev(bsb), to_dev(bs)))
    y_ref, bound = oracle.gemm((aq, asb, as_), (bq, bsb, bs))
    check_gemm(y, y_ref, bound, "random codes")


def test_dense_very_wide_output():
    """n >= 2^22 takes the LDS kernel's per-element epilogue (the buffer-store
    epilogue needs the tile's output bytes under 2^31); a 40-column tail past
    2^22 and every column near the end are compared, plus random entries."""
    m, n, k = 3, (1 << 22) + 40, 256
    rnd = lambda s, shape, hi: (sg.uniform(s, 1, int(np.prod(shape))) * hi).astype(np.int64).reshape(shape)
    aq = rnd(11, (m, k // 2), 256).astype(np.uint8)
    asb = rnd(12, (m, k // 16), 0x7F).astype(np.uint8)
    as_ = np.array([0.5, 3.0, 0.0078125], np.float32)
    # B: a 4096-row random block repeated down the rows (distinct bytes per
    # 4096 columns are enough to place every output), then the tail rows
    blk_q = rnd(13, (4096, k // 2), 256).astype(np.uint8)
    blk_s = (0x28 + rnd(14, (4096, k // 16), 0x20)).astype(np.uint8)
    reps = n // 4096 + 1
    bq = np.tile(blk_q, (reps, 1))[:n]
    bsb = np.tile(blk_s, (reps, 1))[:n]
    bs = np.array([0.25], np.float32)
    y = to_np(nv.nvfp4_gemm((to_dev(aq), to_dev(asb), to_dev(as_)), (to_dev(bq), to_dev(bsb), to_dev(bs))))
    cnt = 20000
    ii = np.concatenate([(sg.uniform(15, 1, cnt) * m).astype(np.int64), np.repeat(np.arange(m), 300)])
    jj = np.concatenate([(sg.uniform(15, 2, cnt) * n).astype(np.int64),
                         np.tile(np.arange(n - 300, n), m)])
    y_ref, bound = oracle.gemm_entries((aq, asb, as_), (bq, bsb, bs), ii, jj, np.zeros_like(ii))
    check_gemm(y[ii, jj], y_ref, bound, "dense %dx%dx%d" % (m, n, k))


def test_dense_k0_and_zero_scales():
    m, n = 5, 7
    e = lambda *s: torch.empty(s, dtype=torch.uint8, device=dev())
    y = nv.nvfp4_gemm((e(m, 0), e(m, 0), torch.ones(m, device=dev())),
                      (e(n, 0), e(n, 0), torch.ones(1, device=dev())))
    assert torch.all(y == 0)
    a, b = quant_pair(5, 40, 30, 256)
    a = (a[0], a[1], np.zeros_like(a[2]))
    y = nv.nvfp4_gemm(dev_op(a), (to_dev(b[0][0]), to_dev(b[1][0]), to_dev(b[2])))
    assert torch.all(y == 0)


def _sample(m, n, count, seed):
    ii = (sg.uniform(seed, 1, count) * m).astype(np.int64)
    jj = (sg.uniform(seed, 2, count) * n).astype(np.int64)
    # plus one full row and one full column at the ends
    ii = np.concatenate([ii, np.full(n, m - 1), np.arange(m)])
    jj = np.concatenate([jj, np.arange(n), np.full(m, n - 1)])
    return ii, jj


@pytest.mark.parametrize("cfg", [1, 2, 5])
def test_dense_workloads(cfg):
    xname, wname = ("x", "w") if cfg != 5 else ("xd", "wd")
    a = oracle_rows(cfg, xname)
    wq, wsb, ws, _ = oracle_weight(cfg, wname)
    b = (wq[0], wsb[0], ws)
    y = to_np(nv.nvfp4_gemm(dev_op(a), dev_op(b)))
    m, n = y.shape
    if m * n <= 1 << 20:
        y_ref, bound = oracle.gemm(a, b)
        check_gemm(y, y_ref, bound, "config %d dense (all entries)" % cfg)
    else:
        ii, jj = _sample(m, n, 60000, cfg)
        y_ref, bound = oracle.gemm_entries(a, b, ii, jj, np.zeros(len(ii), np.int64))
        check_gemm(y[ii, jj], y_ref, bound, "config %d dense (%d sampled entries)" % (cfg, len(ii)))


def test_dense_deterministic():
    a, b = quant_pair(9, 300, 500, 2048)
    bd = (to_dev(b[0][0]), to_dev(b[1][0]), to_dev(b[2]))
    ad = dev_op(a)
    y0 = nv.nvfp4_gemm(ad, bd)
    for _ in range(5):
        assert torch.equal(nv.nvfp4_gemm(ad, bd), y0)


@pytest.mark.parametrize("k", [2048, 640])
def test_dense_rows_batch_invariant_tiled(k):
    """The tiled kernels (m > 64; k = 2048 takes the LDS-staged kernel, 640
    the register-direct one) compute each output row from its own A row in
    a fixed order: rows 70..199 of a 300-row call equal a 130-row call on
    those rows, bit for bit, though they sit at other tile positions (and
    the 130-row call's last round is issued as half tiles)."""
    a, b = quant_pair(19, 300, 333, k)
    bd = (to_dev(b[0][0]), to_dev(b[1][0]), to_dev(b[2]))
    ad = dev_op(a)
    y = nv.nvfp4_gemm(ad, bd)
    sub = tuple(t[70:200].contiguous() for t in ad)
    ys = nv.nvfp4_gemm(sub, bd)
    assert torch.equal(ys, y[70:200])


# ---------------------------------------------------------------- grouped --
def grouped_case(seed, tokens, counts, n, k, row_index=True):
    groups = len(counts)
    x = sg.student_t3_bf16(seed, 1, (tokens, k))
    a = oracle.quantize_rows(x)
    w = sg.normal_bf16(seed, 2, (groups, n, k), 0.0, 0.02)
    bq, bsb, bs, _ = oracle.quantize_weight(w)
    offsets = np.zeros(groups + 1, np.int32)
    offsets[1:] = np.cumsum(counts)
    m_total = int(offsets[-1])
    ri = ((np.arange(m_total) * 7919) % tokens).astype(np.int32) if row_index else None
    return a, (bq, bsb, bs), offsets, ri


@pytest.mark.parametrize("counts,n,k", [
    ([5, 0, 130, 1, 0, 64, 300], 96, 512),
    ([1, 1, 1, 1], 130, 256),
    ([0, 0, 257], 64, 2048),
    ([40, 3, 0, 77], 200, 1040),
    ([128, 128, 128], 128, 128),
    ([3, 70, 0, 129], 160, 384),
])
def test_grouped_small(counts, n, k):
    tokens = 211
    a, b, offsets, ri = grouped_case(len(counts) * 31 + n + k, tokens, counts, n, k)
    m_total = int(offsets[-1])
    y = torch.full((m_total + 3, n), float("nan"), device=dev())
    nv.nvfp4_grouped_gemm(dev_op(a), to_dev(offsets), dev_op(b), row_index=to_dev(ri),
                          m_total=m_total, out=y)
    y = to_np(y)
    y_ref, bound = oracle.grouped_gemm(a, offsets, b, row_index=ri)
    check_gemm(y[:m_total], y_ref, bound, "grouped %s n=%d k=%d" % (counts, n, k))
    assert np.all(np.isnan(y[m_total:])), "rows past offsets[groups] must not be written"


def test_grouped_without_row_index():
    counts = [17, 0, 200, 33]
    a, b, offsets, _ = grouped_case(44, 250, counts, 192, 768, row_index=False)
    y = nv.nvfp4_grouped_gemm(dev_op(a), to_dev(offsets), dev_op(b))
    y_ref, bound = oracle.grouped_gemm(a, offsets, b, m_total=250)
    m = int(offsets[-1])
    check_gemm(to_np(y)[:m], y_ref[:m], bound[:m], "grouped, rows in place")


@pytest.mark.parametrize("n,k", [(512, 768), (1000, 256), (2048, 512)])
def test_grouped_in_place_split_into_column_slices(n, k):
    """A grouped GEMM without row_index and at least 4 column tiles runs its
    XCD regions as 2 row halves x 4 column slices: uneven experts (empty,
    one-slab, several tiles) with a ragged last column tile at n = 1000;
    every entry against the oracle."""
    counts = [300, 0, 17, 129, 1, 64, 0, 250, 33, 96, 5, 400]
    a, b, offsets, _ = grouped_case(61 + n, sum(counts), counts, n, k, row_index=False)
    y = to_np(nv.nvfp4_grouped_gemm(dev_op(a), to_dev(offsets), dev_op(b)))
    y_ref, bound = oracle.grouped_gemm(a, offsets, b)
    check_gemm(y, y_ref, bound, "grouped in place n=%d k=%d" % (n, k))


def test_grouped_single_expert_matches_dense():
    a, b = quant_pair(12, 300, 256, 1024)
    ad, bd = dev_op(a), dev_op(b)
    yd = nv.nvfp4_gemm(ad, (bd[0][0], bd[1][0], bd[2]))
    yg = nv.nvfp4_grouped_gemm(ad, to_dev(np.array([0, 300], np.int32)), bd)
    assert torch.equal(yd, yg)


def test_grouped_invalid_row_index_reads_zero_rows():
    counts = [10, 10]
    a, b, offsets, ri = grouped_case(13, 50, counts, 64, 256)
    ri = ri.copy()
    ri[3] = -1
    ri[15] = 50
    y = to_np(nv.nvfp4_grouped_gemm(dev_op(a), to_dev(offsets), dev_op(b), row_index=to_dev(ri)))
    assert np.all(y[3] == 0) and np.all(y[15] == 0)
    ok = np.ones(20, bool)
    ok[[3, 15]] = False
    ri2 = ri.copy()
    ri2[~ok] = 0
    y_ref, bound = oracle.grouped_gemm(a, offsets, b, row_index=ri2)
    check_gemm(y[ok], y_ref[ok], bound[ok], "valid rows")


def _grouped_sample(offsets, n, count, seed):
    m = int(offsets[-1])
    ii, jj = _sample(m, n, count, seed)
    g = np.searchsorted(offsets, ii, side="right") - 1
    return ii, jj, g


@pytest.mark.parametrize("cfg", [3, 4, 5])
def test_grouped_workloads(cfg):
    if cfg == 3:
        r = routing(3)
        a = oracle_rows(3, "x")
        b = oracle_weight(3, "w")[:3]
        ri, offsets = r["row_index"], r["offsets"]
    elif cfg == 4:
        r = routing(4)
        a = oracle_rows(4, "h", True)
        b = oracle_weight(4, "w")[:3]
        ri, offsets = None, r["offsets"]
    else:
        r = routing(5)
        a = oracle_rows(5, "x")
        b = oracle_weight(5, "w")[:3]
        ri, offsets = r["row_index"], r["offsets"]
    n = b[0].shape[1]
    y = to_np(nv.nvfp4_grouped_gemm(dev_op(a), to_dev(offsets), dev_op(b),
                                    row_index=None if ri is None else to_dev(ri)))
    ii, jj, g = _grouped_sample(offsets, n, 60000, 100 + cfg)
    a_row = ii if ri is None else ri[ii].astype(np.int64)
    bq = b[0].reshape(-1, b[0].shape[-1])
    bsb = b[1].reshape(-1, b[1].shape[-1])
    y_ref, bound = oracle.gemm_entries(a, (bq, bsb, b[2]), a_row, g * n + jj, g)
    check_gemm(y[ii, jj], y_ref, bound, "config %d grouped (%d sampled entries)" % (cfg, len(ii)))
    if cfg == 5:
        # small enough to compare every entry
        y_all, b_all = oracle.grouped_gemm(a, offsets, b, row_index=ri)
        check_gemm(y, y_all, b_all, "config 5 grouped (all entries)")


def test_grouped_config5_down():
    r = routing(5)
    a = oracle_rows(5, "h", True)
    b = oracle.quantize_weight(workload(5, "w_dn")["w_dn"])[:3]
    offsets = r["offsets"]
    y = nv.nvfp4_grouped_gemm(dev_op(a), to_dev(offsets), dev_op(b))
    y_ref, bound = oracle.grouped_gemm(a, offsets, b)
    check_gemm(to_np(y), y_ref, bound, "config 5 down (all entries)")


def _random_k(rng):
    # k % 256 == 0 (LDS-staged, and the few-rows kernel), other multiples of
    # 128 (register-direct) and of 16 (masked), up to 4096
    kind = int(rng.integers(0, 3))
    if kind == 0:
        return 256 * int(rng.integers(1, 17))
    if kind == 1:
        return 128 * (2 * int(rng.integers(0, 16)) + 1)
    return 16 * int(rng.integers(1, 257))


def test_dense_random_shapes():
    """A seeded sweep of 24 dense shapes: m from 1 to 900 (the few-rows
    kernel up to 64 rows when k % 256 == 0, tiled kernels above, with half
    tiles and ragged tails), n from 1 to 900, k as in _random_k; every entry
    within 1e-5 * sum_k |a_k b_k| of the oracle."""
    rng = np.random.default_rng(20261204)
    for case in range(24):
        m = int(rng.integers(1, 65)) if case % 3 == 0 else int(rng.integers(1, 901))
        n = int(rng.integers(1, 901))
        k = _random_k(rng)
        a, b = quant_pair(3000 + case, m, n, k)
        y = nv.nvfp4_gemm(dev_op(a), (to_dev(b[0][0]), to_dev(b[1][0]), to_dev(b[2])))
        y_ref, bound = oracle.gemm(a, (b[0][0], b[1][0], b[2]))
        check_gemm(y, y_ref, bound, "case %d: %dx%dx%d" % (case, m, n, k))


def test_grouped_random_layouts():
    """A seeded sweep of 16 grouped layouts: 1 to 40 experts with 0 to 300
    rows each (some layouts at most 16 rows per expert on average, the
    few-rows kernel when k % 256 == 0), n from 1 to 700, k as in _random_k,
    gathered rows with a few indices outside A; every entry of the rows the
    experts own within the bound, and the rows past offsets[groups] of a
    taller output left untouched."""
    rng = np.random.default_rng(20261205)
    for case in range(16):
        groups = int(rng.integers(1, 41))
        hi = 17 if case % 2 == 0 else 301
        counts = rng.integers(0, hi, groups)
        counts[rng.integers(0, groups)] += 1  # at least one row
        n = int(rng.integers(1, 701))
        # the sparse layouts with k % 256 == 0, so they take the few-rows kernel
        k = 256 * int(rng.integers(1, 17)) if case % 2 == 0 else _random_k(rng)
        tokens = int(rng.integers(1, 400))
        n = max(1, min(n, int(1.5e9 // (int(counts.sum()) * k))))  # bounds the oracle's work
        a, b, offsets, _ = grouped_case(3100 + case, tokens, list(counts), n, k, row_index=False)
        m_total = int(offsets[-1])
        ri = rng.integers(0, tokens, m_total).astype(np.int32)
        ri[rng.random(m_total) < 0.02] = tokens + 5  # outside A: a zero row
        y = torch.full((m_total + 2, n), float("nan"), device=dev())
        nv.nvfp4_grouped_gemm(dev_op(a), to_dev(offsets), dev_op(b), row_index=to_dev(ri),
                              m_total=m_total, out=y)
        y = to_np(y)
        bad = ri >= tokens
        assert np.all(y[:m_total][bad] == 0), "rows gathered from outside A must be zero"
        y_ref, bound = oracle.grouped_gemm(a, offsets, b, row_index=np.where(bad, 0, ri))
        check_gemm(y[:m_total][~bad], y_ref[~bad], bound[~bad], "case %d: %d groups, %d rows, n=%d k=%d" % (
            case, groups, m_total, n, k))
        assert np.all(np.isnan(y[m_total:]))
