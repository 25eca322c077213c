"""GPU parity of the few-rows (rollout-decode) GEMM path against the oracle's
exact result, |Y - Y_ref| <= 1e-5 * sum_k |a_k b_k| per entry, every entry
compared.  The library takes this path for a dense M of at most 64, or at most
16 routed rows per expert on average, when K is a multiple of 256.  Dense
items are 64 rows x 48 columns with K split over the waves of a workgroup and
the partial tiles summed in a fixed order, so the path is checked for several
K splits (1 to 8 waves, even and uneven); grouped items are up to 32 rows
of one expert x 48 columns with K split over up to 3 waves.  Also covered: ragged rows and columns, experts longer
than one item, empty experts, gathered rows, invalid row indices and
bit-identical repeated results.
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


def operands(seed, m, n, k, groups=1):
    a = oracle.quantize_rows(sg.student_t3_bf16(seed, 1, (m, k)))
    b = oracle.quantize_weight(sg.normal_bf16(seed, 2, (groups, n, k), 0.0, 0.02))[:3]
    return a, b


# The path takes K % 256 == 0 (whole chunks of 256 elements) and, dense,
# splits the chunks over up to 8 waves: 256 -> one wave; 512 -> two; 768 ->
# three; 1280 -> five; 2048 -> eight; 2560 -> eight waves of 2, 2 and six of
# 1 chunk; 16384 -> eight waves of 8 chunks.  K = 640 and 64 take the tiled
# kernels instead.
@pytest.mark.parametrize("m,n,k", [(1, 1, 256), (1, 96, 768), (17, 200, 768), (32, 64, 2560),
                                   (33, 130, 2560), (64, 9728, 2560), (64, 1536, 2048),
                                   (5, 300, 16384), (64, 33, 512), (48, 1000, 1280),
                                   (3, 50, 640), (2, 40, 64)])
def test_dense_skinny(m, n, k):
    a, b = operands(900 + m + n + k, m, n, k)
    b2 = (b[0][0], b[1][0], b[2])
    y = to_np(nv.nvfp4_gemm(dev_op(a), dev_op(b2)))
    y_ref, bound = oracle.gemm(a, b2)
    check_gemm(y, y_ref, bound, "skinny dense %dx%dx%d" % (m, n, k))


def test_dense_skinny_deterministic_and_batch_rows():
    """Repeated calls are bit-identical; each output row depends only on its
    own A row (rows quantized alone give the same Y row)."""
    m, n, k = 40, 700, 2560
    a, b = operands(951, m, n, k)
    b2 = dev_op((b[0][0], b[1][0], b[2]))
    ad = dev_op(a)
    y0 = nv.nvfp4_gemm(ad, b2)
    for _ in range(4):
        assert torch.equal(nv.nvfp4_gemm(ad, b2), y0)
    for r in (0, 17, 39):
        yr = nv.nvfp4_gemm(tuple(t[r:r + 1].contiguous() for t in ad), b2)
        assert torch.equal(yr[0], y0[r])


@pytest.mark.parametrize("counts,n,k", [
    ([1, 0, 3, 0, 0, 2, 1, 4], 1536, 2048),      # decode-like: 0-4 rows per expert
    ([0, 70, 1, 0, 0, 3, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0], 96, 768),  # one expert of 3 m-tiles
    ([17, 0, 31, 16, 15, 1], 300, 512),           # one- and two-slab m-tiles, ragged columns
    ([16, 16, 16, 16], 130, 256),
    ([0, 0, 0, 5], 64, 256),
    ([0, 0, 3, 5], 64, 64),                       # K % 256 != 0: the tiled kernel
    ([2] * 64, 2048, 768),
])
def test_grouped_skinny(counts, n, k):
    groups = len(counts)
    tokens = 37
    a, b = operands(960 + groups + n + k, tokens, n, k, groups)
    offsets = np.zeros(groups + 1, np.int32)
    offsets[1:] = np.cumsum(counts)
    m_total = int(offsets[-1])
    assert m_total <= 16 * groups
    ri = ((np.arange(m_total) * 11 + 3) % tokens).astype(np.int32)
    y = torch.full((m_total + 2, n), float("nan"), device=dev())
    nv.nvfp4_grouped_gemm(dev_op(a), to_dev(offsets), dev_op(b), row_index=to_dev(ri),
                          m_total=m_total, out=y)
    y = to_np(y)
    y_ref, bound = oracle.grouped_gemm(a, offsets, b, row_index=ri)
    check_gemm(y[:m_total], y_ref, bound, "skinny grouped %s n=%d k=%d" % (counts, n, k))
    assert np.all(np.isnan(y[m_total:])), "rows past offsets[groups] must not be written"


def test_grouped_skinny_invalid_rows_and_no_row_index():
    counts = [3, 0, 5, 2]
    groups, n, k, tokens = 4, 160, 1024, 12
    a, b = operands(977, tokens, n, k, groups)
    offsets = np.array([0, 3, 3, 8, 10], np.int32)
    ri = ((np.arange(10) * 5) % tokens).astype(np.int32)
    ri[1] = -4
    ri[6] = tokens
    y = to_np(nv.nvfp4_grouped_gemm(dev_op(a), to_dev(offsets), dev_op(b), row_index=to_dev(ri)))
    assert np.all(y[1] == 0) and np.all(y[6] == 0)
    ok = np.ones(10, bool)
    ok[[1, 6]] = False
    ri2 = ri.copy()
    ri2[~ok] = 0
    y_ref, bound = oracle.grouped_gemm(a, offsets, b, row_index=ri2)
    check_gemm(y[ok], y_ref[ok], bound[ok], "valid rows")
    # without row_index: output row i reads A row i
    y = to_np(nv.nvfp4_grouped_gemm(dev_op(a), to_dev(offsets), dev_op(b)))
    y_ref, bound = oracle.grouped_gemm(a, offsets, b, m_total=tokens)
    check_gemm(y[:10], y_ref[:10], bound[:10], "rows in place")
