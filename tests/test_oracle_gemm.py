"""Pins of the oracle's exact block-scaled GEMM (dense and grouped).

The oracle forms sum_k u_A u_B exactly in int64 (u * 2^10 is an integer) and
applies the FP32 outer scales in fp64.  Checked here against:
- a brute-force fp64 triple loop over the decoded operands on tiny shapes
  (K <= 64 keeps every partial sum exact in fp64);
- numpy's fp64 matmul of the decoded operands at non-square shapes, which
  catches a transposed operand or a swapped index;
- the hand-worked value in tests/golden/worked_rows.json (tested with the
  quantizer);
- special cases: grouped with one expert equals dense, empty experts, row
  permutation inside an expert, the row_index gather, sign flips.
"""
import numpy as np
import pytest


def _quant_pair(oracle, synth, seed, m, n, k):
    x = synth.student_t3_bf16(seed, 1, (m, k))
    w = synth.normal_bf16(seed, 2, (1, n, k), 0.0, 0.02)
    a = oracle.quantize_rows(x)
    bq, bsb, bs, _ = oracle.quantize_weight(w)
    return a, (bq[0], bsb[0], bs)


def test_brute_force_fp64_tiny(oracle, synth):
    for (m, n, k) in [(3, 5, 16), (4, 7, 32), (6, 3, 64)]:
        a, b = _quant_pair(oracle, synth, 100 + k, m, n, k)
        y, bound = oracle.gemm(a, b)
        xa = oracle.dequantize(*a)
        xb = oracle.dequantize(b[0], b[1], b[2], s_index=np.zeros(n, np.int64))
        for i in range(m):
            for j in range(n):
                acc = 0.0
                aab = 0.0
                for t in range(k):
                    acc += xa[i, t] * xb[j, t]
                    aab += abs(xa[i, t] * xb[j, t])
                assert abs(acc - y[i, j]) <= 1e-14 * aab + 1e-300
                assert abs(aab - bound[i, j]) <= 1e-14 * aab + 1e-300


def test_matches_numpy_matmul_nonsquare(oracle, synth):
    m, n, k = 37, 53, 512
    a, b = _quant_pair(oracle, synth, 7, m, n, k)
    y, bound = oracle.gemm(a, b)
    xa = oracle.dequantize(*a)
    xb = oracle.dequantize(b[0], b[1], b[2], s_index=np.zeros(n, np.int64))
    ref = xa @ xb.T
    assert np.all(np.abs(ref - y) <= 1e-12 * bound)
    assert np.allclose(np.abs(xa) @ np.abs(xb).T, bound, rtol=1e-12, atol=0)
    # a transposed or mis-indexed operand would not pass
    assert not np.all(np.abs((xa[::-1] @ xb.T) - y) <= 1e-6 * bound)


def test_entries_match_full(oracle, synth):
    m, n, k = 20, 30, 256
    a, b = _quant_pair(oracle, synth, 8, m, n, k)
    y, bound = oracle.gemm(a, b)
    ii = np.array([0, 5, 19, 7, 7])
    jj = np.array([0, 29, 3, 3, 11])
    ye, be = oracle.gemm_entries(a, b, ii, jj, np.zeros(5, np.int64))
    assert np.array_equal(ye, y[ii, jj]) and np.array_equal(be, bound[ii, jj])


def test_sign_and_zero(oracle, synth):
    m, n, k = 8, 8, 128
    a, b = _quant_pair(oracle, synth, 9, m, n, k)
    y, bound = oracle.gemm(a, b)
    an = (a[0] ^ np.uint8(0x88), a[1], a[2])
    yn, bn = oracle.gemm(an, b)
    assert np.array_equal(yn, -y) and np.array_equal(bn, bound)
    az = (a[0], a[1], np.zeros_like(a[2]))
    yz, bz = oracle.gemm(az, b)
    assert np.all(yz == 0) and np.all(bz == 0)


def _grouped_inputs(oracle, synth, seed, tokens, groups, n, k, counts=None):
    x = synth.student_t3_bf16(seed, 1, (tokens, k))
    a = oracle.quantize_rows(x)
    w = synth.normal_bf16(seed, 2, (groups, n, k), 0.0, 0.02)
    bq, bsb, bs, _ = oracle.quantize_weight(w)
    if counts is None:
        counts = (np.arange(groups) * 3) % 5
    offsets = np.zeros(groups + 1, np.int32)
    offsets[1:] = np.cumsum(counts)
    m_total = int(offsets[-1])
    row_index = (np.arange(m_total) * 7 % tokens).astype(np.int32)
    return a, (bq, bsb, bs), offsets, row_index


def test_grouped_single_expert_equals_dense(oracle, synth):
    a, b = _quant_pair(oracle, synth, 10, 24, 40, 256)
    y, bound = oracle.gemm(a, b)
    bg = (b[0][None], b[1][None], b[2])
    yg, bg_ = oracle.grouped_gemm(a, np.array([0, 24], np.int32), bg)
    assert np.array_equal(yg, y) and np.array_equal(bg_, bound)


def test_grouped_matches_per_expert_dense(oracle, synth):
    groups, n, k, tokens = 6, 24, 128, 13
    a, b, offsets, row_index = _grouped_inputs(oracle, synth, 11, tokens, groups, n, k)
    y, bound = oracle.grouped_gemm(a, offsets, b, row_index=row_index)
    for g in range(groups):
        lo, hi = offsets[g], offsets[g + 1]
        if hi == lo:
            continue
        ag = (a[0][row_index[lo:hi]], a[1][row_index[lo:hi]], a[2][row_index[lo:hi]])
        yd, bd = oracle.gemm(ag, (b[0][g], b[1][g], b[2][g:g + 1]))
        assert np.array_equal(y[lo:hi], yd) and np.array_equal(bound[lo:hi], bd)
    # an expert with no rows contributes nothing; rows past offsets[-1] stay untouched
    counts = np.diff(offsets)
    assert (counts == 0).any()
    y2, _ = oracle.grouped_gemm(a, offsets, b, row_index=row_index, m_total=int(offsets[-1]) + 3)
    assert np.all(np.isnan(y2[-3:]))


def test_grouped_row_permutation_within_expert(oracle, synth):
    groups, n, k, tokens = 3, 16, 64, 10
    a, b, offsets, row_index = _grouped_inputs(oracle, synth, 12, tokens, groups, n, k,
                                               counts=np.array([4, 5, 3]))
    y, _ = oracle.grouped_gemm(a, offsets, b, row_index=row_index)
    ri2 = row_index.copy()
    ri2[4:9] = ri2[4:9][::-1]
    y2, _ = oracle.grouped_gemm(a, offsets, b, row_index=ri2)
    assert np.array_equal(y2[4:9], y[4:9][::-1])
    assert np.array_equal(y2[:4], y[:4]) and np.array_equal(y2[9:], y[9:])


def test_grouped_without_row_index_reads_rows_in_place(oracle, synth):
    groups, n, k, tokens = 3, 16, 64, 12
    a, b, offsets, _ = _grouped_inputs(oracle, synth, 13, tokens, groups, n, k,
                                       counts=np.array([5, 0, 7]))
    y, _ = oracle.grouped_gemm(a, offsets, b)
    y2, _ = oracle.grouped_gemm(a, offsets, b, row_index=np.arange(12, dtype=np.int32))
    assert np.array_equal(y, y2)


def test_grouped_rejects_metadata_outside_its_preconditions(oracle, synth):
    """The reference reads A rows through row_index and writes the rows the
    offsets own: indices outside A, decreasing offsets or offsets past the
    output are rejected instead of read or written out of bounds."""
    import pytest
    groups, n, k, tokens = 3, 8, 64, 10
    a, b, offsets, row_index = _grouped_inputs(oracle, synth, 14, tokens, groups, n, k,
                                               counts=np.array([4, 5, 3]))
    for bad in (-1, tokens):
        ri = row_index.copy()
        ri[5] = bad
        with pytest.raises(ValueError):
            oracle.grouped_gemm(a, offsets, b, row_index=ri)
    with pytest.raises(ValueError):
        oracle.grouped_gemm(a, np.array([0, 6, 4, 12], np.int32), b, row_index=row_index)
    with pytest.raises(ValueError):
        oracle.grouped_gemm(a, offsets, b, row_index=row_index, m_total=int(offsets[-1]) - 1)
    with pytest.raises(ValueError):  # without row_index the rows read are 0..offsets[-1]-1
        oracle.grouped_gemm((a[0][:5], a[1][:5], a[2][:5]), offsets, b)


def test_acceptance_rule(oracle):
    y_ref = np.array([1.0, -2.0, 0.0])
    bound = np.array([10.0, 10.0, 0.0])
    assert oracle.gemm_within_bound(np.array([1.0 + 9e-5, -2.0, 0.0]), y_ref, bound).all()
    assert not oracle.gemm_within_bound(np.array([1.0 + 2e-4, -2.0, 0.0]), y_ref, bound)[0]
    assert not oracle.gemm_within_bound(np.array([1.0, -2.0, 1e-30]), y_ref, bound)[2]
