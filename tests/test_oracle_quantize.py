"""Pins of the oracle's quantizer (per-token rows and per-tensor / per-expert
weights) against things other than itself:

- rows worked by hand from the contract (tests/golden/worked_rows.json);
- an exhaustive round trip: every (E4M3 scale code, E2M1 code) pair, placed
  on the grid, must quantize back to itself (idempotence on the grid);
- closed-form error bounds: the decoded value is the nearest grid point of
  its block, and the block scale the nearest E4M3 value of a_b / (6 S);
- invariants the pages ask for: a token's bits do not depend on the other
  tokens in the batch (miniTE report, section 激活精度、缩放粒度与KV Cache;
  Miles page, section 单Token激活缩放的必要性), amax reuse reproduces the same
  bits, gate/up share one outer scale (Miles page, section
  并行度与张量转换的一致性契约); plus power-of-two scaling, negation and block
  permutation equivariance.
"""
import json
import os

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _unpack(q):
    lo = q & 15
    hi = q >> 4
    return np.stack([lo, hi], axis=-1).reshape(q.shape[:-1] + (q.shape[-1] * 2,))


def test_worked_rows(oracle, synth):
    doc = json.load(open(os.path.join(GOLDEN, "worked_rows.json")))
    for case in doc["cases"]:
        x = synth.f32_to_bf16(np.array(case["x"], np.float32)).reshape(1, -1)
        assert np.array_equal(synth.bf16_to_f32(x).ravel(), np.array(case["x"], np.float32))
        q, sb, s = oracle.quantize_rows(x)
        assert q.tobytes().hex() == case["q_hex"], case["name"]
        assert sb.tobytes().hex() == case["sb_hex"], case["name"]
        assert s[0] == np.float32(case["s"]), case["name"]
    # the hand-worked GEMM value of the first row with itself
    x = synth.f32_to_bf16(np.array(doc["cases"][0]["x"], np.float32)).reshape(1, -1)
    q, sb, s = oracle.quantize_rows(x)
    y, bound = oracle.gemm((q, sb, s), (q, sb, np.array([s[0]], np.float32)))
    assert y[0, 0] == doc["gemm"]["y"]


def test_maxes_row(oracle, synth):
    """The 'maxes' class: a row of the largest finite bf16 gives the largest
    block scale and the largest element code, and S = fl32(amax / 2688)."""
    x = np.full((1, 32), 0x7F7F, np.uint16)
    x[0, 1::2] = 0xFF7F   # alternate signs
    q, sb, s = oracle.quantize_rows(x)
    amax = synth.bf16_to_f32(np.array([0x7F7F], np.uint16))[0]
    assert s[0] == np.float32(amax) / np.float32(2688.0)
    assert np.all(sb == 0x7E)
    assert np.all(q == 0xF7)


@pytest.mark.parametrize("k2", [0, -40, 40, -100])
def test_round_trip_all_scale_and_element_codes(oracle, synth, k2):
    """For every finite non-negative E4M3 code c and every E2M1 code q, a row
    holding an anchor block (amax = 2688 * 2^k2, so S = 2^k2 exactly) and a
    block of values 2^k2 * s_b(c) * e2m1(q) for all 16 q must quantize back to
    scale code c and element codes q.  The ratio a_b / (6 S) is exactly s_b(c)
    and x * fl32(1/d) lies within one ulp of the grid value, so any slip in the
    tables, the scale arithmetic, the sign or the nibble order shows up."""
    e2 = oracle.e2m1_table()
    e4 = oracle.e4m3_table()
    rows = []
    codes = []
    for c in range(0x7F):
        d = (2.0 ** k2) * e4[c]
        blk = [d * e2[qq] for qq in range(16)]
        rows.append([2688.0 * 2.0 ** k2] + [0.0] * 15 + blk)
        codes.append(c)
    xf = np.array(rows, np.float64)
    x = synth.f32_to_bf16(xf.astype(np.float32))
    assert np.array_equal(synth.bf16_to_f32(x).astype(np.float64), xf)  # all exact in bf16
    q, sb, s = oracle.quantize_rows(x)
    assert np.all(s == np.float32(2.0 ** k2))
    assert np.all(sb[:, 0] == 0x7E)
    for r, c in enumerate(codes):
        if c == 0:
            # s_b = 0: the block is all (signed) zeros and stays so
            assert sb[r, 1] == 0
            assert np.array_equal(_unpack(q[r:r + 1])[0, 16:], np.array([0] * 8 + [8] * 8, np.uint8))
            continue
        assert sb[r, 1] == c, (c, sb[r, 1])
        assert np.array_equal(_unpack(q[r:r + 1])[0, 16:], np.arange(16, dtype=np.uint8)), c
        # and decoding gives back the values (S * s_b * Q per the decode formula)
        xh = oracle.dequantize(q[r:r + 1], sb[r:r + 1], s[r:r + 1])
        assert np.array_equal(xh[0], xf[r])


def _random_rows(synth, seed, rows, k):
    x = synth.student_t3_bf16(seed, 1, (rows, k))
    return x


def test_decoded_value_is_nearest_grid_point(oracle, synth):
    """Closed-form bound: with d = S * s_b, the decoded value e2m1(q) * d is the
    grid point nearest x / d (up to the one rounding of x * fl32(1/d)), unless
    |x| / d is past the largest magnitude 6, where it saturates."""
    x = _random_rows(synth, 21, 256, 1024)
    q, sb, s = oracle.quantize_rows(x)
    xf = synth.bf16_to_f32(x).astype(np.float64)
    xh = oracle.dequantize(q, sb, s)
    e4 = oracle.e4m3_table()
    d = s[:, None].astype(np.float64) * e4[sb.astype(int)].repeat(16, axis=1)
    r = np.abs(xf) / np.where(d > 0, d, 1.0)
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    dist = np.abs(r[..., None] - grid[None, None, :])
    best = dist.min(axis=-1)
    got = np.abs(np.abs(xh) / np.where(d > 0, d, 1.0) - r)
    live = d > 0
    assert live.mean() > 0.99
    sat = (r > 6.0) & live
    fine = (~sat) & live
    slack = 4.0 * 2.0 ** -24 * np.maximum(r, 1.0)
    assert np.all(got[fine] <= best[fine] + slack[fine])
    assert np.all(np.abs(xh[sat]) == 6.0 * d[sat])
    assert np.all(xh[~live] == 0)
    # signs follow x (zeros aside)
    nz = xh != 0
    assert np.all(np.sign(xh[nz]) == np.sign(xf[nz]))


def test_block_scale_is_nearest_e4m3(oracle, synth):
    """s_b is the E4M3 value nearest a_b / (6 S) (the rounding the Miles page's
    NVFP4 background section states), to within the one rounding of that fp32
    quotient; the row's largest block gets s_b = 448."""
    x = _random_rows(synth, 22, 128, 2048)
    q, sb, s = oracle.quantize_rows(x)
    xf = np.abs(synth.bf16_to_f32(x).astype(np.float64)).reshape(128, -1, 16)
    ab = xf.max(axis=-1)
    ratio = ab / (6.0 * s[:, None].astype(np.float64))
    e4 = oracle.e4m3_table()[:0x7F]
    sbv = e4[sb.astype(int)]
    nearest = np.abs(ratio[..., None] - e4[None, None, :]).min(axis=-1)
    assert np.all(np.abs(sbv - ratio) <= nearest + 1e-6 * ratio)
    assert np.all(sb.max(axis=1) == 0x7E)


def test_batch_invariance(oracle, synth):
    """A token's bits do not depend on which other tokens share the batch."""
    x = _random_rows(synth, 23, 200, 768)
    q, sb, s = oracle.quantize_rows(x)
    rng_idx = [np.array([7]), np.arange(0, 200, 3), np.array([199, 0, 57, 3]),
               np.argsort(synth.uniform(23, 9, 200))[:64]]
    for idx in rng_idx:
        q2, sb2, s2 = oracle.quantize_rows(x[idx])
        assert np.array_equal(q2, q[idx]) and np.array_equal(sb2, sb[idx])
        assert np.array_equal(s2.view(np.uint32), s[idx].view(np.uint32))


def test_amax_reuse_equals_recompute(oracle, synth):
    x = _random_rows(synth, 24, 300, 768)
    amax = synth.row_amax_bf16(x)
    a = oracle.quantize_rows(x)
    b = oracle.quantize_rows(x, amax_in=amax)
    for u, v in zip(a, b):
        assert np.array_equal(np.asarray(u).view(np.uint8), np.asarray(v).view(np.uint8))


def test_power_of_two_equivariance(oracle, synth):
    """Scaling the inputs by 2^j (no over/underflow) keeps q and s_b and
    scales S by exactly 2^j."""
    x = _random_rows(synth, 25, 64, 512)
    xf = synth.bf16_to_f32(x)
    q, sb, s = oracle.quantize_rows(x)
    for j in (-20, -3, 5, 30):
        x2 = synth.f32_to_bf16(xf * np.float32(2.0 ** j))
        assert np.array_equal(synth.bf16_to_f32(x2), xf * np.float32(2.0 ** j))
        q2, sb2, s2 = oracle.quantize_rows(x2)
        assert np.array_equal(q2, q) and np.array_equal(sb2, sb)
        assert np.array_equal(s2, s * np.float32(2.0 ** j))


def test_negation_flips_only_sign_bits(oracle, synth):
    x = _random_rows(synth, 26, 64, 512)
    q, sb, s = oracle.quantize_rows(x)
    qn, sbn, sn = oracle.quantize_rows(x ^ np.uint16(0x8000))
    assert np.array_equal(sbn, sb) and np.array_equal(sn, s)
    assert np.array_equal(qn, q ^ np.uint8(0x88))


def test_block_permutation(oracle, synth):
    x = _random_rows(synth, 27, 32, 512)
    q, sb, s = oracle.quantize_rows(x)
    perm = np.argsort(synth.uniform(27, 5, 32))
    xp = x.reshape(32, 32, 16)[:, perm, :].reshape(32, 512)
    qp, sbp, sp = oracle.quantize_rows(xp)
    assert np.array_equal(sbp, sb[:, perm]) and np.array_equal(sp, s)
    assert np.array_equal(qp.reshape(32, 32, 8), q.reshape(32, 32, 8)[:, perm, :])


def test_weight_is_rows_with_fixed_scale(oracle, synth):
    """Weights: per-expert equals per-tensor on the expert's slice; a group is
    its rows quantized with the group's amax supplied as every row's amax;
    a one-row weight equals the per-token quantization of that row; gate and
    up fused in one group share one outer scale."""
    w = synth.normal_bf16(31, 2, (4, 48, 256), 0.0, 0.02)
    q, sb, s, amax = oracle.quantize_weight(w)
    for g in range(4):
        qg, sbg, sg, ag = oracle.quantize_weight(w[g:g + 1])
        assert np.array_equal(qg[0], q[g]) and np.array_equal(sbg[0], sb[g]) and sg[0] == s[g]
        qr, sbr, sr = oracle.quantize_rows(w[g], amax_in=np.full((48,), amax[g], np.float32))
        assert np.array_equal(qr, q[g]) and np.array_equal(sbr, sb[g]) and np.all(sr == s[g])
        assert amax[g] == np.abs(synth.bf16_to_f32(w[g])).max()
    q1, sb1, s1, a1 = oracle.quantize_weight(w[:1, :1])
    qt, sbt, st = oracle.quantize_rows(w[0, :1])
    assert np.array_equal(q1[0], qt) and np.array_equal(sb1[0], sbt) and s1[0] == st[0]
    # fused gate+up: one group over both halves -> one scale from the joint amax
    gate, up = w[0, :24], w[1, :24]
    fused = np.concatenate([gate, up], axis=0)[None]
    qf, sbf, sf, af = oracle.quantize_weight(fused)
    assert af[0] == max(np.abs(synth.bf16_to_f32(gate)).max(), np.abs(synth.bf16_to_f32(up)).max())
    assert sf.shape == (1,)


def test_rejects_nonfinite_and_bad_k(oracle):
    x = np.zeros((2, 32), np.uint16)
    x[1, 5] = 0x7F80   # +inf
    with pytest.raises(ValueError):
        oracle.quantize_rows(x)
    with pytest.raises(ValueError):
        oracle.quantize_rows(np.zeros((2, 24), np.uint16))
