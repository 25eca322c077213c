"""GPU parity of the fused SwiGLU -> per-token NVFP4 kernel against the oracle.

The chain is the pages' amax reuse plus fusion (miniTE page, section
Transformer Engine路径优化) applied to the MoE layers' fused gate|up output
(Miles page, section 并行度与张量转换的一致性契约).  H's bf16 bits, its row
amax and the NVFP4 codes, block scales and outer scales are compared bit for
bit.  Inputs are synthetic fp32 gate|up blocks (Student-t tails like GEMM
outputs), and for the chained variant the oracle's own exact grouped-GEMM
output of the rollout-decode workload rounded to fp32.
"""
import numpy as np
import pytest
import torch

import nvfp4_token_quantization_amd as nv
import oracle
import synthgen as sg
from gpu_helpers import assert_same_quant, dev, oracle_weight, routing, to_dev, to_np, workload

pytestmark = pytest.mark.gpu


def gate_up_input(rows, f, seed, gstd=2.0, ustd=1.0):
    """fp32 [rows, 2f]: gate N(0, gstd) and up N(0, ustd) with 1% of entries
    times 20 (heavy tails, like the output of a GEMM over t3 activations)."""
    n = rows * 2 * f
    z = sg.normal(seed, sg.S_MISC, n).reshape(rows, 2 * f)
    spike = sg.uniform(seed, sg.S_MISC + 100, n).reshape(rows, 2 * f) < 0.01
    z = np.where(spike, z * 20.0, z)
    z[:, :f] *= gstd
    z[:, f:] *= ustd
    return z.astype(np.float32)


def h_bits(t):
    return to_np(t.view(torch.int16)).view(np.uint16)


def run_all(gu):
    r = nv.nvfp4_swiglu_quantize_rows(to_dev(gu), want_h=True, want_amax=True)
    torch.cuda.synchronize()
    return r


def check_against_oracle(gu, r, what):
    h, amax, q, sb, s = oracle.swiglu_quantize_rows(gu)
    got_h = h_bits(r["h"])
    if not np.array_equal(got_h, h):
        bad = np.argwhere(got_h != h)
        i = tuple(bad[0])
        raise AssertionError("%s h: %d mismatches, first at %s (got %#x want %#x; g=%r u=%r)" % (
            what, len(bad), i, got_h[i], h[i], gu[i[0], i[1]], gu[i[0], gu.shape[1] // 2 + i[1]]))
    assert_same_quant((r["q"], r["sb"], r["s"], r["amax"]), (q, sb, s, amax), what)


@pytest.mark.parametrize("rows,f", [(1, 16), (5, 48), (64, 256), (33, 768), (7, 1040), (16, 2048),
                                    (9, 2064), (4, 4096), (3, 9728), (2, 12288),
                                    # the other kernel sizes: one wave per row (256 columns a
                                    # step) up to 2048, four waves per row (1024 a step) above
                                    (6, 512), (5, 528), (4, 1024), (3, 1536), (3, 1792),
                                    (5, 5120), (3, 6144), (2, 7168), (3, 8192), (2, 9216), (2, 11264)])
def test_swiglu_quantize_matches_oracle(rows, f):
    gu = gate_up_input(rows, f, seed=1000 + f + rows)
    check_against_oracle(gu, run_all(gu), "rows=%d f=%d" % (rows, f))


@pytest.mark.parametrize("gstd,ustd", [(0.05, 0.05), (8.0, 3.0), (60.0, 1e-3)])
def test_swiglu_magnitude_ranges(gstd, ustd):
    gu = gate_up_input(96, 768, seed=77, gstd=gstd, ustd=ustd)
    check_against_oracle(gu, run_all(gu), "gstd=%g ustd=%g" % (gstd, ustd))


def test_swiglu_wide_range_and_thresholds():
    """The kernel evaluates most elements in fp32 and re-evaluates in fp64
    those whose fp32 result lies near a bf16 rounding boundary, below 2^-100,
    or whose gate is below -80; exp(-g) is skipped for g >= 20.  Gates span
    [-90, 30] (across both thresholds, plus a dense grid around each) and up
    magnitudes 2^-120 .. 2^100, so results cover tiny, denormal and huge
    values, and some 1 in 2000 fall inside the rounding test's window."""
    rows, f = 128, 1024
    n = rows * f
    g = sg.uniform(11, sg.S_MISC, n) * 120.0 - 90.0
    g[:4096] = np.linspace(-80.01, -79.99, 4096)
    g[4096:8192] = np.linspace(19.99, 20.01, 4096)
    e = np.floor(sg.uniform(12, sg.S_MISC, n) * 220.0) - 120.0
    u = np.ldexp(sg.uniform(13, sg.S_MISC, n) + 0.5, e.astype(np.int64))
    u = np.where(sg.uniform(14, sg.S_MISC, n) < 0.5, -u, u)
    gu = np.concatenate([g.reshape(rows, f), u.reshape(rows, f)], axis=1).astype(np.float32)
    check_against_oracle(gu, run_all(gu), "wide range")


def test_swiglu_zero_and_special_rows():
    rows, f = 6, 256
    gu = gate_up_input(rows, f, seed=5)
    gu[0] = 0.0                      # H = 0: S = 0, every code 0
    gu[1, f:] = 0.0                  # up = 0 -> signed zeros
    gu[2, :f] = -2000.0              # sigmoid underflows: signed zeros
    gu[3, :f] = 50.0                 # sigmoid == 1: H = bf16(g * u)
    gu[4, :16] = 0.0                 # one all-zero block
    gu[4, f:f + 16] = 0.0
    gu[5, :f] = -0.0
    check_against_oracle(gu, run_all(gu), "special rows")


def test_swiglu_output_subsets():
    gu = gate_up_input(40, 768, seed=9)
    full = run_all(gu)
    gd = to_dev(gu)
    only_q = nv.nvfp4_swiglu_quantize_rows(gd)
    only_h = nv.nvfp4_swiglu_quantize_rows(gd, want_h=True, quantize=False)
    only_a = nv.nvfp4_swiglu_quantize_rows(gd, want_amax=True, quantize=False)
    torch.cuda.synchronize()
    for key in ("q", "sb", "s"):
        assert torch.equal(only_q[key], full[key]), key
    assert torch.equal(only_h["h"].view(torch.int16), full["h"].view(torch.int16))
    assert torch.equal(only_a["amax"], full["amax"])


def test_swiglu_matches_two_kernel_chain():
    """Fused kernel == producer (H, amax) then the per-token quantizer with
    amax_in, and == the quantizer computing the amax itself."""
    gu = gate_up_input(300, 768, seed=21)
    full = run_all(gu)
    q1, sb1, s1 = nv.nvfp4_quantize_rows(full["h"], amax_in=full["amax"])
    q2, sb2, s2 = nv.nvfp4_quantize_rows(full["h"])
    torch.cuda.synchronize()
    for a, b, c in ((full["q"], q1, q2), (full["sb"], sb1, sb2), (full["s"], s1, s2)):
        assert torch.equal(a, b) and torch.equal(a, c)


def test_swiglu_empty_and_errors():
    d = dev()
    gu = torch.zeros((0, 64), dtype=torch.float32, device=d)
    r = nv.nvfp4_swiglu_quantize_rows(gu, want_h=True, want_amax=True)
    assert r["q"].shape == (0, 16)
    gu = torch.zeros((3, 0), dtype=torch.float32, device=d)
    r = nv.nvfp4_swiglu_quantize_rows(gu, want_amax=True)
    torch.cuda.synchronize()
    assert to_np(r["s"]).tolist() == [0.0, 0.0, 0.0] and to_np(r["amax"]).tolist() == [0.0] * 3
    with pytest.raises(nv.NVFP4Error):
        nv.nvfp4_swiglu_quantize_rows(torch.zeros((2, 40), dtype=torch.float32, device=d))
    with pytest.raises(nv.NVFP4Error):
        nv.nvfp4_swiglu_quantize_rows(torch.zeros((2, 2 * 12304), dtype=torch.float32, device=d))


def test_swiglu_batch_invariance():
    gu = gate_up_input(64, 768, seed=31)
    full = run_all(gu)
    for idx in ([0], [17, 3, 63], list(range(1, 64, 2))):
        part = run_all(np.ascontiguousarray(gu[idx]))
        for key in ("h", "amax", "q", "sb", "s"):
            a = full[key][idx]
            b = part[key]
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), (key, idx)


def test_swiglu_moe_down_shape_full_size():
    """The MoE down-projection input at its full size: 32768 routed rows,
    f = 768 (gate|up 1536 columns), every output compared."""
    gu = gate_up_input(32768, 768, seed=sg.config_seed(4))
    check_against_oracle(gu, run_all(gu), "32768x768")


def test_swiglu_chained_rollout_decode():
    """Chained variant on the rollout-decode workload: the oracle's exact
    grouped up-projection of the 64 tokens (512 routed rows, fused gate|up
    weight 128 x 1536 x 2048) rounded to fp32 feeds the fused kernel."""
    d = workload(5, "x")
    xq = oracle.quantize_rows(d["x"])
    wq, wsb, ws, _ = oracle_weight(5, "w")
    rt = routing(5)
    y, _ = oracle.grouped_gemm(xq, rt["offsets"], (wq, wsb, ws), row_index=rt["row_index"])
    gu = y.astype(np.float32)
    check_against_oracle(gu, run_all(gu), "chained rollout decode")
