"""GPU tests of the grouped up-projection with SwiGLU in the epilogue
(nvfp4_grouped_gemm_swiglu): H = silu(gate) * up of the fused gate|up GEMM
output as bf16, and its row amax, without the fp32 output in between
(fusion and amax reuse, miniTE page, section Transformer Engine路径优化;
the fused gate|up weight, Miles page, section 并行度与张量转换的一致性契约).

- Oracle pin: operands whose fp32 sums are exact (unit block and outer
  scales: every product is a multiple of 1/4 below 37 and every partial sum
  fits 24 bits), so the GEMM output is the oracle's exact one and H and the
  amax must equal the oracle's SwiGLU of it bit for bit, and the requantize
  with amax reuse the oracle's quantizer.
- Chain: on real-scaled data the fused H and amax equal, bit for bit, the
  unfused chain on the GPU (the tiled grouped GEMM's fp32 output, then the
  SwiGLU kernel), also at the full MoE up-projection size.
- Gathered and invalid rows, rows past offsets[groups], ragged f, errors.
"""
import numpy as np
import pytest
import torch

import nvfp4_token_quantization_amd as nv
import oracle
import synthgen as sg
from gpu_helpers import assert_same_quant, dev, to_dev, to_np, workload

pytestmark = pytest.mark.gpu


def bf16_bits(t):
    return to_np(t.view(torch.int16)).view(np.uint16)


def unit_scale_operand(seed, shape_rows, k):
    """Random E2M1 codes with every block scale 1.0 (E4M3 0x38) and S = 1."""
    n = int(np.prod(shape_rows))
    q = (sg.uniform(seed, sg.S_MISC, n * (k // 2)) * 256).astype(np.uint8).reshape(*shape_rows, k // 2)
    sb = np.full(tuple(shape_rows) + (k // 16,), 0x38, np.uint8)
    return q, sb


def layout(counts, tokens, seed):
    off = np.zeros(len(counts) + 1, np.int32)
    off[1:] = np.cumsum(counts)
    m_total = int(off[-1])
    ri = ((np.arange(m_total) * 7 + seed) % tokens).astype(np.int32)
    return off, ri, m_total


@pytest.mark.parametrize("counts,f,k", [
    ([40, 0, 200, 3, 130, 1], 96, 512),      # ragged experts, f = 1.5 column tiles
    ([300, 260], 768, 2048),                 # the MoE shape's f and k
    ([129, 0, 0, 64], 33, 256),              # f below one tile (H and amax only)
    ([17] * 12, 200, 768),                   # f not a multiple of 16 (H and amax only)
])
def test_fused_swiglu_exact_sums_match_oracle(counts, f, k):
    groups, tokens = len(counts), 97
    off, ri, m_total = layout(counts, tokens, 3)
    aq, asb = unit_scale_operand(11 + f, (tokens,), k)
    bq, bsb = unit_scale_operand(12 + f, (groups, 2 * f), k)
    a = (aq, asb, np.ones(tokens, np.float32))
    b = (bq, bsb, np.ones(groups, np.float32))
    y_ref, _ = oracle.grouped_gemm(a, off, b, row_index=ri)
    y32 = y_ref.astype(np.float32)
    assert np.array_equal(y32.astype(np.float64), y_ref), "operands must give fp32-exact sums"
    h_ref = oracle.swiglu_rows(y32)
    amax_ref = np.abs((h_ref.astype(np.uint32) << 16).view(np.float32)).max(axis=1).astype(np.float32)
    h, amax = nv.nvfp4_grouped_gemm_swiglu(tuple(to_dev(t) for t in a), to_dev(off),
                                           tuple(to_dev(t) for t in b), row_index=to_dev(ri))
    got = bf16_bits(h)
    if not np.array_equal(got, h_ref):
        bad = np.argwhere(got != h_ref)
        i = tuple(bad[0])
        raise AssertionError("%d H mismatches, first %s: got %#x want %#x (g=%r u=%r)" % (
            len(bad), i, got[i], h_ref[i], y32[i[0], i[1]], y32[i[0], f + i[1]]))
    assert np.array_equal(to_np(amax).view(np.uint32), amax_ref.view(np.uint32))
    if f % 16 == 0:  # the quantizer's block size
        q, sb, s = nv.nvfp4_quantize_rows(h, amax_in=amax)
        assert_same_quant((q, sb, s), oracle.quantize_rows(h_ref), "requantize of the fused H")


def real_operands(seed, tokens, groups, f, k):
    a = oracle.quantize_rows(sg.student_t3_bf16(seed, 1, (tokens, k)))
    w = sg.normal_bf16(seed, 2, (groups, 2 * f, k), 0.0, 0.02)
    b = oracle.quantize_weight(w)[:3]
    return tuple(to_dev(t) for t in a), tuple(to_dev(t) for t in b)


def unfused_chain(a, off, b, ri, m_total):
    y = nv.nvfp4_grouped_gemm(a, off, b, row_index=ri, m_total=m_total)
    r = nv.nvfp4_swiglu_quantize_rows(y, want_h=True, want_amax=True)
    return y, r


@pytest.mark.parametrize("counts,f,k", [
    ([100, 0, 37, 512, 2, 65], 768, 2048),
    ([300, 5, 250], 144, 256),
    ([200] * 8, 1008, 1280),
])
def test_fused_swiglu_equals_unfused_chain(counts, f, k):
    groups, tokens = len(counts), 211
    off, ri, m_total = layout(counts, tokens, 5)
    # more than 16 routed rows per expert on average: the unfused GEMM takes
    # the tiled kernel, whose sums the fused epilogue shares
    assert m_total > 16 * groups
    a, b = real_operands(700 + f, tokens, groups, f, k)
    off_d, ri_d = to_dev(off), to_dev(ri)
    y, r = unfused_chain(a, off_d, b, ri_d, m_total)
    h, amax = nv.nvfp4_grouped_gemm_swiglu(a, off_d, b, row_index=ri_d)
    assert torch.equal(h.view(torch.int16), r["h"].view(torch.int16))
    assert torch.equal(amax.view(torch.int32), r["amax"].view(torch.int32))


def test_fused_swiglu_full_moe_up_projection():
    """4096 tokens, top-8 of 128 experts (Zipf-routed), fused gate|up
    1536 x 2048: the fused H and amax equal the unfused chain everywhere, and
    the requantize with the fused amax equals the SwiGLU kernel's codes."""
    d = workload(3, "x,w")
    route = oracle.route(workload(3, "logits")["logits"], 8)
    x = nv.nvfp4_quantize_rows(to_dev(d["x"]))
    w = nv.nvfp4_quantize_weight(to_dev(d["w"]))[:3]
    off, ri = to_dev(route["offsets"]), to_dev(route["row_index"])
    m_total = int(route["offsets"][-1])
    y, r = unfused_chain(x, off, w, ri, m_total)
    h, amax = nv.nvfp4_grouped_gemm_swiglu(x, off, w, row_index=ri)
    assert torch.equal(h.view(torch.int16), r["h"].view(torch.int16))
    assert torch.equal(amax.view(torch.int32), r["amax"].view(torch.int32))
    q, sb, s = nv.nvfp4_quantize_rows(h, amax_in=amax)
    assert torch.equal(q, r["q"]) and torch.equal(sb, r["sb"]) and torch.equal(s, r["s"])


def test_fused_swiglu_invalid_rows_and_rows_past_offsets():
    counts, f, k, tokens = [30, 0, 41], 80, 256, 19
    groups = len(counts)
    off, ri, m_total = layout(counts, tokens, 1)
    ri[4] = -1
    ri[50] = tokens
    aq, asb = unit_scale_operand(31, (tokens,), k)
    bq, bsb = unit_scale_operand(32, (groups, 2 * f), k)
    a = (aq, asb, np.ones(tokens, np.float32))
    b = (bq, bsb, np.ones(groups, np.float32))
    rows = m_total + 5
    h = torch.full((rows, f), float("nan"), dtype=torch.bfloat16, device=dev())
    amax = torch.full((rows,), 7.0, device=dev())
    ri_full = np.concatenate([ri, np.zeros(5, np.int32)])
    nv.nvfp4_grouped_gemm_swiglu(tuple(to_dev(t) for t in a), to_dev(off), tuple(to_dev(t) for t in b),
                                 row_index=to_dev(ri_full), m_total=rows, out=(h, amax))
    hn = bf16_bits(h)
    am = to_np(amax)
    assert np.all(hn[[4, 50]] == 0) and np.all(am[[4, 50]] == 0)
    assert np.all(np.isnan(to_np(h.float())[m_total:])), "rows past offsets[groups] must not be written"
    assert np.all(am[m_total:] == 0)
    ok = np.ones(m_total, bool)
    ok[[4, 50]] = False
    ri_ok = np.where(ok, ri, 0).astype(np.int32)
    y_ref, _ = oracle.grouped_gemm(a, off, b, row_index=ri_ok)
    h_ref = oracle.swiglu_rows(y_ref.astype(np.float32))
    assert np.array_equal(hn[:m_total][ok], h_ref[ok])


def test_fused_swiglu_argument_errors():
    d = dev()
    a = (torch.zeros((4, 64), dtype=torch.uint8, device=d), torch.zeros((4, 8), dtype=torch.uint8, device=d),
         torch.ones(4, device=d))
    b = (torch.zeros((1, 6, 64), dtype=torch.uint8, device=d), torch.zeros((1, 6, 8), dtype=torch.uint8, device=d),
         torch.ones(1, device=d))
    off = torch.tensor([0, 4], dtype=torch.int32, device=d)
    with pytest.raises(nv.NVFP4Error):          # k = 128 is not a multiple of 256
        nv.nvfp4_grouped_gemm_swiglu(a, off, b)
    b_odd = (b[0][:, :5].contiguous(), b[1][:, :5].contiguous(), b[2])
    with pytest.raises(ValueError):
        nv.nvfp4_grouped_gemm_swiglu(a, off, b_odd)
