"""GPU parity of NVFP4 -> bf16 dequantization (dequantized-backward mode,
Miles page, section 反量化反向模式) against the oracle: every bf16 output bit
must match (one exact rounding of S * s_b * e2m1(q))."""
import numpy as np
import pytest
import torch

import nvfp4_token_quantization_amd as nv
import oracle
import synthgen as sg
from gpu_helpers import dev, oracle_rows, oracle_weight, to_dev, to_np

pytestmark = pytest.mark.gpu


def bf16_bits(t):
    return to_np(t.view(torch.int16)).view(np.uint16)


def check(q, sb, s, rows_per_scale=1, what=""):
    got = bf16_bits(nv.nvfp4_dequantize_rows(to_dev(q), to_dev(sb), to_dev(s), rows_per_scale))
    torch.cuda.synchronize()
    want = oracle.dequantize_bf16(q.reshape(-1, q.shape[-1]), sb.reshape(-1, sb.shape[-1]), s,
                                  rows_per_scale).reshape(got.shape)
    if not np.array_equal(got, want):
        bad = np.argwhere(got != want)
        i = tuple(bad[0])
        raise AssertionError("%s: %d mismatches, first at %s (got %#x want %#x)" % (
            what, len(bad), i, got[i], want[i]))


@pytest.mark.parametrize("rows,k", [(1, 16), (7, 48), (64, 2560), (300, 768), (33, 4112)])
def test_dequantize_random_rows(rows, k):
    x = sg.student_t3_bf16(700 + rows, sg.S_X, (rows, k))
    q, sb, s = oracle.quantize_rows(x)
    check(q, sb, s, what="rows=%d k=%d" % (rows, k))


# One K per dequantize layout (16, 32 or 64 lanes per row x 1 to 8
# half-blocks per lane where the half-blocks divide evenly; the general
# kernel for the rest), the general kernel also at small, odd and large K.
DEQ_LAYOUT_K = [16, 128, 384, 640, 144, 256, 768, 1280, 512, 1024, 1536, 2048, 2560, 3072,
                272, 400, 4096, 4112, 8192, 12304]


@pytest.mark.parametrize("k", DEQ_LAYOUT_K)
def test_dequantize_every_layout(k):
    """130 rows (partial row groups in the last block), each scaled by its own
    power of two from 2^-40 to 2^40 before quantizing; per-token scales, and
    one outer scale per 13 rows (the weight form)."""
    rows = 130
    x = sg.bf16_to_f32(sg.student_t3_bf16(5000 + k, sg.S_X, (rows, k)))
    e = (sg.uniform(5000 + k, 2, rows) * 81).astype(np.int64) - 40
    x = sg.f32_to_bf16(x * np.exp2(e.astype(np.float32))[:, None])
    q, sb, s = oracle.quantize_rows(x)
    check(q, sb, s, what="k=%d" % k)
    w = oracle.quantize_weight(x.reshape(10, 13, k))
    check(w[0], w[1], w[2], rows_per_scale=13, what="weight k=%d" % k)


def test_dequantize_every_scale_and_code():
    """All 127 finite block-scale codes x all 16 element codes, under outer
    scales with few significant bits (frequent ties), ordinary ones, tiny
    ones (subnormal bf16 results) and huge ones."""
    codes = np.arange(256, dtype=np.uint8)                 # every byte = every nibble pair
    scales = [1.0, 1.00390625, 1.0 + 2 ** -9 + 2 ** -12, 0.7071067, 3.1e-41, 2.0 ** -140,
              1.2e-38, 5.0e35, 1.2e38, 0.0]
    rows = len(scales)
    k = 127 * 16
    q = np.empty((rows, k // 2), np.uint8)
    for r in range(rows):
        q[r] = np.roll(np.tile(codes, 4)[: k // 2], 13 * r)
    sb = np.tile(np.arange(127, dtype=np.uint8), (rows, 1))
    s = np.array(scales, np.float32)
    check(q, sb, s, what="exhaustive codes")


def test_dequantize_fp32_halfway_cases():
    """Outer scales for which 1.5 * S rounds in fp32 exactly onto a bf16
    halfway point: the kernel's correction branch decides these."""
    from test_oracle_dequant import fp32_tie_scales
    s = fp32_tie_scales(512)
    rows = len(s)
    q = np.tile(np.array([0x33, 0xBB, 0x53, 0x3B, 0x35, 0x73, 0xB3, 0x37], np.uint8), (rows, 1))
    sb = np.full((rows, 1), 0x38, np.uint8)
    check(q, sb, s, what="fp32 halfway cases")


def test_dequantize_tie_heavy_scales():
    q, sb, s = oracle_rows(2, "x")
    s = (s.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32).copy()  # 8 significant bits
    check(q[:512], sb[:512], s[:512], what="8-bit outer scales")


def test_dequantize_full_dense_activation():
    q, sb, s = oracle_rows(2, "x")
    check(q, sb, s, what="X 4096x2560")


def test_dequantize_full_moe_down_input():
    q, sb, s = oracle_rows(4, "h", True)
    check(q, sb, s, what="H 32768x768")


def test_dequantize_weights_per_tensor_and_per_expert():
    wq, wsb, ws, _ = oracle_weight(2, "w")
    check(wq[0], wsb[0], ws, rows_per_scale=wq.shape[1], what="W 9728x2560 per tensor")
    w = sg.normal_bf16(77, sg.S_W, (8, 96, 256), 0.0, 0.02)
    q, sb, s, _ = oracle.quantize_weight(w)
    check(q, sb, s, rows_per_scale=96, what="8 experts 96x256")


def test_dequantize_matches_quantizer_round_trip_on_gpu():
    """Quantize on the GPU, dequantize on the GPU: equals the oracle's
    dequantization of the oracle's codes (the codes being identical)."""
    x = sg.student_t3_bf16(91, sg.S_X, (256, 2048))
    q, sb, s = nv.nvfp4_quantize_rows(to_dev(x))
    got = bf16_bits(nv.nvfp4_dequantize_rows(q, sb, s))
    torch.cuda.synchronize()
    oq, osb, os_ = oracle.quantize_rows(x)
    assert np.array_equal(got, oracle.dequantize_bf16(oq, osb, os_))


def test_dequantize_empty():
    d = dev()
    out = nv.nvfp4_dequantize_rows(torch.zeros((0, 8), dtype=torch.uint8, device=d),
                                   torch.zeros((0, 1), dtype=torch.uint8, device=d),
                                   torch.zeros((1,), dtype=torch.float32, device=d))
    assert out.shape == (0, 16)
