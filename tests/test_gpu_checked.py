"""GPU tests of the checked build, libnvfp4_checked.so: the same library with
the device-side preconditions validated on the call's stream before any of
its work (finite bf16 / f32 inputs, supplied amax and scales; a supplied
amax >= 0; no NaN E4M3 or E8M0 scale codes, nor NaN E4M3 element codes in
MXFP8 operands; non-decreasing offsets).

- On valid inputs every entry point of the checked build writes the same
  bits as the product library (the same kernels run after the checks).
- Each violation returns NVFP4_ERROR_PRECONDITION and leaves the outputs as
  they were (nothing else is launched), including a violation in the last
  element of a tensor that takes the check kernels' full grid-stride loop.
- A valid call after a rejected one succeeds (the violation flag is
  cleared per call).
"""
import numpy as np
import pytest
import torch

import nvfp4_token_quantization_amd as nv
import synthgen as sg
from gpu_helpers import to_dev

pytestmark = pytest.mark.gpu

NAN_BF16, INF_BF16 = 0x7FC0, 0x7F80
SENTINEL = 0xA5


@pytest.fixture
def use():
    """use("checked") or use("product") routes the binding through that build;
    the binding's library is restored afterwards."""
    saved = nv._lib

    def pick(which):
        nv._lib = nv.load(nv.CHECKED_LIB_PATH if which == "checked" else nv.PRODUCT_LIB_PATH)
    yield pick
    nv._lib = saved


def bf16(seed, shape, std=1.0):
    return to_dev(sg.normal_bf16(seed, 3, shape, 0.0, std)).view(torch.bfloat16)


def set_bits(x, idx, pattern):
    """Store the bf16 bit pattern at x[idx]."""
    x.view(torch.int16)[idx] = int(np.uint16(pattern).view(np.int16))


def filled(shape, dtype):
    t = torch.empty(shape, dtype=dtype, device=torch.device("cuda:0"))
    t.view(torch.uint8).fill_(SENTINEL)
    return t


def same_bits(a, b):
    return torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8))


def untouched(*ts):
    for t in ts:
        assert bool((t.view(torch.uint8) == SENTINEL).all()), "an output was written"


def expect_precondition(fn, *args, **kw):
    with pytest.raises(nv.NVFP4Error) as e:
        fn(*args, **kw)
    assert e.value.status == nv.ERROR_PRECONDITION


def operands(seed, m, n, k, groups=None):
    """Quantized A [m, k] and B ([n, k], or [groups, n, k]) from the product
    library."""
    a = nv.nvfp4_quantize_rows(bf16(seed, (m, k)))
    if groups is None:
        b = nv.nvfp4_quantize_weight(bf16(seed + 1, (1, n, k), 0.02))
    else:
        b = nv.nvfp4_quantize_weight(bf16(seed + 1, (groups, n, k), 0.02))
    return a, b[:3]


def test_checked_build_matches_product_on_valid_inputs(use):
    torch.manual_seed(0)
    x = bf16(11, (300, 512))
    amax = x.float().abs().amax(dim=1).contiguous()
    w = bf16(12, (4, 96, 256), 0.02)
    gu = torch.randn((70, 2 * 128), dtype=torch.float32, device=torch.device("cuda:0"))
    logits = torch.randn((200, 64), dtype=torch.float32, device=torch.device("cuda:0"))
    use("product")
    a, bw = operands(20, 150, 192, 512, groups=4)
    _, b1 = operands(21, 1, 96, 512)
    offs = torch.tensor([0, 40, 40, 110, 150], dtype=torch.int32, device=torch.device("cuda:0"))
    mx_a = nv.nvfp4_mxfp8_quantize_rows(bf16(30, (150, 512)))
    mx_b = nv.nvfp4_mxfp8_quantize_rows(bf16(31, (4 * 192, 512), 0.02))
    mx_bg = (mx_b[0].view(4, 192, 512), mx_b[1].view(4, 192, 16))

    def run():
        return {
            "rows": nv.nvfp4_quantize_rows(x),
            "rows_reuse": nv.nvfp4_quantize_rows(x, amax_in=amax),
            "weight": nv.nvfp4_quantize_weight(w),
            "weight_in": nv.nvfp4_quantize_weight(w, amax_in=torch.full((4,), 3.0, device=x.device)),
            "swiglu": tuple(nv.nvfp4_swiglu_quantize_rows(gu, want_h=True, want_amax=True).values()),
            "route": tuple(nv.nvfp4_moe_route(logits, 8).values()),
            "deq": (nv.nvfp4_dequantize_rows(*a),),
            "gemm": (nv.nvfp4_gemm(a, b1),),
            "grouped": (nv.nvfp4_grouped_gemm(a, offs, bw),),
            "grouped_swiglu": nv.nvfp4_grouped_gemm_swiglu(a, offs, bw),
            "mx_rows": nv.nvfp4_mxfp8_quantize_rows(x),
            "mx_gemm": (nv.nvfp4_mxfp8_gemm(mx_a, (mx_b[0][:192], mx_b[1][:192])),),
            "mx_grouped": (nv.nvfp4_mxfp8_grouped_gemm(mx_a, offs, mx_bg),),
        }

    want = run()
    use("checked")
    got = run()
    torch.cuda.synchronize()
    for key in want:
        for i, (g, r) in enumerate(zip(got[key], want[key])):
            assert same_bits(g, r), "%s output %d differs from the product build" % (key, i)


def test_quantizers_reject_non_finite_inputs(use):
    use("checked")
    dev = torch.device("cuda:0")
    for bad in (NAN_BF16, INF_BF16, INF_BF16 | 0x8000):
        x = bf16(40, (64, 256))
        set_bits(x, (37, 200), bad)
        out = (filled((64, 128), torch.uint8), filled((64, 16), torch.uint8), filled((64,), torch.float32))
        expect_precondition(nv.nvfp4_quantize_rows, x, out=out)
        untouched(*out)
        expect_precondition(nv.nvfp4_mxfp8_quantize_rows, x)
        wout = (filled((4, 16, 128), torch.uint8), filled((4, 16, 16), torch.uint8),
                filled((4,), torch.float32), filled((4,), torch.float32))
        expect_precondition(nv.nvfp4_quantize_weight, x.view(4, 16, 256), out=wout)
        untouched(*wout)
    x = bf16(41, (64, 256))
    for bad in (float("nan"), float("inf"), -1.0):
        amax = x.float().abs().amax(dim=1).contiguous()
        amax[63] = bad
        expect_precondition(nv.nvfp4_quantize_rows, x, amax_in=amax)
        expect_precondition(nv.nvfp4_quantize_weight, x.view(64, 1, 256), amax_in=amax)
    # -0.0 is a valid amax (of an all-zero row); a valid call after the
    # rejected ones succeeds
    x[0] = 0
    amax = x.float().abs().amax(dim=1).contiguous()
    amax[0] = -0.0
    nv.nvfp4_quantize_rows(x, amax_in=amax)
    gu = torch.randn((16, 64), dtype=torch.float32, device=dev)
    gu[15, 63] = float("-inf")
    expect_precondition(nv.nvfp4_swiglu_quantize_rows, gu, want_h=True)
    logits = torch.randn((32, 16), dtype=torch.float32, device=dev)
    logits[5, 3] = float("nan")
    expect_precondition(nv.nvfp4_moe_route, logits, 4)


def test_violation_in_the_last_element_of_a_large_tensor(use):
    # 4096 x 4096 bf16: 16M elements, 64 per thread of the check's capped grid
    use("checked")
    x = torch.zeros((4096, 4096), dtype=torch.bfloat16, device=torch.device("cuda:0"))
    nv.nvfp4_quantize_rows(x)
    set_bits(x, (-1, -1), INF_BF16)
    expect_precondition(nv.nvfp4_quantize_rows, x)
    set_bits(x, (-1, -1), 0)
    nv.nvfp4_quantize_rows(x)


def test_gemms_reject_nan_scales_and_codes(use):
    use("product")
    dev = torch.device("cuda:0")
    a, bw = operands(50, 64, 128, 256, groups=2)
    _, b1 = operands(51, 1, 128, 256)
    offs = torch.tensor([0, 30, 64], dtype=torch.int32, device=dev)
    use("checked")
    for which, idx, val in (("a", 1, 0x7F), ("a", 1, 0xFF), ("b", 1, 0xFF)):
        aa = [t.clone() for t in a]
        bb = [t.clone() for t in b1]
        (aa if which == "a" else bb)[idx].view(-1)[-1] = val
        y = filled((64, 128), torch.float32)
        expect_precondition(nv.nvfp4_gemm, tuple(aa), tuple(bb), out=y)
        untouched(y)
        if which == "a":
            expect_precondition(nv.nvfp4_dequantize_rows, *aa)
        else:
            expect_precondition(nv.nvfp4_dequantize_rows, *bb, rows_per_scale=128)
    for which, bad in (("a", float("nan")), ("a", float("inf")), ("b", float("nan"))):
        aa = [t.clone() for t in a]
        bg = [t.clone() for t in bw]
        (aa if which == "a" else bg)[2][-1] = bad
        expect_precondition(nv.nvfp4_grouped_gemm, tuple(aa), offs, tuple(bg))
        expect_precondition(nv.nvfp4_grouped_gemm_swiglu, tuple(aa), offs, tuple(bg))
        if which == "a":
            expect_precondition(nv.nvfp4_dequantize_rows, *aa)
    bg = [t.clone() for t in bw]
    bg[1][1, 127, 15] = 0x7F
    expect_precondition(nv.nvfp4_grouped_gemm, a, offs, tuple(bg))
    nv.nvfp4_grouped_gemm(a, offs, bw)


def test_mxfp8_gemms_reject_nan_codes(use):
    use("product")
    dev = torch.device("cuda:0")
    ma = nv.nvfp4_mxfp8_quantize_rows(bf16(60, (64, 256)))
    mb = nv.nvfp4_mxfp8_quantize_rows(bf16(61, (2 * 96, 256)))
    offs = torch.tensor([0, 10, 64], dtype=torch.int32, device=dev)
    use("checked")
    cases = [(0, 0x7F), (0, 0xFF), (1, 0xFF)]  # E4M3 element NaNs, E8M0 NaN scale
    for idx, val in cases:
        aa = [t.clone() for t in ma]
        aa[idx].view(-1)[-1] = val
        y = filled((64, 96), torch.float32)
        expect_precondition(nv.nvfp4_mxfp8_gemm, tuple(aa), (mb[0][:96], mb[1][:96]), out=y)
        untouched(y)
        bb = [t.clone().view(2, 96, -1) for t in mb]
        bb[idx][1, 95, -1] = val
        expect_precondition(nv.nvfp4_mxfp8_grouped_gemm, ma, offs, tuple(bb))
    nv.nvfp4_mxfp8_grouped_gemm(ma, offs, (mb[0].view(2, 96, 256), mb[1].view(2, 96, 8)))


@pytest.mark.parametrize("offs", [[0, 40, 30, 64], [0, 64, 64, 63], [5, 4, 10, 64],
                                  [0] * 200 + [1] + [0]])
def test_grouped_gemms_reject_decreasing_offsets(use, offs):
    use("product")
    dev = torch.device("cuda:0")
    groups = len(offs) - 1
    a, bw = operands(70 + groups, 64, 128, 256, groups=groups)
    ma = nv.nvfp4_mxfp8_quantize_rows(bf16(72, (64, 256)))
    mb = nv.nvfp4_mxfp8_quantize_rows(bf16(73, (groups * 32, 256)))
    use("checked")
    o = torch.tensor(offs, dtype=torch.int32, device=dev)
    y = filled((64, 128), torch.float32)
    expect_precondition(nv.nvfp4_grouped_gemm, a, o, bw, out=y)
    untouched(y)
    expect_precondition(nv.nvfp4_grouped_gemm_swiglu, a, o, bw)
    expect_precondition(nv.nvfp4_mxfp8_grouped_gemm, ma, o,
                        (mb[0].view(groups, 32, 256), mb[1].view(groups, 32, 8)))
    # offsets outside [0, m_total] but non-decreasing are clamped (defined)
    o = torch.tensor([-5] + sorted(max(v, 0) for v in offs[1:-1]) + [1000], dtype=torch.int32, device=dev)
    nv.nvfp4_grouped_gemm(a, o, bw)
