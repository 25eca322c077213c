"""GPU tests of the one-pass weight quantizer (nvfp4_quantize_weight without
amax_in, at least 8 groups of at least 512 KiB of bf16 each): each group is
read once and held in registers by a team of workgroups on one XCD that
agree on the group amax through amax_out and a counter in s (Miles page, section
并行度与张量转换的一致性契约: one FP32 scale per tensor or per expert).

Every output must equal the oracle's quantize_weight bit for bit:
- the product path at shapes that take the one-pass kernel: ragged row
  groups (rows not a multiple of the rows per row group), group counts that
  do not fill the last round of teams, an all-zero group and a group holding
  the largest finite bf16, every lanes-per-row layout (16, 32 and 64 lanes,
  1 to 8 half-blocks per lane), and slot areas (the first 64 code dwords of
  a group, written last) that span several rows or end inside one;
- the self-test hook with a zero time limit, where workgroups that do not
  find their team complete read the whole group themselves;
- the hook on small groups and few groups (below the library's thresholds,
  teams spanning XCDs);
- repeated calls give identical bits (the amax is an order-free maximum).
"""
import numpy as np
import pytest
import torch

import nvfp4_token_quantization_amd as nv
import nvfp4_token_quantization_amd.selftest as st
import oracle
import synthgen as sg
from gpu_helpers import assert_same_quant, oracle_weight, to_dev, workload

pytestmark = pytest.mark.gpu

MAXBF = 0x7F7F  # largest finite bf16


def weight(seed, groups, rows, k, std=0.02):
    w = sg.normal_bf16(seed, 2, (groups, rows, k), 0.0, std)
    return w


@pytest.mark.parametrize("groups,rows,k", [
    (11, 1025, 256),   # 32 lanes x 1 half-block, odd rows, 11 groups over 8 teams
    (16, 700, 768),    # 32 x 3 (the MoE down-projection's k), 16 teams
    (8, 200, 4096),    # 64 x 8
    (9, 1000, 592),    # 16 x 5, a row's last lanes idle
    (12, 130, 2048),   # 64 x 4
    (16, 16384, 16),   # 16 x 1, two rounds: a slot area spans 32 rows
    (32, 6000, 48),    # 16 x 1, two rounds: a slot area ends inside a row
])
def test_onepass_product_path_matches_oracle(groups, rows, k):
    # groups of at least 512 KiB and at least 8 of them (one team per XCD)
    assert rows * k * 2 >= 512 * 1024 and groups >= 8, "the shape must take the one-pass kernel"
    w = weight(900 + k, groups, rows, k)
    if groups > 2:
        w[1] = 0                     # an all-zero group: S = 0, every code 0
        w[2, rows // 2, :16] = MAXBF  # a group whose amax is the largest bf16
    got = nv.nvfp4_quantize_weight(to_dev(w))
    assert_same_quant(got, oracle.quantize_weight(w), "one-pass %dx%dx%d" % (groups, rows, k))


def test_onepass_repeat_is_bit_identical():
    w = to_dev(weight(77, 16, 1536, 512))
    ref = [t.clone() for t in nv.nvfp4_quantize_weight(w)]
    for _ in range(5):
        got = nv.nvfp4_quantize_weight(w)
        for a, b in zip(got, ref):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))


@pytest.mark.parametrize("groups,rows,k", [(5, 3, 16), (40, 17, 272), (3, 1000, 768), (9, 64, 2048),
                                           (1, 130, 2048), (2, 200, 4096)])
@pytest.mark.parametrize("limit_ms", [10.0, 0.0])
def test_onepass_hook_small_groups_and_timeout_path(groups, rows, k, limit_ms):
    """The kernel forced at any size and team count (fewer than 8 groups give
    teams that span XCDs; one group gives one team of every workgroup); a
    zero time limit sends every workgroup that does not find its team
    complete down the read-the-group path."""
    w = weight(300 + rows + k, groups, rows, k)
    w[groups // 2] = 0
    w[0, 0, :16] = MAXBF
    got = st.nvfp4_debug_quantize_weight_onepass(to_dev(w), limit_ms=limit_ms)
    assert_same_quant(got, oracle.quantize_weight(w), "hook %dx%dx%d limit %g" % (groups, rows, k, limit_ms))


def test_onepass_timeout_path_full_expert_weight():
    """128 experts of 1536 x 2048 with a zero time limit: the fallback at the
    MoE up-projection's size equals the normal one-pass result and the
    oracle."""
    wd = to_dev(workload(3, "w")["w"])
    assert tuple(wd.shape) == (128, 1536, 2048)
    got0 = st.nvfp4_debug_quantize_weight_onepass(wd, limit_ms=0.0)
    assert_same_quant(got0, oracle_weight(3, "w"), "W_up one-pass, zero time limit")
    got = nv.nvfp4_quantize_weight(wd)
    for a, b in zip(got0, got):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))


def test_onepass_hook_rejects_rows_it_cannot_hold():
    # 16384-element rows need 32 half-blocks per lane: the one-pass kernel
    # holds at most 8, so the hook reports UNSUPPORTED_SHAPE (the library
    # quantizes such weights in two passes)
    w = torch.zeros((1, 4, 16384), dtype=torch.bfloat16, device=torch.device("cuda:0"))
    with pytest.raises(nv.NVFP4Error):
        st.nvfp4_debug_quantize_weight_onepass(w)
    q, sb, s, amax = nv.nvfp4_quantize_weight(w)
    assert float(s[0]) == 0.0 and float(amax[0]) == 0.0
    assert int(q.sum()) == 0 and int(sb.sum()) == 0


def test_onepass_concurrent_streams():
    """Two one-pass quantizations launched back to back on two streams (32
    groups of 2048 x 512 each: a slot round and an atomic round per team)
    compete for the CUs, so a team's members need not all be resident at
    once; whatever each member's wait does (the team completes, or its time
    limit sends it down the read-the-group path), both results equal the
    oracle's."""
    G, R, K = 32, 2048, 512
    w1 = weight(501, G, R, K)
    w2 = weight(502, G, R, K, std=0.05)
    want1, want2 = oracle.quantize_weight(w1), oracle.quantize_weight(w2)
    d1, d2 = to_dev(w1), to_dev(w2)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    for rep in range(3):
        with torch.cuda.stream(s1):
            got1 = nv.nvfp4_quantize_weight(d1)
        with torch.cuda.stream(s2):
            got2 = nv.nvfp4_quantize_weight(d2)
        torch.cuda.synchronize()
        assert_same_quant(got1, want1, "stream 1, repeat %d" % rep)
        assert_same_quant(got2, want2, "stream 2, repeat %d" % rep)


def test_onepass_hook_random_shapes():
    """A seeded sweep of shapes through the hook (any size, any team count):
    k from 16 to 4096 (every lanes-per-row layout the kernel takes, ragged
    rows in a lane's last half-blocks), 1 to 40 groups, 1 to 700 rows, the
    normal time limit and a zero one; every output equals the oracle's."""
    rng = np.random.default_rng(20261203)
    ks = [16, 48, 112, 256, 272, 592, 768, 1040, 2048, 2576, 4096]
    for case in range(24):
        k = int(ks[case % len(ks)])
        groups = int(rng.integers(1, 41))
        rows = int(rng.integers(1, 701))
        if groups * rows * k > 12_000_000:
            rows = max(1, 12_000_000 // (groups * k))
        limit = 0.0 if case % 3 == 2 else 10.0
        w = weight(1000 + case, groups, rows, k, std=float(rng.choice([0.02, 1.0, 300.0])))
        if case % 4 == 1:
            w[rng.integers(0, groups)] = 0
        got = st.nvfp4_debug_quantize_weight_onepass(to_dev(w), limit_ms=limit)
        assert_same_quant(got, oracle.quantize_weight(w),
                          "case %d: %dx%dx%d limit %g" % (case, groups, rows, k, limit))
