"""GPU parity of on-device top-k routing into the contiguous per-expert
layout (miniTE page, section Transformer Engine路径优化: contiguous layouts,
device-side metadata, tokens quantized once) against the oracle: experts,
offsets, row_index and slot_of must match exactly (integer work)."""
import numpy as np
import pytest
import torch

import nvfp4_token_quantization_amd as nv
import oracle
import synthgen as sg
from gpu_helpers import check_gemm, dev, oracle_weight, to_dev, to_np, workload

pytestmark = pytest.mark.gpu


def check_route(lg, topk, what):
    got = nv.nvfp4_moe_route(to_dev(lg), topk)
    torch.cuda.synchronize()
    want = oracle.route(lg, topk)
    for key in ("experts", "offsets", "row_index", "slot_of"):
        g = to_np(got[key]).reshape(want[key].shape)
        if not np.array_equal(g, want[key]):
            bad = np.argwhere(g != want[key])
            raise AssertionError("%s %s: %d mismatches, first at %s (got %s want %s)" % (
                what, key, len(bad), tuple(bad[0]), g[tuple(bad[0])], want[key][tuple(bad[0])]))
    return got


@pytest.mark.parametrize("T,E,topk", [(1, 8, 1), (7, 16, 4), (64, 128, 8), (4096, 128, 8),
                                      (300, 256, 8), (1000, 1024, 16), (513, 64, 64),
                                      (20000, 128, 8), (129, 3, 2),
                                      # the 17-32 and 257-512 expert kernels
                                      (77, 20, 3), (50, 32, 4), (333, 512, 8), (100, 300, 16)])
def test_route_matches_oracle(T, E, topk):
    lg = sg.router_logits(sg.config_seed(50) + T + E, T, E)
    check_route(lg, topk, "T=%d E=%d topk=%d" % (T, E, topk))


def test_route_moe_workload():
    lg = workload(3, "logits")["logits"]
    check_route(lg, 8, "MoE 4096 tokens, 128 experts")


def test_route_ties_signed_zero_and_equal_logits():
    rng = np.random.default_rng(8)
    lg = (rng.integers(-2, 3, size=(777, 128)) * 0.25).astype(np.float32)
    lg = np.where(rng.random(lg.shape) < 0.3, np.float32(-0.0), lg).astype(np.float32)
    lg[0] = 0.0
    lg[1] = -0.0
    lg[2, ::2] = -0.0
    check_route(lg, 8, "ties")
    check_route(np.zeros((40, 128), np.float32), 8, "all equal")
    check_route(np.full((40, 64), 3.0e38, np.float32), 64, "topk = E")


def test_route_empty_batch_writes_zero_offsets():
    d = dev()
    r = nv.nvfp4_moe_route(torch.zeros((0, 128), dtype=torch.float32, device=d), 8)
    torch.cuda.synchronize()
    assert to_np(r["offsets"]).tolist() == [0] * 129


def test_route_deterministic():
    lg = to_dev(sg.router_logits(5, 8192, 128))
    a = nv.nvfp4_moe_route(lg, 8)
    b = nv.nvfp4_moe_route(lg, 8)
    torch.cuda.synchronize()
    for key in a:
        assert torch.equal(a[key], b[key]), key


def test_device_route_feeds_grouped_gemm():
    """Quantize-once rollout-decode chain entirely on the device: route the
    64 tokens, quantize each once, grouped up-projection through row_index;
    every output entry checked against the oracle's chain."""
    d = workload(5, "x,logits")
    rt = nv.nvfp4_moe_route(to_dev(d["logits"]), 8)
    xq = nv.nvfp4_quantize_rows(to_dev(d["x"]))
    wq, wsb, ws, _ = oracle_weight(5, "w")
    b = (to_dev(wq), to_dev(wsb), to_dev(ws))
    y = nv.nvfp4_grouped_gemm(xq, rt["offsets"], b, row_index=rt["row_index"])
    torch.cuda.synchronize()
    want = oracle.route(d["logits"], 8)
    oq = oracle.quantize_rows(d["x"])
    y_ref, bound = oracle.grouped_gemm(oq, want["offsets"], (wq, wsb, ws), row_index=want["row_index"])
    check_gemm(y, y_ref, bound, "device-routed grouped GEMM")
