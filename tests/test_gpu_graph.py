"""HIP graph capture of the hot path: weight quantize (per expert), token
quantize, on-device routing and the grouped GEMM recorded once in a graph and
replayed, with the program's own eager work and synchronizations between the
replays.  Every replay must reproduce the eager results bit for bit (the same
kernels on the same inputs are deterministic), which also checks that no step
relies on anything a graph does not record (host-side memsets, host reads of
device metadata)."""
import numpy as np
import pytest
import torch

import nvfp4_token_quantization_amd as nv
import oracle
import synthgen as sg
from gpu_helpers import assert_same_quant, dev, to_dev

pytestmark = pytest.mark.gpu


def _step(wd, xd, logits, outs):
    """One pass: quantize W [E, N, K] per expert and X [T, K] per token, route
    T tokens top-2 over E experts, grouped GEMM through row_index."""
    wq, xq, rt, y = outs
    nv.nvfp4_quantize_weight(wd, out=wq)
    nv.nvfp4_quantize_rows(xd, out=xq)
    nv.nvfp4_moe_route(logits, topk=2, out=rt)
    nv.nvfp4_grouped_gemm(xq, rt["offsets"], wq[:3], row_index=rt["row_index"], out=y)


def _alloc(E, N, K, T, topk):
    d = dev()
    u8, f32, i32 = torch.uint8, torch.float32, torch.int32
    wq = (torch.empty((E, N, K // 2), dtype=u8, device=d), torch.empty((E, N, K // 16), dtype=u8, device=d),
          torch.empty((E,), dtype=f32, device=d), torch.empty((E,), dtype=f32, device=d))
    xq = (torch.empty((T, K // 2), dtype=u8, device=d), torch.empty((T, K // 16), dtype=u8, device=d),
          torch.empty((T,), dtype=f32, device=d))
    rt = {"experts": torch.empty((T, topk), dtype=i32, device=d),
          "offsets": torch.empty((E + 1,), dtype=i32, device=d),
          "row_index": torch.empty((T * topk,), dtype=i32, device=d),
          "slot_of": torch.empty((T, topk), dtype=i32, device=d)}
    y = torch.empty((T * topk, N), dtype=f32, device=d)
    return wq, xq, rt, y


def _flat(outs):
    wq, xq, rt, y = outs
    return list(wq) + list(xq) + [rt[k] for k in ("experts", "offsets", "row_index", "slot_of")] + [y]


def test_graph_replays_match_eager():
    E, N, K, T, topk = 8, 96, 256, 300, 2
    wd = to_dev(sg.normal_bf16(91, sg.S_W, (E, N, K), 0.0, 0.02))
    xd = to_dev(sg.student_t3_bf16(92, sg.S_X, (T, K)))
    logits = to_dev(sg.router_logits(93, T, experts=E))

    eager = _alloc(E, N, K, T, topk)
    _step(wd, xd, logits, eager)
    torch.cuda.synchronize()
    want = [t.clone() for t in _flat(eager)]

    outs = _alloc(E, N, K, T, topk)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _step(wd, xd, logits, outs)  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _step(wd, xd, logits, outs)

    other = _alloc(E, N, K, T, topk)
    x2 = to_dev(sg.student_t3_bf16(94, sg.S_X, (T, K)))
    for rep in range(4):
        for t in _flat(outs):
            t.fill_(90 if t.dtype == torch.uint8 else -7)  # eager fill kernels
        g.replay()
        _step(wd, x2, logits, other)  # eager work between replays
        torch.cuda.synchronize()
        for name, got, w in zip(range(len(want)), _flat(outs), want):
            if not torch.equal(got, w):
                bad = int((got != w).sum())
                raise AssertionError("replay %d: output %d differs from eager in %d entries" % (
                    rep, name, bad))


def test_graph_replays_one_pass_weight_quantize():
    """The one-pass weight quantizer (its clear kernel, then the team kernel
    with a slot round and an atomic round per team: 32 groups of 4096 x 256)
    recorded in a graph: every replay, with a different weight quantized
    eagerly in between on the same kind of buffers, equals the eager result
    and the oracle."""
    G, R, K = 32, 4096, 256
    assert R * K * 2 >= 512 * 1024 and G >= 8
    w = sg.normal_bf16(95, sg.S_W, (G, R, K), 0.0, 0.02)
    wd, w2 = to_dev(w), to_dev(sg.normal_bf16(96, sg.S_W, (G, R, K), 0.0, 0.05))
    want = oracle.quantize_weight(w)

    def alloc():
        d = dev()
        return (torch.empty((G, R, K // 2), dtype=torch.uint8, device=d),
                torch.empty((G, R, K // 16), dtype=torch.uint8, device=d),
                torch.empty((G,), dtype=torch.float32, device=d), torch.empty((G,), dtype=torch.float32, device=d))

    outs = alloc()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        nv.nvfp4_quantize_weight(wd, out=outs)  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        nv.nvfp4_quantize_weight(wd, out=outs)
    other = alloc()
    for rep in range(4):
        for t in outs:
            t.fill_(77 if t.dtype == torch.uint8 else 3.0)  # stale values in the slot and counter words
        g.replay()
        nv.nvfp4_quantize_weight(w2, out=other)  # eager work between replays
        torch.cuda.synchronize()
        assert_same_quant(outs, want, "replay %d" % rep)
