"""Pins for the oracle's top-k routing into the contiguous per-expert layout
(miniTE page, section Transformer Engine路径优化: contiguous layouts and
device-side metadata for the grouped GEMMs).

  - library routine: numpy's stable argsort of -logits gives the top-k with
    ties to the lower expert id; numpy's lexsort by (expert, token) gives the
    layout;
  - invariants: offsets are the running counts, row_index is increasing inside
    each expert, slot_of inverts the layout, every token appears topk times;
  - special cases: all-equal logits pick experts 0..topk-1; topk = E orders
    every expert; +0 and -0 tie.
"""
import numpy as np
import pytest

import synthgen as sg


def numpy_route(lg, topk):
    T, E = lg.shape
    experts = np.argsort(-lg.astype(np.float64), axis=1, kind="stable")[:, :topk]
    tok = np.repeat(np.arange(T), topk)
    exp = experts.reshape(-1)
    order = np.lexsort((tok, exp))
    offsets = np.zeros(E + 1, np.int64)
    offsets[1:] = np.cumsum(np.bincount(exp, minlength=E))
    slot = np.empty(T * topk, np.int64)
    slot[order] = np.arange(T * topk)
    return experts, offsets, tok[order], slot.reshape(T, topk)


def check(oracle, lg, topk):
    r = oracle.route(lg, topk)
    e, off, ri, slot = numpy_route(lg, topk)
    assert np.array_equal(r["experts"], e)
    assert np.array_equal(r["offsets"], off)
    assert np.array_equal(r["row_index"], ri)
    assert np.array_equal(r["slot_of"], slot)
    return r


@pytest.mark.parametrize("T,E,topk", [(1, 8, 1), (37, 16, 4), (512, 128, 8), (300, 256, 8),
                                      (64, 1024, 16)])
def test_route_matches_numpy(oracle, T, E, topk):
    lg = sg.router_logits(sg.config_seed(40) + T, T, E)
    check(oracle, lg, topk)


def test_route_ties_and_signed_zero(oracle):
    rng = np.random.default_rng(3)
    lg = (rng.integers(-3, 4, size=(200, 32)) * 0.5).astype(np.float32)  # many ties
    lg[:, 5] = np.where(lg[:, 5] == 0, -0.0, lg[:, 5]).astype(np.float32)
    lg[0] = 0.0
    lg[0, 7] = -0.0
    r = check(oracle, lg, 6)
    assert r["experts"][0].tolist() == [0, 1, 2, 3, 4, 5]


def test_route_invariants_on_moe_workload(oracle):
    lg = sg.workload(3, part={"logits"})["logits"]
    r = check(oracle, lg, 8)
    T, topk = r["experts"].shape
    off, ri, slot = r["offsets"], r["row_index"], r["slot_of"]
    assert off[0] == 0 and off[-1] == T * topk and np.all(np.diff(off) >= 0)
    for e in range(len(off) - 1):
        seg = ri[off[e]:off[e + 1]]
        assert np.all(np.diff(seg) > 0)                     # token order inside an expert
        assert np.all((r["experts"][seg] == e).sum(axis=1) == 1)
    assert np.array_equal(ri[slot], np.repeat(np.arange(T), topk).reshape(T, topk))
    assert np.array_equal(np.bincount(ri, minlength=T), np.full(T, topk))
    # the Zipf bias makes the load uneven: the busiest expert far above the mean
    assert r["counts"].max() > 4 * T * topk / len(r["counts"])


def test_route_all_experts_and_equal_logits(oracle):
    lg = np.zeros((5, 12), np.float32)
    r = check(oracle, lg, 12)
    assert np.array_equal(r["experts"], np.tile(np.arange(12), (5, 1)))
    lg = sg.router_logits(99, 9, 12)
    r = check(oracle, lg, 12)
    assert np.all(np.diff(np.take_along_axis(lg, r["experts"], axis=1), axis=1) <= 0)


def test_route_rejects_bad_input(oracle):
    with pytest.raises(ValueError):
        oracle.route(np.zeros((4, 8), np.float32), topk=9)
    lg = np.zeros((4, 8), np.float32)
    lg[2, 3] = np.nan
    with pytest.raises(ValueError):
        oracle.route(lg, topk=2)
