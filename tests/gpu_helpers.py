"""Shared helpers for the GPU parity tests: device transfer and cached
workloads.  Inputs come from synthgen; expected values from the oracle."""
import functools

import numpy as np
import torch

import oracle
import synthgen as sg


def dev():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a ROCm GPU (cuda:0)")
    return torch.device("cuda:0")


def to_dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(dev())


def to_np(t):
    return t.cpu().numpy()


def bits(a):
    a = np.asarray(a)
    return a.view(np.uint32) if a.dtype == np.float32 else a


def assert_same_quant(got, want, what=""):
    """Bit-exact comparison of (q, sb, s[, amax]) tuples; reports the first
    mismatching row."""
    names = ["q", "sb", "s", "amax"]
    for name, g, w in zip(names, got, want):
        g = bits(to_np(g) if isinstance(g, torch.Tensor) else g)
        w = bits(w)
        g = g.reshape(w.shape)
        if not np.array_equal(g, w):
            bad = np.argwhere(g != w)
            raise AssertionError("%s %s: %d mismatches, first at %s (got %s want %s)" % (
                what, name, len(bad), tuple(bad[0]), g[tuple(bad[0])], w[tuple(bad[0])]))


def check_gemm(y, y_ref, bound, what=""):
    y = to_np(y) if isinstance(y, torch.Tensor) else y
    ok = oracle.gemm_within_bound(y, y_ref, bound)
    if not ok.all():
        bad = np.argwhere(~ok)
        i = tuple(bad[0])
        raise AssertionError("%s: %d of %d entries outside 1e-5*sum|ab|; first %s got %r want %r "
                             "bound %r" % (what, len(bad), ok.size, i, y[i], y_ref[i], bound[i]))
    zero = bound == 0
    assert np.all(y[zero] == 0), what + ": entries with zero bound must be +-0"


@functools.lru_cache(maxsize=None)
def workload(c, part):
    return sg.workload(c, part=set(part.split(",")))


@functools.lru_cache(maxsize=None)
def routing(c):
    """The oracle's top-8 contiguous layout of workload c's router logits."""
    return oracle.route(workload(c, "logits")["logits"], topk=8)


@functools.lru_cache(maxsize=None)
def oracle_weight(c, name):
    w = workload(c, name)[name]
    return oracle.quantize_weight(w)


@functools.lru_cache(maxsize=None)
def oracle_rows(c, name, reuse=False):
    d = workload(c, name)
    amax = d.get(name + "_amax") if reuse else None
    return oracle.quantize_rows(d[name], amax_in=amax)
