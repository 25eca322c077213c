"""Seeded synthetic inputs for the per-token NVFP4 path.

Shared by the tests, the benchmark and the oracle's self-checks.  This module
draws random numbers (activations, weights, router logits); it holds none of the
quantizer's, the router's or the GEMM's arithmetic.  The random streams are SplitMix64
(counter-based, see ``synthgen.c``), so a tensor's bytes depend only on
(seed, stream, index), never on thread count or machine.

Workloads (shapes and value distributions of the layers the pages train:
Qwen3-4B dense and Qwen3-30B-A3B MoE; no weights or activations of those
models are used):

  1 tiny dense     X 128x512 N(0,1) with 1% of entries x50, W 256x512 N(0,0.02)
  2 dense linear   X 4096x2560 Student-t(3)/sqrt(3), W 9728x2560 N(0,0.02)
  3 MoE up         X 4096x2048 t3, fp32 router logits N(0,1) + Zipf(1.1) expert
                   bias for 128 experts (top-8 routing), W_up 128x1536x2048 N(0,0.02)
  4 MoE down       H 32768x768 t3 in the contiguous layout of config 3's
                   routing (its logits), exact row amax supplied for reuse,
                   W_dn 128x2048x768
  5 rollout decode 64 tokens: X 64x2048 and H 512x768 t3, router logits of its own,
                   the config 3/4 expert shapes, and dense 64x2560 -> 9728
"""
import ctypes
import math
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synthgen.c")
_LIB = os.path.join(_HERE, "libsynthgen.so")


def build(force=False):
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
                               "-ffp-contract=off", "-Wall", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB)
        U64, I64, D, P = ctypes.c_uint64, ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
        L.synth_u64.argtypes = [U64, U64, U64]
        L.synth_u64.restype = U64
        L.synth_uniform_f64.argtypes = [U64, U64, I64, P]
        L.synth_normal_f64.argtypes = [U64, U64, I64, P]
        L.synth_normal_bf16.argtypes = [U64, U64, I64, D, D, P]
        L.synth_student_t3_bf16.argtypes = [U64, U64, I64, D, P]
        L.synth_normal_outliers_bf16.argtypes = [U64, U64, I64, D, D, D, P]
        L.synth_f32_to_bf16.argtypes = [P, I64, P]
        _lib = L
    return _lib


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def config_seed(c):
    return 0x5EED0000 + int(c)


# stream ids per tensor role
S_X, S_W, S_LOGITS, S_PERM, S_WDN, S_H, S_XD, S_WD, S_MISC = 1, 2, 3, 4, 5, 6, 7, 8, 9


def u64(seed, stream, i):
    return int(lib().synth_u64(seed, stream, i))


def uniform(seed, stream, n):
    out = np.empty((n,), np.float64)
    lib().synth_uniform_f64(seed, stream, n, _p(out))
    return out


def normal(seed, stream, n):
    out = np.empty((n,), np.float64)
    lib().synth_normal_f64(seed, stream, n, _p(out))
    return out


def normal_bf16(seed, stream, shape, mean=0.0, std=1.0):
    n = int(np.prod(shape))
    out = np.empty((n,), np.uint16)
    lib().synth_normal_bf16(seed, stream, n, mean, std, _p(out))
    return out.reshape(shape)


def student_t3_bf16(seed, stream, shape, unit_std=True):
    n = int(np.prod(shape))
    out = np.empty((n,), np.uint16)
    lib().synth_student_t3_bf16(seed, stream, n, 1.0 / math.sqrt(3.0) if unit_std else 1.0, _p(out))
    return out.reshape(shape)


def normal_outliers_bf16(seed, stream, shape, std=1.0, p=0.01, mult=50.0):
    n = int(np.prod(shape))
    out = np.empty((n,), np.uint16)
    lib().synth_normal_outliers_bf16(seed, stream, n, std, p, mult, _p(out))
    return out.reshape(shape)


def f32_to_bf16(a):
    """Round fp32 values to bf16 bits (nearest even); inputs must be finite."""
    a = np.ascontiguousarray(a, np.float32)
    out = np.empty(a.shape, np.uint16)
    lib().synth_f32_to_bf16(_p(a), a.size, _p(out))
    return out


def bf16_to_f32(b):
    return (np.ascontiguousarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)


def permutation(seed, stream, n):
    """Fisher-Yates shuffle of 0..n-1 driven by the SplitMix64 stream."""
    perm = list(range(n))
    for t, i in enumerate(range(n - 1, 0, -1)):
        j = u64(seed, stream, t) % (i + 1)
        perm[i], perm[j] = perm[j], perm[i]
    return np.array(perm, np.int64)


def router_logits(seed, tokens, experts=128, zipf_s=1.1):
    """fp32 router logits [tokens, experts]: N(0,1) plus a Zipf(s) expert
    bias.  Expert e has popularity rank r_e (a seeded permutation of 1..E) and
    bias ln(r_e^-s / sum_r r^-s), so a few experts draw most tokens, as in a
    trained MoE router.  Formed in fp64 and rounded to fp32 (nearest even)."""
    ranks = permutation(seed, S_PERM, experts) + 1
    w = np.arange(1, experts + 1, dtype=np.float64) ** (-zipf_s)
    bias = np.log(ranks.astype(np.float64) ** (-zipf_s) / w.sum())
    z = normal(seed, S_LOGITS, tokens * experts).reshape(tokens, experts) + bias[None, :]
    return z.astype(np.float32)


def row_amax_bf16(x_bf16):
    """Exact row max of |x| for bf16 rows (a producer-side statistic supplied
    to the amax-reuse path; plain max of the widened values)."""
    return np.abs(bf16_to_f32(x_bf16)).max(axis=1).astype(np.float32)


def workload(c, part=None):
    """Inputs of workload c (1..5) as numpy arrays (bf16 as uint16 bits).

    `part` restricts generation to some tensors (a set of names), since the
    expert weights of configs 3-5 are large.
    """
    seed = config_seed(c)
    want = (lambda name: part is None or name in part)
    d = {"config": c, "seed": seed}
    if c == 1:
        if want("x"):
            d["x"] = normal_outliers_bf16(seed, S_X, (128, 512), 1.0, 0.01, 50.0)
        if want("w"):
            d["w"] = normal_bf16(seed, S_W, (1, 256, 512), 0.0, 0.02)
    elif c == 2:
        if want("x"):
            d["x"] = student_t3_bf16(seed, S_X, (4096, 2560))
        if want("w"):
            d["w"] = normal_bf16(seed, S_W, (1, 9728, 2560), 0.0, 0.02)
    elif c == 3:
        if want("x"):
            d["x"] = student_t3_bf16(seed, S_X, (4096, 2048))
        if want("logits"):
            d["logits"] = router_logits(seed, 4096)
        if want("w"):
            d["w"] = normal_bf16(seed, S_W, (128, 1536, 2048), 0.0, 0.02)
    elif c == 4:
        if want("h"):
            d["h"] = student_t3_bf16(seed, S_H, (32768, 768))
            d["h_amax"] = row_amax_bf16(d["h"])
        if want("logits"):
            d["logits"] = router_logits(config_seed(3), 4096)
        if want("w"):
            d["w"] = normal_bf16(seed, S_WDN, (128, 2048, 768), 0.0, 0.02)
    elif c == 5:
        if want("x"):
            d["x"] = student_t3_bf16(seed, S_X, (64, 2048))
        if want("logits"):
            d["logits"] = router_logits(seed, 64)
        if want("h"):
            d["h"] = student_t3_bf16(seed, S_H, (512, 768))
            d["h_amax"] = row_amax_bf16(d["h"])
        if want("xd"):
            d["xd"] = student_t3_bf16(seed, S_XD, (64, 2560))
        if want("w"):
            d["w"] = normal_bf16(seed, S_W, (128, 1536, 2048), 0.0, 0.02)
        if want("w_dn"):
            d["w_dn"] = normal_bf16(seed, S_WDN, (128, 2048, 768), 0.0, 0.02)
        if want("wd"):
            d["wd"] = normal_bf16(seed, S_WD, (1, 9728, 2560), 0.0, 0.02)
    else:
        raise ValueError("workload %r: configs are 1..5" % (c,))
    return d
