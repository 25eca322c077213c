"""Build libnvfp4.so (HIP, gfx950), its checked variant libnvfp4_checked.so
(the same sources with NVFP4_CHECKED=1 plus checks.hip: device-side
preconditions validated before each call's work) and the test-only codec
self-test library libnvfp4_selftest.so in-tree with hipcc: one object per
source and flag set, compiled in parallel, then linked into the shared
libraries."""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libnvfp4.so")
SOURCES = ["abi_common.hip", "host_util.hip", "quantize.hip", "swiglu_quantize.hip", "route.hip",
           "dequantize.hip", "mxfp8.hip", "mxfp8_gemm.hip", "gemm.hip", "gemm_skinny.hip"]
CHECKED_LIB = os.path.join(HERE, "libnvfp4_checked.so")
CHECKED_SOURCES = SOURCES + ["checks.hip"]
CHECKED_FLAGS = ("-DNVFP4_CHECKED=1",)
SELFTEST_LIB = os.path.join(HERE, "libnvfp4_selftest.so")
SELFTEST_SOURCES = ["selftest.hip", "host_util.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # correctly rounded fp32 division and reciprocal, denormals kept, no
    # fast-math: the quantizer's fp32 steps are part of its contract
    "-fno-fast-math", "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    # never emit packed fp32 arithmetic
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def _filter(out):
    # the host pass does not know the packed-fp32 feature and says so
    return "\n".join(l for l in out.splitlines() if "packed-fp32-ops" not in l and l.strip())


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    return r.returncode, _filter(r.stdout + r.stderr)


def build(verbose=False, sources=None, lib=None, jobs=None, extra_flags=()):
    """Compile and link the libraries.  By default: libnvfp4.so from SOURCES,
    libnvfp4_checked.so from CHECKED_SOURCES with CHECKED_FLAGS and
    libnvfp4_selftest.so from SELFTEST_SOURCES.  With `sources` and `lib`:
    that one library.  `extra_flags` are added to every compile.  Returns the
    path of the (first) library."""
    if sources or lib:
        targets = [(lib or LIB, list(sources or SOURCES), ())]
    else:
        targets = [(LIB, SOURCES, ()), (CHECKED_LIB, CHECKED_SOURCES, CHECKED_FLAGS),
                   (SELFTEST_LIB, SELFTEST_SOURCES, ())]
    units = sorted({(s, fl) for _, srcs, fl in targets for s in srcs})
    objdir = os.path.join(os.path.dirname(os.path.abspath(targets[0][0])), "_build")
    os.makedirs(objdir, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    tag = "%d" % os.getpid()
    jobs = jobs or min(len(units), int(os.environ.get("MAX_JOBS", "8")), os.cpu_count() or 1)

    def compile_one(unit):
        src, fl = unit
        kind = "checked." if fl else ""
        obj = os.path.join(objdir, os.path.splitext(src)[0] + "." + kind + tag + ".o")
        cmd = [HIPCC] + FLAGS + list(fl) + list(extra_flags) + inc + ["-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        rc, msg = _run(cmd)
        return unit, obj, rc, msg

    with ThreadPoolExecutor(max_workers=jobs) as ex:
        results = list(ex.map(compile_one, units))
    obj_of = {u: o for u, o, _, _ in results}
    failed = [(u[0], m) for u, _, rc, m in results if rc != 0]
    try:
        if failed:
            raise RuntimeError("hipcc failed:\n" + "\n".join("%s:\n%s" % f for f in failed))
        for path, srcs, fl in targets:
            tmp = path + ".tmp" + tag
            cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC"] + [obj_of[(s, fl)] for s in srcs]
            cmd += ["-o", tmp]
            if verbose:
                print(" ".join(cmd), flush=True)
            rc, msg = _run(cmd)
            if rc != 0:
                raise RuntimeError("link failed:\n" + msg)
            os.replace(tmp, path)
    finally:
        for o in obj_of.values():
            if os.path.exists(o):
                os.remove(o)
    return targets[0][0]


if __name__ == "__main__":
    print(build(verbose=True))
