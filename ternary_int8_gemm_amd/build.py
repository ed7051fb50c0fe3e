"""Build libbitnet_hip.so (the C ABI of include/bitnet.h) for gfx950 with hipcc.

The layer's sources under csrc/ are compiled for gfx950 only and linked into
one shared library next to this file.  No fast-math, no floating-point
contraction, and no packed fp32 instructions.  csrc/probe.hip (machine-ceiling
microbenchmarks for the benchmark script, not part of the C ABI) becomes a
second library, libbitnet_probe.so.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libbitnet_hip.so")
SOURCES = ["api.hip", "quant.hip", "gemv.hip", "gemv_mfma.hip", "gemm.hip", "epilogue.hip", "w8a16.hip"]
PROBE_SOURCE = "probe.hip"
PROBE_LIB = os.path.join(HERE, "libbitnet_probe.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-fvisibility=hidden", "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]

# Per-source additions.  The GEMM's main loop interleaves MFMAs with the VALU
# work of the operand expansion; the ILP-oriented machine scheduler overlaps
# them better than the default (occupancy-oriented) one.
SOURCE_FLAGS = {
    "gemm.hip": ["-mllvm", "-amdgpu-sched-strategy=max-ilp"],
}


def build(out=LIB, extra_flags=(), verbose=False, probe_out=PROBE_LIB):
    """Compile every source to an object (in parallel), then link the library
    (and the probe library, unless probe_out is None)."""
    from concurrent.futures import ThreadPoolExecutor

    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        cmd = [hipcc, *HIPCC_FLAGS, *SOURCE_FLAGS.get(src, []), *extra_flags, "-I", os.path.join(ROOT, "include"),
               "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), file=sys.stderr)
        subprocess.run(cmd, check=True)
        return obj

    srcs = SOURCES + ([PROBE_SOURCE] if probe_out else [])
    with ThreadPoolExecutor(max_workers=min(len(srcs), 4)) as ex:
        objs = dict(zip(srcs, ex.map(compile_one, srcs)))

    def link(obj_list, dst):
        tmp = dst + ".tmp"
        cmd = [hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *obj_list, "-o", tmp]
        if verbose:
            print(" ".join(cmd), file=sys.stderr)
        subprocess.run(cmd, check=True)
        os.replace(tmp, dst)

    link([objs[s] for s in SOURCES], out)
    if probe_out:
        link([objs[PROBE_SOURCE]], probe_out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
