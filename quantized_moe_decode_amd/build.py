"""Build libhfq4moe.so in-tree with hipcc for gfx950.

    python quantized_moe_decode_amd/build.py   (or build() from Python)

(Run it as a script: importing the package would load the library first.)

Every source under csrc/ is compiled into one shared library next to this
file (libhfq4moe.so, the decode library); the latency probes under probes/
into a second one (libhfq4probe.so, measurement only, and once more as
libhfq4probe_kp.so with the kernel arguments preloaded into scalar
registers).  All HIP code is built with packed-FP32 instructions disabled.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libhfq4moe.so")
SOURCES = ["api.cpp", "pack.hip", "gemv.hip", "moe.hip", "moe_mfma.hip", "turbo.hip"]
HOST_SOURCES = ["host_cpu.cpp", "placement.cpp", "turbo_tables.cpp"]   # host-only C++
PROBE_LIB = os.path.join(HERE, "libhfq4probe.so")
# the probes once more with kernel arguments preloaded into scalar registers
# (measured against the default argument loads by the launch-chain probe)
PROBE_LIB_KP = os.path.join(HERE, "libhfq4probe_kp.so")
KP_FLAGS = ["-mllvm", "-amdgpu-kernarg-preload-count=16"]
PROBE_SOURCES = [os.path.join(HERE, "probes", "probe.hip")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
]


HOST_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function"]


def _host_objects(verbose):
    objs = []
    for src in HOST_SOURCES:
        obj = os.path.join(HERE, os.path.splitext(src)[0] + ".host.o")
        cmd = [HIPCC] + HOST_FLAGS + ["-x", "c++", "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            sys.stderr.write(r.stdout + r.stderr)
            raise RuntimeError("compiling %s failed" % src)
        objs.append(obj)
    return objs


def _hipcc(srcs, lib, verbose, objs=(), extra=()):
    tmp = lib + ".tmp"
    cmd = [HIPCC] + FLAGS + list(extra) + ["-x", "hip"] + srcs + ["-x", "none"] + list(objs) + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed building %s" % os.path.basename(lib))
    os.replace(tmp, lib)


def build(verbose=False):
    objs = _host_objects(verbose)
    _hipcc([os.path.join(CSRC, s) for s in SOURCES], LIB, verbose, objs)
    for o in objs:
        os.remove(o)
    _hipcc(PROBE_SOURCES, PROBE_LIB, verbose)
    _hipcc(PROBE_SOURCES, PROBE_LIB_KP, verbose, extra=KP_FLAGS)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
