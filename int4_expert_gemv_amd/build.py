"""Build libqmoe.so (hand-written HIP for gfx950) in-tree with hipcc.

Every csrc/*.hip file is compiled for gfx950 only (packed-fp32 instructions
disabled) into an object under _build/, in parallel, and the objects are
linked into one shared object that exports the C ABI of include/qmoe.h.
Run `python -m int4_expert_gemv_amd.build`.
"""
import concurrent.futures
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libqmoe.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function", "-I", os.path.join(ROOT, "include")]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def host_sources():
    """Host-only C++ (packing and validation): built with g++."""
    return sorted(glob.glob(os.path.join(CSRC, "*.cpp")))


HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-fvisibility=hidden", "-Wall", "-I", os.path.join(ROOT, "include")]


# The sources the decode kernels are built from (the fused gate+up kernel
# whose counters the bench reports, and the down kernel).
DECODE_SOURCES = ("device.hpp", "launch.hpp", "planes.hpp", "moe_decode.hip", "qmoe.hip")


# The sources of the prefill kernels.
PREFILL_SOURCES = ("device.hpp", "launch.hpp", "moe_prefill.hip", "qmoe.hip")


def source_digest(names=None):
    """sha256 over kernel sources and the public header (in name order), with
    the compile flags: a hardware-counter summary taken from a build is valid
    only while this digest is unchanged.  `names` limits it to those files of
    the kernel directory (the ones a given kernel is built from); default all."""
    import hashlib
    h = hashlib.sha256()
    srcs = glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.hpp"))
    if names is not None:
        srcs = [f for f in srcs if os.path.basename(f) in names]
    files = sorted(srcs + glob.glob(os.path.join(ROOT, "include", "*.h")))
    for f in files:
        h.update(os.path.basename(f).encode() + b"\0")
        with open(f, "rb") as fh:
            h.update(fh.read())
    h.update(" ".join(FLAGS[:-2]).encode())
    return h.hexdigest()[:16]


def _compile(src, extra):
    obj = os.path.join(BUILD, os.path.basename(src).rsplit(".", 1)[0] + ".o")
    if src.endswith(".cpp"):
        cmd = ["g++", *HOST_FLAGS, *extra, "-c", "-o", obj, src]
    else:
        cmd = [HIPCC, *FLAGS, *extra, "-c", "-o", obj, src]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops' is not a recognized" not in l]
    if r.returncode:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, "\n".join(msgs)))
    return obj, msgs


def build(out=LIB, verbose=False, extra=(), jobs=None):
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources() + host_sources()
    jobs = jobs or min(len(srcs), os.cpu_count() or 4, 16)
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(lambda s: _compile(s, list(extra) if not s.endswith(".cpp") else []), srcs))
    for obj, msgs in results:
        if verbose and msgs:
            print("\n".join(msgs))
    tmp = out + ".tmp%d" % os.getpid()
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp,
                    *[o for o, _ in results]], check=True)
    os.replace(tmp, out)
    if verbose:
        print("built", out, flush=True)
    return out


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
