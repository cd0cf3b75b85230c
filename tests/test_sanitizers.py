"""AddressSanitizer + UndefinedBehaviorSanitizer runs on the CPU.

1. The oracle (plain C) built with -fsanitize=address,undefined runs its own
   pins (tests/test_oracle.py) in a child process with the sanitizer
   runtimes preloaded; any report aborts the child.
2. The host side of libqmoe (argument validation, workspace sizing, packing)
   built the same way (the device code unsanitized, and never launched here)
   runs the ABI and packer tests.
A sanitizer finding fails the child with a non-zero status; its report is in
the assertion message.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]
ENV_SAN = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1", "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _run(cmd, env):
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, (r.stdout[-4000:] + r.stderr[-4000:])
    return r


def _gcc_runtime(name):
    return subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True, text=True).stdout.strip()


def test_oracle_under_asan_ubsan(tmp_path):
    from oracle import ref
    lib = str(tmp_path / "libqmref_san.so")
    cmd = [c for c in ref.gcc_cmd(lib) if c != "-O2"]
    subprocess.run(cmd[:1] + SAN + cmd[1:], check=True)
    env = dict(os.environ, **ENV_SAN, QMREF_LIB=lib,
               LD_PRELOAD=_gcc_runtime("libasan.so") + ":" + _gcc_runtime("libubsan.so"))
    _run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "tests/test_oracle.py"], env)


def _clang_asan_runtime():
    hits = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    return hits[0] if hits else None


@pytest.mark.skipif(_clang_asan_runtime() is None, reason="clang ASan runtime not found")
def test_host_abi_under_asan_ubsan(tmp_path):
    csrc = os.path.join(ROOT, "int4_expert_gemv_amd", "csrc")
    inc = ["-I", os.path.join(ROOT, "include")]
    import concurrent.futures

    def hip(src):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        # the host code sanitized (the device code is compiled as usual, unsanitized)
        subprocess.run(["/opt/rocm/bin/hipcc", "--offload-arch=gfx950", "-std=c++17", "-fPIC", "-O1", "-g",
                        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                        "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                        "-Xarch_host", "-fno-sanitize-recover=all", *inc, "-c", "-o", obj, src],
                       check=True, capture_output=True)
        return obj

    with concurrent.futures.ThreadPoolExecutor(8) as ex:
        objs = list(ex.map(hip, sorted(glob.glob(os.path.join(csrc, "*.hip")))))
    for src in sorted(glob.glob(os.path.join(csrc, "*.cpp"))):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        subprocess.run(["/opt/rocm/llvm/bin/clang++", "-std=c++17", "-fPIC", *SAN, *inc, "-c", "-o", obj, src],
                       check=True)
        objs.append(obj)
    lib = str(tmp_path / "libqmoe_san.so")
    subprocess.run(["/opt/rocm/llvm/bin/clang++", "-shared", "-shared-libasan", *SAN[:2], "-o", lib, *objs,
                    "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"], check=True)
    env = dict(os.environ, **ENV_SAN, QMOE_LIB_PATH=lib, LD_PRELOAD=_clang_asan_runtime())
    _run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "tests/test_abi.py",
          "tests/test_pack.py"], env)
