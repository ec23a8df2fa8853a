"""Host AddressSanitizer + UndefinedBehaviorSanitizer check of the library's host
code and of the CPU input generator.

Builds a copy of libmoe_nvfp4.so whose host code (argument validation, workspace
layout, launch set-up, the C-ABI glue) is instrumented with ASan and UBSan,
and a copy of synth/synth_cpu.c instrumented the same way, both under
_build/asan/; then runs the CPU test suite (pytest -m "not gpu") against them
in a child process with the sanitizer runtime preloaded.  Any report stops the
run with a non-zero status.  Device code is compiled as usual and never runs
here (there is no GPU on a build host); GPU code is never built with a
sanitizer.

    python -m nvfp4_block_scaled_softmax_amd.sanitize
"""
import concurrent.futures as cf
import glob
import os
import subprocess
import sys

from . import build as b

ROOT = os.path.dirname(b.HERE)
OUT = os.path.join(ROOT, "_build", "asan")
LLVM = os.path.join(os.path.dirname(os.path.dirname(b.HIPCC)), "llvm")
CLANG = os.path.join(LLVM, "bin", "clang")
# host-only instrumentation: every sanitizer flag applies to the host pass
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
FLAGS = ["-O1", "-g", "-std=c++17", "-fPIC", f"--offload-arch={b.ARCH}",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wno-unused-command-line-argument"]


def _run(cmd):
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"failed: {' '.join(cmd)}\n{p.stdout}{p.stderr}")


def _obj(src):
    obj = os.path.join(OUT, os.path.basename(src) + ".o")
    _run([b.HIPCC, *FLAGS, *HOST_SAN, "-c", src, "-o", obj])
    return obj


def asan_runtime():
    rt = glob.glob(os.path.join(LLVM, "lib", "clang", "*", "lib", "linux", "libclang_rt.asan-x86_64.so"))
    if not rt:
        raise RuntimeError("clang's ASan runtime (libclang_rt.asan-x86_64.so) not found under " + LLVM)
    return rt[0]


def build_libs(jobs=None):
    os.makedirs(OUT, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(b.CSRC, "*.hip")))
    with cf.ThreadPoolExecutor(jobs or min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(_obj, srcs))
    lib = os.path.join(OUT, "libmoe_nvfp4_asan.so")
    _run([b.HIPCC, "-shared", "-fPIC", f"--offload-arch={b.ARCH}", "-Xarch_host", "-fsanitize=address",
          "-Xarch_host", "-fsanitize=undefined", "-shared-libsan", *objs, "-o", lib])
    # the generator, with clang so that one sanitizer runtime serves the process
    # (OpenMP off: the same arithmetic per element, one thread)
    synth = os.path.join(OUT, "libsynth_cpu_asan.so")
    _run([CLANG, "-O1", "-g", "-fPIC", "-shared", "-ffp-contract=off", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-shared-libsan",
          os.path.join(ROOT, "synth", "synth_cpu.c"), "-o", synth])
    return lib, synth


def main():
    lib, synth = build_libs()
    env = dict(os.environ, LD_PRELOAD=asan_runtime(), MOE_NVFP4_LIB=lib, SYNTH_CPU_LIB=synth,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    args = sys.argv[1:] or ["tests", "-m", "not gpu", "-x", "-q", "-p", "no:cacheprovider"]
    return subprocess.run([sys.executable, "-m", "pytest", *args], cwd=ROOT, env=env).returncode


if __name__ == "__main__":
    sys.exit(main())
