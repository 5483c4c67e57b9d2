"""Build libwhisper_mi355x.so for gfx950 with hipcc (in-tree, no JIT cache).

Every HIP source is compiled with packed-fp32 instruction selection turned
off; objects are built in parallel and linked into one shared library next to
this file.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libwhisper_mi355x.so")
SOURCES = ["gemm.hip", "decode_gemm.hip", "attention.hip", "cross_enc.hip", "elementwise.hip", "logmel.hip", "peak.hip",
           "api.cpp"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wno-unused-result", "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def _compile(src):
    obj = os.path.join(BUILD, src.replace(".", "_") + ".o")
    cmd = [HIPCC, *FLAGS, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), 8)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


ASAN_LIB = os.path.join(BUILD, "asan", "libwhisper_mi355x_asan.so")


def asan_runtime():
    """The compiler's AddressSanitizer runtime, to be preloaded into the
    (uninstrumented) Python process that loads the ASan build."""
    clang = os.path.join(os.path.dirname(os.path.realpath(HIPCC)), "..", "llvm", "bin", "clang")
    r = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isfile(path):
        raise RuntimeError("AddressSanitizer runtime not found")
    return path


def build_asan(verbose=False):
    """The same library with the host side of the C ABI (api.cpp: argument
    checks, sizing, planning) built with AddressSanitizer; device code and the
    other objects are the ordinary ones. Only host code is instrumented: the
    flag is given to the host compilation alone."""
    if not all(os.path.exists(os.path.join(BUILD, s.replace(".", "_") + ".o")) for s in SOURCES):
        build()
    out = os.path.dirname(ASAN_LIB)
    os.makedirs(out, exist_ok=True)
    obj = os.path.join(out, "api_cpp_asan.o")
    cmd = [HIPCC, *FLAGS, "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer", "-x", "hip",
           "-c", os.path.join(CSRC, "api.cpp"), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc (ASan) failed for api.cpp:\n{r.stderr}")
    objs = [os.path.join(BUILD, s.replace(".", "_") + ".o") for s in SOURCES if s != "api.cpp"] + [obj]
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", "-Xarch_host", "-fsanitize=address", "-shared-libasan",
           *objs, "-o", ASAN_LIB]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link (ASan) failed:\n{r.stderr}")
    if verbose:
        print("built", ASAN_LIB)
    return ASAN_LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
