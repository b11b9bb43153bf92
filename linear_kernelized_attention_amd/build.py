"""Build libfavor.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

Also builds _build/libfavor_hostsan.so: the same library with its host
dispatch (favor_api.cpp: argument checks, workspace sizing, the host ORF
construction) compiled with AddressSanitizer and UndefinedBehaviorSanitizer
on the host side only, linked with the normal kernel objects.  The ABI
tests load it in a child process (tests/test_abi_hostsan.py).

Usage: python -m linear_kernelized_attention_amd.build [--jobs N]
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libfavor.so")
HOSTSAN_LIB = os.path.join(BUILD, "libfavor_hostsan.so")
HOSTSAN_SRC = "favor_api.cpp"

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")

COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    "-mcode-object-version=5",
    # packed fp32 instructions are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else ["-x", "hip"]
    cmd = [HIPCC, *COMMON, *lang, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(jobs: int | None = None, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(8, len(srcs))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources")
    return LIB


# Host-side sanitizer flags: each -fsanitize option is scoped to the host
# compilation with -Xarch_host (the device code is built as usual).
HOSTSAN = [
    "-Xarch_host", "-fsanitize=address",
    "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-sanitize-recover=all",
    "-Xarch_host", "-fno-omit-frame-pointer",
]


def asan_runtime() -> str:
    """Path of the compiler's shared AddressSanitizer runtime (to preload)."""
    r = subprocess.run([HIPCC, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                       text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("the compiler's AddressSanitizer runtime was not found")
    return path


def build_hostsan() -> str:
    """libfavor_hostsan.so: favor_api.cpp with host ASan/UBSan, linked with
    the kernel objects of the last build()."""
    objs = [os.path.join(BUILD, os.path.basename(s) + ".o") for s in sources()
            if os.path.basename(s) != HOSTSAN_SRC]
    missing = [o for o in objs if not os.path.exists(o)]
    if missing:
        raise RuntimeError(f"run build() first; missing {missing}")
    obj = os.path.join(BUILD, "favor_api_hostsan.o")
    flags = [f for f in COMMON if f != "-O3"]
    cmd = [HIPCC, *flags, "-O1", "-g", *HOSTSAN, "-x", "hip", "-c",
           os.path.join(CSRC, HOSTSAN_SRC), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    tmp = HOSTSAN_LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *HOSTSAN[:4], "-shared-libsan",
           "-o", tmp, obj, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, HOSTSAN_LIB)
    return HOSTSAN_LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    args = ap.parse_args()
    build(args.jobs, verbose=True)
    build_hostsan()
    sys.exit(0)
