"""Builds libkvhier.so (HIP sources in csrc/, gfx950) next to this file.

Usage: python -m hierarchical_sparse_kv_verify_amd.build [--force]
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libkvhier.so")
SOURCES = ["plan.hip", "copy.hip", "attn.hip", "runtime.hip"]
ARCH = "gfx950"

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH,
    # packed fp32 vector ops are kept off in every HIP translation unit
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the HIP toolchain is required to build libkvhier.so")


def _compile(src: str) -> str:
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), *HIPCC_FLAGS, "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("compile of %s failed:\n%s\n%s" % (src, " ".join(cmd), res.stderr))
    return obj


def build(force: bool = True, verbose: bool = False) -> str:
    """Compiles every HIP source (always, unless force=False and the library is
    newer than all sources) and links libkvhier.so; returns its path."""
    deps = [os.path.join(CSRC, s) for s in SOURCES] + [os.path.join(CSRC, "common.h"),
                                                       os.path.join(INCLUDE, "kv_hier.h")]
    if not force and os.path.exists(LIB) and all(os.path.getmtime(LIB) >= os.path.getmtime(d) for d in deps):
        return LIB
    os.makedirs(OBJDIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=4) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [_hipcc(), "-shared", "-fPIC", "--offload-arch=" + ARCH, *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), res.stderr))
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


SAN_DIR = os.path.join(OBJDIR, "san")
SAN_LIB = os.path.join(SAN_DIR, "libkvhier.so")
# host-side sanitizers only: each flag applies to the host compilation of the
# HIP sources (device code is built as usual)
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def build_sanitized() -> str:
    """libkvhier.so with AddressSanitizer and UBSan in its host code, for the
    CPU-reachable paths (argument checks, failed creation, null handles); run
    it with the clang sanitizer runtime preloaded.  Returns its path."""
    os.makedirs(SAN_DIR, exist_ok=True)

    def comp(src):
        obj = os.path.join(SAN_DIR, os.path.splitext(src)[0] + ".o")
        cmd = [_hipcc(), *HIPCC_FLAGS, *SAN_FLAGS, "-g", "-I", INCLUDE, "-I", CSRC, "-c",
               os.path.join(CSRC, src), "-o", obj]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError("compile of %s failed:\n%s\n%s" % (src, " ".join(cmd), res.stderr))
        return obj

    with concurrent.futures.ThreadPoolExecutor(max_workers=4) as ex:
        objs = list(ex.map(comp, SOURCES))
    cmd = [_hipcc(), "-shared", "-fPIC", "--offload-arch=" + ARCH, *SAN_FLAGS, "-shared-libsan", *objs,
           "-o", SAN_LIB]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), res.stderr))
    return SAN_LIB


def sanitizer_runtime() -> str:
    """The clang AddressSanitizer runtime the sanitized build links against."""
    res = subprocess.run([_hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                         text=True)
    path = res.stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("clang sanitizer runtime not found (%r)" % path)
    return path


if __name__ == "__main__":
    build(force="--no-force" not in sys.argv, verbose=True)
