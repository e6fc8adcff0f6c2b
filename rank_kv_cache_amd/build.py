"""Build liblra.so (the gfx950 HIP kernels + C ABI) in-tree with hipcc.

    python -m rank_kv_cache_amd.build              # compile every source, link liblra.so
    python -m rank_kv_cache_amd.build --sanitize   # host code under ASan + UBSan -> _build/sanitize/liblra.so

Object files go to ``_build/`` at the repository root; the shared library is written next to
this file so the Python binding (and a machine receiving a copy of the tree) finds it without installing.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "liblra.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
ARCH = "gfx950"

SOURCES = ["api.hip", "decode.hip", "key_expand.hip", "key_scores.hip", "precompute.hip", "prefill.hip", "read_probe.hip",
           "value_expand.hip"]
# per-source flags: the prefill kernel takes row maxima of matrix-core outputs, which are never
# signalling NaNs; without this the compiler quiets every input of every max first
SOURCE_FLAGS = {"prefill.hip": ["-fno-honor-nans"]}

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-fvisibility=hidden",
    "-ffp-contract=fast",
    "-munsafe-fp-atomics",
    # packed fp32 VALU forms stay off on this target
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the ROCm toolchain is required to build liblra")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out, flush=True)


# AddressSanitizer and UndefinedBehaviorSanitizer on the host code only (argument validation,
# workspace layouts, launch set-up): each -fsanitize= goes to the host compilation (-Xarch_host), the
# device code is built as usual. The library then needs the sanitizer runtime loaded first
# (LD_PRELOAD=`sanitizer_runtime()`); it is for CPU test runs, never shipped.
SANITIZE_DIR = os.path.join(BUILD_DIR, "sanitize")
SANITIZE_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
                  "-Xarch_host", "-g", "-Xarch_host", "-shared-libsan"]


def _compile_and_link(out_dir: str, lib_path: str, extra_flags, link_flags, verbose: bool) -> str:
    hipcc = _hipcc()
    os.makedirs(out_dir, exist_ok=True)
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(out_dir, src.replace(".hip", ".o"))
        objs.append(obj)
        cmds.append([hipcc, *HIPCC_FLAGS, *SOURCE_FLAGS.get(src, []), *extra_flags, "-c", os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(max(1, min(len(cmds), os.cpu_count() or 1))) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    tmp = lib_path + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *link_flags, "-o", tmp, *objs], verbose)
    os.replace(tmp, lib_path)
    return lib_path


def build(verbose: bool = True, extra_flags=()) -> str:
    """Compile every HIP source for gfx950 and link ``liblra.so``; returns its path."""
    return _compile_and_link(BUILD_DIR, LIB_PATH, extra_flags, (), verbose)


def build_sanitized(verbose: bool = True) -> str:
    """The same library with its host code under ASan + UBSan, as ``_build/sanitize/liblra.so``."""
    return _compile_and_link(SANITIZE_DIR, os.path.join(SANITIZE_DIR, LIB_NAME), SANITIZE_FLAGS, SANITIZE_FLAGS, verbose)


def sanitizer_runtime() -> str:
    """Path of the compiler's shared ASan runtime (to preload before a sanitized library)."""
    hipcc = _hipcc()
    clang = os.path.join(os.path.dirname(os.path.realpath(hipcc)), "..", "llvm", "bin", "clang")
    if not os.path.exists(clang):
        clang = shutil.which("clang") or "/opt/rocm/llvm/bin/clang"
    r = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], stdout=subprocess.PIPE, text=True)
    path = r.stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("the ASan runtime of the ROCm clang was not found")
    return path


if __name__ == "__main__":
    if "--sanitize" in sys.argv:
        build_sanitized(verbose="-q" not in sys.argv)
    else:
        build(verbose="-q" not in sys.argv)
