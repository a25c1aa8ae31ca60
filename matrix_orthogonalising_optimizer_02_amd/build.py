"""Build libmuon_rocm.so (HIP, gfx950) in-tree with hipcc.

Every source under csrc/ is compiled for gfx950 and linked into one shared
library next to this file; the Python binding loads it from there.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys
import tempfile

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG_DIR, "csrc")
LIB_NAME = "libmuon_rocm.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
ARCH = "gfx950"

SOURCES = ["k_elementwise.hip", "k_gemm.hip", "k_adamw.hip", "k_spectrum.hip", "noalloc.hip", "k_ceiling.hip",
           "muon_abi.cpp"]

COMMON_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    f"--offload-arch={ARCH}",
    # packed fp32 VALU ops stay off: scalar fp32 code is what the kernels are written for
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # the GEMM epilogues index the accumulator array with loop variables; they must
    # unroll completely or the accumulators end up in scratch memory
    "-mllvm", "-pragma-unroll-threshold=1000000",
]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libmuon_rocm.so")


# Host-side AddressSanitizer and UndefinedBehaviorSanitizer (the device code is built
# as usual: -Xarch_host keeps every sanitizer option on the host compilation).
SANITIZE_HOST_FLAGS = [
    "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
    "-Xarch_host", "-g",
]
SANITIZED_LIB_PATH = os.path.join(PKG_DIR, "libmuon_rocm_hostsan.so")


def build(verbose: bool = False, defines=(), out: str = LIB_PATH, host_sanitize: bool = False) -> str:
    """Compile all sources and link the shared library; returns its path.

    `defines` are extra -D options (tile-configuration constants); `out` places the
    library elsewhere, e.g. to compare configurations side by side. host_sanitize
    builds the host code with AddressSanitizer and UndefinedBehaviorSanitizer, for
    CPU-only runs of the C ABI's validation paths; load it with the sanitizer runtime
    preloaded (sanitizer_runtime()).
    """
    cc = hipcc()
    dflags = [f"-D{d}" for d in defines] + (SANITIZE_HOST_FLAGS if host_sanitize else [])
    tmp = tempfile.mkdtemp(prefix="muon_build_")
    try:
        cmds, objs = [], []
        for src in SOURCES:
            path = os.path.join(CSRC, src)
            obj = os.path.join(tmp, os.path.splitext(src)[0] + ".o")
            lang = ["-x", "hip"] if src.endswith(".hip") else []
            cmds.append([cc, *COMMON_FLAGS, *dflags, *lang, "-c", path, "-o", obj])
            objs.append(obj)
        # the sources compile independently; at most `jobs` compilers at once
        jobs = max(1, min(len(cmds), int(os.environ.get("MAX_JOBS", "0") or 0) or os.cpu_count() or 1, 8))
        with concurrent.futures.ThreadPoolExecutor(jobs) as pool:
            for f in [pool.submit(_run, c, verbose) for c in cmds]:
                f.result()
        out_tmp = out + ".tmp"
        link_san = ["-shared-libsan", *SANITIZE_HOST_FLAGS[:4]] if host_sanitize else []
        _run([cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *link_san, *objs, "-o", out_tmp], verbose)
        os.replace(out_tmp, out)
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    return out


def sanitizer_runtime() -> str:
    """Path of the compiler's shared AddressSanitizer runtime (it carries the
    UndefinedBehaviorSanitizer handlers too), to preload for the sanitized library."""
    res = subprocess.run([os.path.join(os.path.dirname(hipcc()), "..", "llvm", "bin", "clang"),
                          "-print-file-name=libclang_rt.asan-x86_64.so"], stdout=subprocess.PIPE, text=True)
    path = res.stdout.strip()
    if res.returncode != 0 or not os.path.exists(path):
        raise RuntimeError("the compiler's AddressSanitizer runtime was not found")
    return os.path.realpath(path)


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature; harmless
    lines = [ln for ln in res.stdout.splitlines() if "packed-fp32-ops" not in ln]
    if res.returncode != 0:
        raise RuntimeError("build failed:\n" + " ".join(cmd) + "\n" + "\n".join(lines))
    if verbose and lines:
        print("\n".join(lines), flush=True)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
