"""Build libedda.so in-tree with hipcc for gfx950.

    python -m whisper_asr_encoder_amd.build        # or: python whisper_asr_encoder_amd/build.py

Each source compiles to an object in parallel, then one hipcc link produces
whisper_asr_encoder_amd/libedda.so. Always recompiles, so a successful run
shows that the current sources compile.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libedda.so")
SOURCES = ["api.cpp", "gemm.hip", "flash_attn.hip", "verify_attn.hip", "norm_im2col.hip", "skinny.hip", "decoder_fused.hip"]
ARCH = "gfx950"

COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # Packed fp32 VALU forms are disabled for every kernel.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument", "-Wno-unused-result",
]


def hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found; a ROCm toolchain is required to build libedda.so")
    return exe


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *COMMON, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr[-4000:]}")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), 8)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc link failed:\n{r.stderr[-4000:]}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


# Host-sanitizer build of the C ABI layer, for the CPU tests of its validation paths: api.cpp's
# host code with AddressSanitizer, UndefinedBehaviorSanitizer and libstdc++ assertions (the
# device code of every file is built exactly as in the product library, unsanitized).
SAN_HOST = ["-O1", "-g", "-D_GLIBCXX_ASSERTIONS", "-Xarch_host", "-fno-omit-frame-pointer",
            "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]  # noqa: E501


def sanitizer_runtime() -> str:
    """Path of the shared ASan (+UBSan) runtime of ROCm's clang, to LD_PRELOAD into Python."""
    import glob
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise RuntimeError("no libclang_rt.asan-x86_64.so under /opt/rocm/llvm")
    return hits[-1]


def build_sanitized(out_dir: str) -> str:
    """Build libedda_san.so into out_dir (api.cpp host code sanitized, the rest as the product)."""
    os.makedirs(out_dir, exist_ok=True)

    def one(src):
        obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
        flags = [f for f in COMMON if f != "-O3"] + SAN_HOST if src == "api.cpp" else COMMON
        r = subprocess.run([hipcc(), *flags, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj],
                           capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr[-4000:]}")
        return obj

    with ThreadPoolExecutor(max_workers=min(len(SOURCES), 8)) as ex:
        objs = list(ex.map(one, SOURCES))
    lib = os.path.join(out_dir, "libedda_san.so")
    link = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-shared-libsan", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]  # noqa: E501
    r = subprocess.run([*link, *objs, "-o", lib], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc link failed:\n{r.stderr[-4000:]}")
    return lib


if __name__ == "__main__":
    build()
    sys.exit(0)
