"""Build libvsa.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

    python -m block_sparse_attention_19_amd.build_lib
    python -m block_sparse_attention_19_amd.build_lib --sanitize

Objects go to ``_build/`` at the repository root; the shared library is written
next to this file so that the Python binding finds it.

``--sanitize`` builds a checking copy of the library instead,
``_build/san/libvsa_san.so``: the host code (argument validation, layout and
workspace arithmetic, launches) instrumented with AddressSanitizer and
UndefinedBehaviorSanitizer, the device code unchanged.  It is for host-only
test runs on a machine without a GPU; load it through the binding with
``VSA_LIBRARY`` and the clang ASan runtime preloaded, e.g.

    VSA_LIBRARY=_build/san/libvsa_san.so ASAN_OPTIONS=detect_leaks=0 \
    LD_PRELOAD=$(python -m block_sparse_attention_19_amd.build_lib --asan-runtime) \
    python -m pytest tests/test_lib_host.py
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJ_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libvsa.so")
ARCH = "gfx950"

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

# Packed-fp32 VALU forms are kept out of the device code; the host pass warns
# that it does not know the feature, which is harmless.
COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Wno-unused-function", "-Wno-unused-command-line-argument",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


# Device-only flags per source: the attention kernel treats NaN as absent
# (scores are finite or -inf), which lets max/min skip NaN canonicalisation.
DEVICE_FLAGS = {
    "attn.hip": ["-Xarch_device", "-fno-honor-nans", "-Xarch_device", "-mno-amdgpu-ieee"],
}


# Host-pass sanitizers of the checking build (each flag behind -Xarch_host so
# the device code is compiled as in the product build).
SAN_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined",
            "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-g"]
SAN_DIR = os.path.join(OBJ_DIR, "san")
SAN_LIB = os.path.join(SAN_DIR, "libvsa_san.so")


def asan_runtime() -> str:
    """The clang ASan runtime matching hipcc (to preload into a Python process)."""
    base = os.path.join(os.path.dirname(os.path.dirname(HIPCC)), "lib", "llvm", "lib", "clang")
    hits = sorted(glob.glob(os.path.join(base, "*", "lib", "linux", "libclang_rt.asan-x86_64.so")))
    if not hits:
        raise RuntimeError(f"no libclang_rt.asan-x86_64.so under {base}")
    return hits[-1]


def _compile(src: str, verbose: bool, sanitize: bool = False) -> str:
    odir = SAN_DIR if sanitize else OBJ_DIR
    obj = os.path.join(odir, os.path.basename(src) + ".o")
    extra = SAN_HOST if sanitize else []
    cmd = [HIPCC, *COMMON, *extra, *DEVICE_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{out}")
    if verbose and out.strip():
        print(out, file=sys.stderr)
    return obj


def build(verbose: bool = False, sanitize: bool = False) -> str:
    """Compile every HIP source and link libvsa.so (or, with sanitize, the
    checking copy _build/san/libvsa_san.so); returns the library path."""
    os.makedirs(SAN_DIR if sanitize else OBJ_DIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, sanitize), srcs))
    lib = SAN_LIB if sanitize else LIB
    tmp = lib + ".tmp"
    link_extra = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-shared-libsan"] if sanitize else []
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *link_extra, *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    if "--asan-runtime" in sys.argv:
        print(asan_runtime())
    else:
        print(build(verbose=True, sanitize="--sanitize" in sys.argv))
