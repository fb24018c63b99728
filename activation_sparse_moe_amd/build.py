"""Build libblockffn.so (HIP, gfx950) in-tree with hipcc.

    python -m activation_sparse_moe_amd.build

Compiles every ``csrc/*.hip`` to an object under ``_build/`` and links them
into ``activation_sparse_moe_amd/libblockffn.so``.  Every HIP source is built
with packed-fp32 code generation disabled.

The library carries a digest of the sources it was built from
(``blockffn_build_digest()``); the binding refuses a library whose digest
differs from that of the sources beside it, so a stale build cannot be
tested or timed by mistake.
"""
from __future__ import annotations

import glob
import hashlib
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libblockffn.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"), shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; set ROCM_PATH")


COMPILE_FLAGS = [
    "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-fvisibility=hidden",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def library_sources() -> list:
    """Every file the library is built from: csrc/* and include/blockffn.h."""
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.h")) +
                  [os.path.join(ROOT, "include", "blockffn.h")])


def library_digest() -> str:
    """sha256 prefix over the library's sources (relative name, then contents, in name order)."""
    h = hashlib.sha256()
    for path in library_sources():
        h.update(os.path.relpath(path, ROOT).encode())
        h.update(b"\0")
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _compile(src: str, digest: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc(), *COMPILE_FLAGS, f'-DBLOCKFFN_BUILD_DIGEST="{digest}"', "-I", os.path.join(ROOT, "include"),
           "-I", CSRC, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    digest = library_digest()
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda src: _compile(src, digest), srcs))
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = [hipcc(), "-shared", f"--offload-arch={ARCH}", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources, digest {digest}")
    return LIB


HOSTSAN_LIB = os.path.join(PKG, "libblockffn_hostsan.so")
# AddressSanitizer and UndefinedBehaviorSanitizer on the host code only (the C ABI's validation and
# launch set-up); the gfx950 code is built as usual.  Each -fsanitize= goes right after -Xarch_host.
HOSTSAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer", "-g"]


def build_host_sanitized(verbose: bool = False) -> str:
    """libblockffn_hostsan.so: the library with ASan + UBSan in its host code, for CPU tests of the C ABI
    (load it with the compiler's ASan runtime preloaded).  Same sources, same digest."""
    san_dir = os.path.join(BUILD, "hostsan")
    os.makedirs(san_dir, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    digest = library_digest()

    def compile_one(src: str) -> str:
        obj = os.path.join(san_dir, os.path.basename(src) + ".o")
        cmd = [hipcc(), *COMPILE_FLAGS, *HOSTSAN_FLAGS, f'-DBLOCKFFN_BUILD_DIGEST="{digest}"', "-I",
               os.path.join(ROOT, "include"), "-I", CSRC, "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
        return obj

    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(compile_one, srcs))
    tmp = HOSTSAN_LIB + f".tmp{os.getpid()}"
    cmd = [hipcc(), "-shared", f"--offload-arch={ARCH}", "-fPIC", "-Xarch_host", "-fsanitize=address",
           "-Xarch_host", "-fsanitize=undefined", "-shared-libsan", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, HOSTSAN_LIB)
    if verbose:
        print(f"built {HOSTSAN_LIB}")
    return HOSTSAN_LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
