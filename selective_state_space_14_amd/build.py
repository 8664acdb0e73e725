"""Build libssd.so in-tree with hipcc for gfx950.

Usage: python -m selective_state_space_14_amd.build   (always recompiles)
       python -m selective_state_space_14_amd.build --host-sanitized
           also builds _build/libssd_hostsan.so: the same library with its host
           code (the C ABI's validation in api.cpp) under AddressSanitizer and
           UndefinedBehaviorSanitizer, for the CPU-side ABI checks.  Load it with
           SSD_LIBRARY=<path> and the clang ASan runtime preloaded
           (host_sanitizer_runtime()).
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libssd.so")
SOURCES = ["api.cpp", "conv.hip", "scan.hip", "step.hip", "s6.hip", "bwd.hip"]
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    # packed fp32 (v_pk_*_f32) codegen stays off on this target
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _compile(src: str, obj_dir: str) -> str:
    obj = os.path.join(obj_dir, os.path.basename(src) + ".o")
    cmd = [HIPCC, *CFLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = True) -> str:
    obj_dir = os.path.join(HERE, "_build")
    os.makedirs(obj_dir, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, obj_dir), SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


# Host-only sanitizer flags: every -fsanitize= sits behind -Xarch_host, so no
# device code is instrumented.
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-shared-libasan"]


def host_sanitizer_runtime() -> str:
    """The clang ASan runtime (shared) that a host-sanitized build needs preloaded."""
    root = os.path.join(os.path.dirname(os.path.dirname(HIPCC)), "llvm", "lib", "clang")
    for ver in sorted(os.listdir(root), reverse=True) if os.path.isdir(root) else []:
        p = os.path.join(root, ver, "lib", "linux", "libclang_rt.asan-x86_64.so")
        if os.path.exists(p):
            return p
    raise RuntimeError(f"no libclang_rt.asan-x86_64.so under {root}")


def build_host_sanitized(verbose: bool = True) -> str:
    """_build/libssd_hostsan.so: api.cpp compiled with host ASan + UBSan, linked with the device objects."""
    obj_dir = os.path.join(HERE, "_build")
    os.makedirs(obj_dir, exist_ok=True)
    objs = []
    for src in SOURCES:
        if src == "api.cpp":
            obj = os.path.join(obj_dir, "api.hostsan.o")
            cmd = [HIPCC, *CFLAGS, "-O1", "-g", *SAN_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
            r = subprocess.run(cmd, capture_output=True, text=True)
            if r.returncode != 0:
                raise RuntimeError(f"hipcc failed on {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
            objs.append(obj)
        else:
            obj = os.path.join(obj_dir, src + ".o")
            objs.append(obj if os.path.exists(obj) else _compile(src, obj_dir))
    out = os.path.join(obj_dir, "libssd_hostsan.so")
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *SAN_FLAGS, *objs, "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    if verbose:
        print(f"built {out}")
    return out


if __name__ == "__main__":
    build()
    if "--host-sanitized" in sys.argv[1:]:
        build_host_sanitized()
    sys.exit(0)
