"""Builds libipttt.so (the HIP kernels + C ABI) in-tree for gfx950 with hipcc.

Usage: python -m test_weight_mlp_amd.build [--jobs N] [--sanitize]

--sanitize builds a second copy, _build/sanitize/libipttt.so, whose host code
(argument validation, workspace layout, segment tables, launch set-up) is
instrumented with AddressSanitizer and UndefinedBehaviorSanitizer; device
code is compiled as usual.  It is for CPU tests of the host paths only, run
with the ASan runtime preloaded (see sanitizer_runtime()).
"""
from __future__ import annotations

import argparse
import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libipttt.so")
SAN_OBJDIR = os.path.join(OBJDIR, "sanitize")
SAN_LIB = os.path.join(SAN_OBJDIR, "libipttt.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")

SOURCES = ["seg.hip", "gated_z.hip", "target.hip", "delta.hip", "apply.hip", "backward.hip", "noalloc.hip",
           "api.cpp"]

# Packed-fp32 instructions stay off: plain fp32 code is what every kernel here
# is written and tested as.
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
          f"-I{INCLUDE}", f"-I{CSRC}"]
DEVICE = ["--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# Host-only instrumentation: every sanitizer flag goes through -Xarch_host so
# that no GPU code is built with it.
SANITIZE = [a for f in ("-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined",
                        "-fno-omit-frame-pointer", "-shared-libasan") for a in ("-Xarch_host", f)]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def _compile(src: str, sanitize: bool = False) -> str:
    obj = os.path.join(SAN_OBJDIR if sanitize else OBJDIR, os.path.splitext(src)[0] + ".o")
    path = os.path.join(CSRC, src)
    cmd = [hipcc()] + COMMON + (["-g"] + SANITIZE if sanitize else [])
    if src.endswith(".hip"):
        cmd += DEVICE + ["-c", path, "-o", obj]
    else:
        cmd += ["-x", "c++", "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include", "-c", path, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{err}")
    return obj


def build(jobs: int = 8, verbose: bool = False, sanitize: bool = False) -> str:
    lib = SAN_LIB if sanitize else LIB
    os.makedirs(SAN_OBJDIR if sanitize else OBJDIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(lambda src: _compile(src, sanitize), SOURCES))
    tmp = lib + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", "--offload-arch=gfx950"] + (SANITIZE if sanitize else []) + \
        ["-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}")
    return lib


def sanitizer_runtime() -> str:
    """Path of the compiler's shared ASan runtime, which a process that loads
    the sanitized library must preload."""
    res = subprocess.run([hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = res.stdout.strip()
    if res.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError(f"ASan runtime not found ({res.stdout.strip()} {res.stderr.strip()})")
    return path


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=min(8, os.cpu_count() or 1))
    ap.add_argument("--sanitize", action="store_true", help="host-sanitized copy under _build/sanitize")
    args = ap.parse_args(argv)
    build(args.jobs, verbose=True, sanitize=args.sanitize)
    return 0


if __name__ == "__main__":
    sys.exit(main())
