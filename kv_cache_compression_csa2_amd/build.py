"""Build the CSA2 HIP library in-tree for gfx950: ``python -m kv_cache_compression_csa2_amd.build``.

Compiles every source under ``csrc/`` with hipcc into ``_build/`` and links
``libcsa2.so`` next to this file.  Always recompiles (each file takes
seconds); sources are compiled in parallel.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libcsa2.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

ARCH = "gfx950"
CFLAGS = [
    "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-Wall", "-Wno-unused-function",
    # keep the compiler from emitting packed float32 VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def sources() -> list[str]:
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *CFLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    warn = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip())
    if warn:
        print(warn, file=sys.stderr)
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources")
    return LIB


# Host files built with AddressSanitizer and UndefinedBehaviorSanitizer for
# the CPU check (each -fsanitize applies to the host code only; device code
# is built as usual)
HOST_SOURCES = ("abi.cpp", "plan.cpp", "trace.cpp", "noalloc.hip")
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer", "-g"]


def build_host_check() -> str:
    """Build csrc_check/abi_host_check.cpp against the library's host files
    built with the sanitizers (the other sources' objects from build());
    returns the executable's path."""
    san = os.path.join(BUILD, "san")
    os.makedirs(san, exist_ok=True)
    objs = []
    for f in HOST_SOURCES:
        obj = os.path.join(san, f + ".o")
        cmd = [HIPCC, *CFLAGS, *SAN_FLAGS, "-c", os.path.join(CSRC, f), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
        objs.append(obj)
    others = [os.path.join(BUILD, os.path.basename(src) + ".o") for src in sources()
              if os.path.basename(src) not in HOST_SOURCES]
    missing = [o for o in others if not os.path.exists(o)]
    if missing:
        build(verbose=False)
    driver = os.path.join(ROOT, "kv_cache_compression_csa2_amd", "csrc_check", "abi_host_check.cpp")
    drv_obj = os.path.join(san, "abi_host_check.o")
    cmd = [HIPCC, *CFLAGS, *SAN_FLAGS, "-c", driver, "-o", drv_obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    exe = os.path.join(san, "abi_host_check")
    cmd = [HIPCC, f"--offload-arch={ARCH}", *SAN_FLAGS, drv_obj, *objs, *others, "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return exe


if __name__ == "__main__":
    build()
