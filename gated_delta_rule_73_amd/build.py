"""Build libgdr.so in-tree with hipcc for gfx950.

Each source is compiled to an object under ``_build/`` (in parallel), then
linked into ``gated_delta_rule_73_amd/libgdr.so``.  Run as a module:
``python -m gated_delta_rule_73_amd.build``.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libgdr.so")
ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -packed-fp32-ops: keep the compiler from forming packed fp32 VALU ops.
DEVICE_FLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
                "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-Wno-unused-command-line-argument"]


# Host-side AddressSanitizer + UndefinedBehaviorSanitizer build (device code
# is compiled as usual): -Xarch_host applies each flag to the host pass only.
SANITIZE_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
SANITIZE_DIR = os.path.join(BUILD, "sanitize")
SANITIZE_LIB = os.path.join(SANITIZE_DIR, "libgdr.so")


def sources():
    return sorted(f for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def _compile(src: str, sanitize: bool = False) -> str:
    obj = os.path.join(SANITIZE_DIR if sanitize else BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *DEVICE_FLAGS, *(SANITIZE_FLAGS if sanitize else []), "-I", os.path.join(ROOT, "include"), "-c",
           os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(jobs: int | None = None, verbose: bool = False, sanitize: bool = False) -> str:
    """Compile every source and link libgdr.so; with sanitize, a host-ASan/UBSan
    variant under _build/sanitize/ instead (it needs the clang ASan runtime
    preloaded into the process that loads it)."""
    os.makedirs(SANITIZE_DIR if sanitize else BUILD, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(len(srcs), max(1, min(16, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, sanitize), srcs))
    out = SANITIZE_LIB if sanitize else LIB
    tmp = out + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out} from {len(srcs)} sources")
    return out


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
