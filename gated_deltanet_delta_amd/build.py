"""Build libgdn.so (HIP, gfx950) in-tree with hipcc.

    python -m gated_deltanet_delta_amd.build          # compile every source, link libgdn.so

Each source compiles to its own object under ``_build/`` (in parallel), then one hipcc link writes
``gated_deltanet_delta_amd/libgdn.so``.  The build always recompiles: it is cheap, and a stale
object would silently hide a source change.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIBRARY = os.path.join(PKG, "libgdn.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# -packed-fp32-ops off: hipcc -O3 forms packed fp32 instructions by itself from plain float code;
# keep them out of every kernel.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", f"--offload-arch={ARCH}", f"-I{INCLUDE}", f"-I{CSRC}"]

SOURCES = ["gdn_api.cpp", "recurrent.hip", "chunk_f32.hip", "chunk_mfma.hip", "norm.hip", "conv1d.hip",
           "chunk_bwd.hip", "chunk_bwd_ex.hip", "noalloc.hip"]

# Per-source code-generation options.  chunk_mfma.hip: matrix-core results go to ordinary VGPRs
# (not AGPRs), because every product there is post-processed on the vector ALU (splits, decays),
# and an AGPR result would cost one copy instruction per element.
EXTRA = {"chunk_mfma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *COMMON, *DEVICE_FLAGS, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd = [HIPCC, "-x", "hip", *COMMON, *DEVICE_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if err.strip():
        print(f"[{src}]\n{err}", file=sys.stderr)
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIBRARY + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIBRARY)
    if verbose:
        print(f"built {LIBRARY}")
    return LIBRARY


if __name__ == "__main__":
    build()
