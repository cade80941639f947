"""Build libst.so (HIP, gfx950) in-tree: temporal_attention_amd/libst.so.

    python temporal_attention_amd/build.py      # or build() from __graft_entry__

(Run it as a script, not as `-m temporal_attention_amd.build`: importing the
package loads the existing libst.so, which may predate the sources.)

Each .hip source compiles to an object under temporal_attention_amd/_build/
(in parallel), then one shared library is linked next to this file.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libst.so")
BUILD = os.path.join(PKG, "_build")
ARCH = "gfx950"

# Packed fp32 VALU forms are disabled: hipcc generates them from ordinary float code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall", "-Wno-unused-function"]
# Attention scores are finite or -inf by construction (never NaN), so max/min
# need no NaN-quieting of their operands.
PER_FILE = {"attn_bf16.hip": ["-fno-honor-nans"]}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def torch_lib_dir() -> str:
    """Directory of the HIP runtime torch ships; libst.so must share that runtime with torch."""
    import importlib.util
    spec = importlib.util.find_spec("torch")
    if spec is None or spec.origin is None:
        raise RuntimeError("torch is not importable")
    d = os.path.join(os.path.dirname(spec.origin), "lib")
    if not os.path.exists(os.path.join(d, "libamdhip64.so")):
        raise RuntimeError(f"no libamdhip64.so under {d}")
    return d


def clangxx() -> str:
    for cand in ("/opt/rocm/llvm/bin/clang++", "/opt/rocm/lib/llvm/bin/clang++", shutil.which("amdclang++")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("clang++ of ROCm not found")


def sources() -> list[str]:
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src)[:-4] + ".o")
    cmd = [hipcc(), *COMMON, *DEVICE_FLAGS, *PER_FILE.get(os.path.basename(src), []), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    """Compile every HIP source for gfx950 and link libst.so; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = OUT + ".tmp"
    # Link against the HIP runtime torch loads (same soname), not a second copy:
    # device memory and streams come from torch and must belong to the same runtime.
    tl = torch_lib_dir()
    cmd = [clangxx(), "-shared", "-fPIC", *objs, "-o", tmp, f"-L{tl}", "-l:libamdhip64.so", f"-Wl,-rpath,{tl}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT} from {len(srcs)} sources")
    return OUT


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
