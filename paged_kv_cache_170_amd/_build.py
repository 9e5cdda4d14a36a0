"""Compiles the HIP sources into libpagedkv.so for gfx950 (in place, next to this file)."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SOURCES = ["status.hip", "cache.hip", "decode.hip", "prefill.hip", "mixed.hip", "block_manager.cpp", "scheduler.cpp"]
LIB_NAME = "libpagedkv.so"
ARCH = "gfx950"


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


def command(out_path: str, extra=()) -> list:
    srcs = [os.path.join(HERE, "csrc", s) for s in SOURCES]
    return [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
            # Packed fp32 instructions stay off: the compiler emits plain VALU ops instead.
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            # No wave-level aggregation of atomics: the decode's work-queue fetch is issued by one
            # lane and its result is read only when the item ends.
            "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
            "-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc"),
            *extra, *srcs, "-o", out_path]


def build(verbose: bool = False) -> str:
    """Compile every source; returns the library path.  Raises CalledProcessError on failure."""
    out = os.path.join(HERE, LIB_NAME)
    tmp = out + ".tmp"
    cmd = command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # The host pass does not know the packed-fp32 feature and says so; that line is harmless.
    noise = [ln for ln in (res.stdout + res.stderr).splitlines() if "packed-fp32-ops" not in ln]
    if res.returncode != 0:
        sys.stderr.write("\n".join(noise) + "\n")
        raise subprocess.CalledProcessError(res.returncode, cmd)
    if verbose and noise:
        print("\n".join(noise))
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
