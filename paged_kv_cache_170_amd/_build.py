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


FLAGS = ["-O3", "-std=c++17", "-fPIC",
         # Packed fp32 instructions stay off: the compiler emits plain VALU ops instead.
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         # No wave-level aggregation of atomics: the decode's work-queue fetch is issued by one
         # lane and its result is read only when the item ends.
         "-mllvm", "-amdgpu-atomic-optimizer-strategy=None"]


def compile_command(src: str, obj: str, extra=()) -> list:
    return [hipcc(), f"--offload-arch={ARCH}", *FLAGS, "-I", os.path.join(ROOT, "include"),
            "-I", os.path.join(HERE, "csrc"), *extra, "-c", src, "-o", obj]


def link_command(objs, out_path: str) -> list:
    return [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", out_path]


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    # The host pass does not know the packed-fp32 feature and says so; that line is harmless.
    noise = [ln for ln in (res.stdout + res.stderr).splitlines() if "packed-fp32-ops" not in ln]
    return res.returncode, noise


def build(verbose: bool = False, extra=()) -> str:
    """Compile every source (one hipcc process per file, in parallel) and link the library in
    place; returns its path.  Raises CalledProcessError on failure."""
    from concurrent.futures import ThreadPoolExecutor

    out = os.path.join(HERE, LIB_NAME)
    obj_dir = os.path.join(HERE, "_build")
    os.makedirs(obj_dir, exist_ok=True)
    jobs = []
    for s in SOURCES:
        obj = os.path.join(obj_dir, os.path.splitext(s)[0] + ".o")
        jobs.append((compile_command(os.path.join(HERE, "csrc", s), obj, extra), obj))
    workers = min(len(jobs), max(1, min(16, os.cpu_count() or 1)))
    with ThreadPoolExecutor(workers) as ex:
        results = list(ex.map(lambda j: _run(j[0]), jobs))
    for (cmd, _), (rc, noise) in zip(jobs, results):
        if verbose:
            print(" ".join(cmd), flush=True)
        if rc != 0:
            sys.stderr.write("\n".join(noise) + "\n")
            raise subprocess.CalledProcessError(rc, cmd)
        if verbose and noise:
            print("\n".join(noise))
    tmp = out + ".tmp"
    cmd = link_command([o for _, o in jobs], tmp)
    rc, noise = _run(cmd)
    if verbose:
        print(" ".join(cmd), flush=True)
    if rc != 0:
        sys.stderr.write("\n".join(noise) + "\n")
        raise subprocess.CalledProcessError(rc, cmd)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
