"""Build libmsscan.so in-tree with hipcc for gfx950.

    python -m selective_state_space_81_amd.build        # or build() from Python

Packed fp32 VALU instructions are disabled for all device code (the
``-packed-fp32-ops`` target feature); hipcc's host pass warns that it does not
know the feature, which is harmless.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmsscan.so")
# hardware rate probes used by bench.py (not part of libmsscan's C ABI)
PROBE_SRC = os.path.join(CSRC, "probe.hip")
PROBE_LIB = os.path.join(HERE, "libmsprobe.so")
SOURCES = [os.path.join(CSRC, "scan_kernels.hip"), os.path.join(CSRC, "scan_tile.hip"),
           os.path.join(CSRC, "scan_lane.hip"), os.path.join(CSRC, "scan_row.hip"),
           os.path.join(CSRC, "scan_row_wide.hip"), os.path.join(CSRC, "scan_row_dtproj.hip"),
           os.path.join(CSRC, "scan_row_ckpt.hip"),
           os.path.join(CSRC, "decode.hip"),
           os.path.join(CSRC, "conv.hip"), os.path.join(CSRC, "scan_bwd.hip"),
           os.path.join(CSRC, "bwd_wide.hip"), os.path.join(CSRC, "bwd_row.hip"),
           os.path.join(CSRC, "api.cpp"), os.path.join(CSRC, "profile.cpp"),
           os.path.join(CSRC, "noalloc.hip")]
ARCH = os.environ.get("MSSCAN_ARCH", "gfx950")


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libmsscan)")


def flags() -> list:
    return ["-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wno-unused-command-line-argument",
            "-I", os.path.join(ROOT, "include")]


def _jobs() -> int:
    """Parallel compiles: the MAX_JOBS setting if any, else the CPU count,
    at most 8 (one per source)."""
    n = os.environ.get("MAX_JOBS")
    n = int(n) if n and n.isdigit() else (os.cpu_count() or 1)
    return max(1, min(n, 8, len(SOURCES)))


def build(verbose: bool = False) -> str:
    """Compile every source (in parallel) and link libmsscan.so (always
    rebuilds)."""
    from concurrent.futures import ThreadPoolExecutor
    bdir = os.path.join(HERE, "_build")
    os.makedirs(bdir, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(bdir, os.path.basename(src) + ".o")
        lang = ["-x", "hip"]  # both files go through the HIP front end
        cmd = [hipcc()] + flags() + lang + ["-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
        return obj

    with ThreadPoolExecutor(max_workers=_jobs()) as pool:
        objs = list(pool.map(compile_one, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC"] + objs + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    build_probe(verbose)
    return LIB


def build_probe(verbose: bool = False) -> str:
    """Compile libmsprobe.so (the benchmark's rate probes) for gfx950."""
    tmp = PROBE_LIB + ".tmp"
    cmd = [hipcc()] + flags() + ["-x", "hip", "-shared", PROBE_SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {PROBE_SRC}:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, PROBE_LIB)
    return PROBE_LIB


def asm(out_dir: str) -> None:
    """Write the gfx950 assembly of the kernels (for inspecting our own code)."""
    os.makedirs(out_dir, exist_ok=True)
    for src in [x for x in SOURCES if x.endswith(".hip")]:
        out = os.path.join(out_dir, os.path.basename(src).replace(".hip", ".s"))
        cmd = [hipcc()] + flags() + ["-x", "hip", "--cuda-device-only", "-S", src, "-o", out]
        subprocess.run(cmd, check=True)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
