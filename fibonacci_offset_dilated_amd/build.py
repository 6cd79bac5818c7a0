"""Build the HIP library libfibattn.so in-tree for gfx950 (hipcc, no JIT cache).

Usage: python -m fibonacci_offset_dilated_amd.build [--jobs N]
Each .hip source is compiled to an object in parallel, then linked into one shared library
next to this file. Packed-fp32 instructions are disabled in device code.
"""
from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libfibattn.so")
BUILD = os.path.join(PKG, "_build")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def flags():
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-ffp-contract=fast",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            # MFMA results in ordinary VGPRs: the kernels read them back with VALU code
            "-mllvm", "-amdgpu-mfma-vgpr-form",
            "-Wno-unused-command-line-argument", "-I", CSRC]


def build(jobs: int = 8, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))
    cc = hipcc()

    def compile_one(src):
        obj = os.path.join(BUILD, src[:-4] + ".o")
        cmd = [cc, *flags(), "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
        if verbose and r.stderr.strip():
            print(r.stderr, file=sys.stderr)
        return obj

    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(compile_one, srcs))
    tmp = OUT + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, OUT)
    build_probe()
    return OUT


PROBE_SRC = os.path.join(PKG, "probe", "memprobe.hip")
PROBE_OUT = os.path.join(PKG, "probe", "memprobe")


def build_probe() -> str:
    """The memory-delivery probe (a measurement aid that bench.py --memprobe runs; not part
    of the library)."""
    cmd = [hipcc(), *[f for f in flags() if f not in ("-fPIC",)], PROBE_SRC, "-o", PROBE_OUT + ".tmp"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on memprobe.hip:\n{r.stdout}\n{r.stderr}")
    os.replace(PROBE_OUT + ".tmp", PROBE_OUT)
    return PROBE_OUT


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=8)
    ap.add_argument("-v", "--verbose", action="store_true")
    args = ap.parse_args()
    print(build(args.jobs, args.verbose))


if __name__ == "__main__":
    main()
