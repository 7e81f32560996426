"""Compile the HIP sources into libllm.so for gfx950 (in-tree)."""
from __future__ import annotations

import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libllm.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

FLAGS = ["-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-Wall", "-Wno-unused-function",
         "-I", os.path.join(ROOT, "include"),
         # packed fp32 VALU forms are kept out of the generated code
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _compile(src: str, obj: str) -> None:
    cmd = [HIPCC, *FLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed on {os.path.basename(src)}")
    noise = [l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l and l.strip()]
    if noise:
        sys.stderr.write("\n".join(noise) + "\n")


def build(verbose: bool = True) -> str:
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = [os.path.join(objdir, os.path.basename(s) + ".o") for s in srcs]
    jobs = min(len(srcs), int(os.environ.get("MAX_JOBS", "8")))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        list(ex.map(lambda so: _compile(*so), zip(srcs, objs)))
    tmp = OUT + f".tmp{os.getpid()}"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("link failed")
    os.replace(tmp, OUT)
    # the counter-run driver: a plain C++ program on the C ABI
    drv = os.path.join(HERE, "profile_driver")
    cmd = ["g++", "-O2", "-std=c++17", "-Wall", "-I", os.path.join(ROOT, "include"),
           os.path.join(CSRC, "profile_driver.cpp"), "-o", drv + f".tmp{os.getpid()}",
           "-L", HERE, "-lllm", "-Wl,-rpath,$ORIGIN"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("profile_driver build failed")
    os.replace(drv + f".tmp{os.getpid()}", drv)
    if verbose:
        print(f"built {OUT}")
    return OUT


if __name__ == "__main__":
    build()
