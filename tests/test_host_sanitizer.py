"""The library's host logic (argument checks, call-protocol state, the
memory plan, the paged cache's block bookkeeping and table refresh) run
under AddressSanitizer with the HIP runtime and the kernel launchers
replaced by host stand-ins (tests/hostcheck), on the CPU.  The stand-in
launchers check that every KV-cache address a kernel would compute lies in
the cache allocation and that every paged position has a block, so a
missing table refresh or an uncovered position fails here instead of on a
GPU."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.mark.skipif(not os.path.exists(HIPCC) or shutil.which("g++") is None, reason="needs hipcc and g++")
def test_host_logic_under_asan(tmp_path):
    src = os.path.join(HERE, "hostcheck")
    host = os.path.join(ROOT, "llama_decoder_forward_amd", "csrc", "llm_host.hip")
    objs = []
    for f in (host, os.path.join(src, "runtime_stub.hip")):
        o = str(tmp_path / (os.path.basename(f) + ".o"))
        subprocess.run([HIPCC, "-x", "hip", "--offload-host-only", "-std=c++17", "-g", "-O1",
                        "-Xarch_host", "-fsanitize=address", "-c", f, "-o", o],
                       check=True, capture_output=True)
        objs.append(o)
    drv = str(tmp_path / "driver.o")
    subprocess.run(["g++", "-g", "-O1", "-fsanitize=address", "-c", os.path.join(src, "driver.cpp"), "-o", drv],
                   check=True, capture_output=True)
    exe = str(tmp_path / "hostcheck")
    subprocess.run(["g++", "-no-pie", "-fsanitize=address", drv, *objs, "-o", exe], check=True, capture_output=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0 and r.stdout.strip().endswith("done"), r.stdout[-3000:] + r.stderr[-3000:]
