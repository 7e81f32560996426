"""The counter waits of the prefill product, checked on its generated code.

`gemm_tile256_xreg_kernel` loads its X fragments with instructions issued
from inline assembly, which the compiler's own wait-count tracking does not
see.  Its explicit counter waits alone must ensure that a fragment has
landed before any instruction reads the fragment's registers, and that no
instruction writes those registers while the load may still be writing them
(the load would then overwrite whatever the compiler placed there, an
address for instance).  This test compiles the kernel's source for gfx950
and simulates, for every instantiation, the vector-memory counter over the
prologue, several trips of the main loop and the code after it (the next
tile's first loads, the epilogue): vector memory operations complete in
issue order, and `s_waitcnt vmcnt(N)` leaves at most the N newest
outstanding.  No GPU is used.
"""
import os
import re
import shutil
import subprocess

import pytest

from llama_decoder_forward_amd import build as bld

HIPCC = bld.HIPCC
SRC = os.path.join(bld.CSRC, "gemm.hip")
KERNEL = "gemm_tile256_xreg_kernel"

REG = re.compile(r"\bv\[(\d+):(\d+)\]|\bv(\d+)\b")
# first operand not written: stores, LDS writes, LDS-DMA copies (their first
# operand is an address), compares and lane reads (scalar destinations)
NO_VDST = ("global_store", "buffer_store", "ds_write", "global_load_lds", "buffer_load_lds", "s_",
           "v_cmp", "v_readfirstlane", "v_readlane")
VMEM = ("global_", "buffer_", "flat_")


def regs(text):
    out = set()
    for m in REG.finditer(text):
        if m.group(3):
            out.add(int(m.group(3)))
        else:
            out.update(range(int(m.group(1)), int(m.group(2)) + 1))
    return out


def operands(line):
    parts = line.split(None, 1)
    return parts[0], (parts[1].split(",") if len(parts) > 1 else [])


def kernels(asm):
    """name -> (prologue, loop body, epilogue) instruction lists.

    The k-loop is the innermost loop (the product walks its tiles in an outer
    loop).  The prologue is the code laid out before it; the epilogue runs
    from the loop's exit to the end of the kernel in layout order (a superset
    of every path: the next tile's first loads, this tile's epilogue, the
    final wait)."""
    out = {}
    for name in re.findall(r"^(_ZN\w*" + KERNEL + r"\w*):", asm, re.M):
        body = asm[asm.index(name + ":"):]
        body = body[:body.index(".Lfunc_end")]
        lines = [l.strip() for l in body.splitlines()[1:]]
        mark = next(i for i, l in enumerate(lines) if "Inner Loop Header" in l)
        head = next(i for i in range(mark, -1, -1) if lines[i].startswith(".LBB") and ":" in lines[i])
        label = lines[head].split(":")[0]
        back = next(i for i in range(head + 1, len(lines))
                    if lines[i].startswith("s_cbranch") and lines[i].split()[-1] == label)
        exit_ = back + 1
        if lines[exit_].startswith("s_branch"):  # the loop exits by a jump over other blocks
            target = lines[exit_].split()[-1]
            exit_ = next(i for i, l in enumerate(lines) if l.startswith(target + ":"))
        out[name] = (keep(lines[:head]), keep(lines[head + 1:back]), keep(lines[exit_:]))
    return out


def keep(lines):
    """Instructions with a mark: "A " for those written in inline assembly
    (between the compiler's ASMSTART / ASMEND comments), "C " for the
    compiler's own."""
    out, inasm = [], False
    for l in lines:
        if ";;#ASMSTART" in l:
            inasm = True
        elif ";;#ASMEND" in l:
            inasm = False
        core = l.split(";")[0].strip()
        if core and not core.startswith(".") and not core.endswith(":"):
            out.append(("A " if inasm else "C ") + core)
    return out


def simulate(prologue, loop, epilogue, trips=5):
    """Violations of the register rules above over the prologue, `trips`
    trips of the loop and the whole epilogue."""
    pending = []  # (vector memory operation index, registers an assembly load writes)
    bad = []
    seq = [l if l[:2] in ("A ", "C ") else "A " + l for l in prologue + loop * trips + epilogue]
    for n, marked in enumerate(seq):
        line = marked[2:]
        if line.startswith("s_endpgm"):
            break
        op, ops = operands(line)
        if op.startswith("s_waitcnt"):
            m = re.search(r"vmcnt\((\d+)\)", line)
            if m:
                del pending[:max(0, len(pending) - int(m.group(1)))]
            continue
        if op.startswith(("s_", ";")):
            continue
        writes = set() if op.startswith(NO_VDST) or not ops else regs(ops[0])
        reads = regs(",".join(ops if op.startswith(NO_VDST) else ops[1:]))
        for _, dst in pending:
            if reads & dst:
                bad.append(("reads a register a load is still writing", n, line))
            if writes & dst:
                bad.append(("writes a register a load is still writing", n, line))
        if op.startswith(VMEM):
            # every vector memory operation counts; the destination registers
            # of the compiler's own loads are the compiler's to protect
            pending.append((n, writes if "load" in op and marked.startswith("A ") else set()))
    return bad


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("needs hipcc")
    out = str(tmp_path_factory.mktemp("asm") / "gemm.s")
    r = subprocess.run([HIPCC, *bld.FLAGS, "--cuda-device-only", "-S", SRC, "-o", out],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    with open(out) as f:
        return f.read()


def test_prefill_product_waits_cover_assembly_loads(asm):
    ks = kernels(asm)
    # five epilogue kinds x two token-tile widths
    assert len(ks) == 10, sorted(ks)
    for name, (pro, loop, epi) in ks.items():
        assert any(l[2:].startswith("v_mfma") for l in loop), name
        # the X fragments come from assembly loads inside the loop
        assert sum(l.startswith("A global_load_dwordx4") for l in loop) > 0, name
        bad = simulate(pro, loop, epi)
        assert not bad, (name, bad[:3])


def test_checker_catches_a_missing_wait():
    """The simulation itself: a load whose register is read with no wait
    between, and a register written while a load into it is outstanding."""
    pro = ["global_load_dwordx4 v[4:7], v[0:1], off", "s_waitcnt vmcnt(1)"]
    loop = ["v_mfma_f32_16x16x32_f16 v[8:11], v[12:15], v[4:7], v[8:11]"]
    assert simulate(pro, loop, [])
    pro = ["global_load_dwordx4 v[4:7], v[0:1], off", "global_load_dwordx4 v[16:19], v[2:3], off",
           "s_waitcnt vmcnt(1)"]
    assert not simulate(pro, loop, [])
    epi = ["v_add_u32_e32 v18, 1, v0", "s_waitcnt vmcnt(0)"]
    assert simulate(pro, loop, epi)
