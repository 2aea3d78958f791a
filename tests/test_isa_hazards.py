"""Wait-state check of the direct-to-LDS loads in the built library.

CPU only: disassembles the gfx950 code objects of libspd.so with ROCm's
llvm-objdump (code built here) and checks each `global_load_lds_*`.

The loads are issued from inline assembly, which the compiler does not look
inside, so it pads none of their hazards.  A vector-memory instruction must
follow a VALU write of an SGPR it reads by at least 5 wait states, and an LDS
DMA must follow a write of M0 by at least one.  The helper that issues the
loads copies the address base and M0 with scalar moves right before each load;
this test checks, in the machine code actually shipped, that both operands of
every such load were last written by a scalar instruction inside that short
window, with a wait state after the M0 write, and that no VALU instruction
wrote either of them in between.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "shared_prompt_dedup_amd", "libspd.so")
OBJDUMP = "/opt/rocm/llvm/bin/llvm-objdump"

pytestmark = pytest.mark.skipif(not (os.path.exists(LIB) and os.path.exists(OBJDUMP)),
                                reason="libspd.so or ROCm's llvm-objdump missing")

WINDOW = 6   # instructions looked back from each load


def _regs(tok):
    tok = tok.strip()
    m = re.fullmatch(r"s\[(\d+):(\d+)\]", tok)
    if m:
        return {f"s{i}" for i in range(int(m.group(1)), int(m.group(2)) + 1)}
    if re.fullmatch(r"s\d+", tok) or tok == "m0":
        return {tok}
    if tok == "vcc":
        return {"vcc_lo", "vcc_hi"}
    return set()


def _sgpr_dests(op, args):
    """SGPRs (and M0) an instruction writes, as far as this check needs."""
    if op.startswith("s_") and not op.startswith(("s_nop", "s_waitcnt", "s_cbranch", "s_branch", "s_barrier",
                                                  "s_store", "s_cmp", "s_bitcmp", "s_setprio", "s_sleep")):
        return _regs(args[0]) if args else set()
    if op.startswith(("v_readlane", "v_readfirstlane")) or (op.startswith("v_cmp") and op.endswith("_e64")):
        return _regs(args[0])
    if op.startswith("v_cmp"):
        return {"vcc_lo", "vcc_hi"}
    if re.match(r"v_(add|sub|subrev)_co_|v_(addc|subb|subbrev)_co_|v_div_scale|v_mad_(u64_u32|i64_i32)", op):
        return _regs(args[1]) if len(args) > 1 else set()
    return set()


def _code_objects(tmp):
    lib = os.path.join(tmp, "libspd.so")
    shutil.copy(LIB, lib)
    subprocess.run([OBJDUMP, "--offloading", lib], cwd=tmp, check=True, capture_output=True)
    objs = sorted(os.path.join(tmp, f) for f in os.listdir(tmp) if f.endswith("amdgcn-amd-amdhsa--gfx950"))
    assert objs, "no gfx950 code object in libspd.so"
    return objs


def _instructions(obj):
    out = subprocess.run([OBJDUMP, "-d", "--no-show-raw-insn", obj], check=True, capture_output=True,
                         text=True).stdout
    fn, seq = None, []
    for line in out.splitlines():
        m = re.match(r"^[0-9a-f]+ <(.+)>:$", line)
        if m:
            fn = m.group(1)
            continue
        text = line.split("//")[0].strip()
        if fn and text and not text.endswith(":"):
            parts = text.split(None, 1)
            args = [a.strip() for a in parts[1].split(",")] if len(parts) > 1 else []
            seq.append((fn, parts[0], args))
    return seq


def test_lds_dma_operands_written_by_scalar_moves(tmp_path):
    checked, bad = 0, []
    for obj in _code_objects(str(tmp_path)):
        seq = _instructions(obj)
        for n, (fn, op, args) in enumerate(seq):
            if not op.startswith("global_load_lds"):
                continue
            checked += 1
            assert len(args) >= 2 and args[1] != "off", f"{fn}: LDS DMA without an SGPR base: {op} {args}"
            pending = _regs(args[1]) | {"m0"}
            waits, m0_waits, problem = 0, None, None
            for k in range(n - 1, max(n - 1 - WINDOW, -1), -1):
                kfn, kop, kargs = seq[k]
                if kfn != fn:
                    break
                dests = _sgpr_dests(kop, kargs) & pending
                if dests and not kop.startswith("s_"):
                    problem = f"{kop} {', '.join(kargs)} writes {sorted(dests)} {waits} wait states before the load"
                    break
                if "m0" in dests:
                    m0_waits = waits
                pending -= dests
                if not pending:
                    break
                waits += int(kargs[0], 0) + 1 if kop == "s_nop" and kargs else 1
            if problem is None and pending:
                problem = f"{sorted(pending)} not written by a scalar instruction within {WINDOW} instructions"
            if problem is None and m0_waits < 1:
                problem = "M0 written with no wait state before the load"
            if problem:
                bad.append(f"{fn}: {problem}")
    assert checked > 0, "no direct-to-LDS loads found: the attention kernels are missing from the library"
    assert not bad, "\n".join(bad[:20])
