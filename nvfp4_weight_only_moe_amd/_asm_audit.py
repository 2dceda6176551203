"""Audit of the expert kernels' gfx950 assembly for the matrix-core pipeline
waits that the compiler cannot insert by itself.

The 128-row expert GEMM blocks issue their MFMAs through inline assembly
(mlp.hip, mfma_acc): the compiler then does not know those statements are
MFMAs and inserts none of the waits an MFMA needs, so the code does.  This
audit checks the generated assembly for the two waits that matter:

* a VALU instruction writing a register that an MFMA reads (a, b or the
  accumulator) needs two wait states before the MFMA;
* an MFMA result read by any non-MFMA instruction needs the MFMA's latency
  first (10 wait states covers a 16x16x32 f16 MFMA; the kernels give 24).

A wait state is one instruction issued by the wave; ``s_nop N`` gives N + 1.
Used by the CPU tests on a device-only assembly build of mlp.hip.
"""
import os
import re
import subprocess

from . import _build

VALU_TO_MFMA = 2
MFMA_TO_READ = 10


def _regs(text):
    out = set()
    for m in re.finditer(r"\b([va])(\d+)\b|\b([va])\[(\d+):(\d+)\]", text):
        if m.group(1):
            out.add(m.group(1) + m.group(2))
        else:
            out |= {m.group(3) + str(x) for x in range(int(m.group(4)), int(m.group(5)) + 1)}
    return out


def _instructions(asm, kernel):
    i = asm.index(kernel + ":")
    j = asm.index(".Lfunc_end", i)
    return [l.strip() for l in asm[i:j].splitlines()
            if l.strip() and not l.strip().startswith((";", ".")) and not l.strip().endswith(":")]


def _operands(ins):
    parts = ins.split(None, 1)
    return [p.strip() for p in parts[1].split(",")] if len(parts) > 1 else []


def _wait(ins):
    return int(ins.split()[1]) + 1 if ins.startswith("s_nop") else 1


def audit_kernel(asm, kernel):
    """Problems found in one kernel of `asm` (straight-line lookback within
    basic blocks and across fall-through; loops are unrolled in these
    kernels, so the lookback sees every predecessor that matters)."""
    body = _instructions(asm, kernel)
    problems = []
    for k, ins in enumerate(body):
        if ins.startswith("v_mfma"):
            srcs = set().union(*[_regs(o) for o in _operands(ins)[1:]])
            waits = 0
            for back in range(1, 8):
                if k - back < 0:
                    break
                prev = body[k - back]
                if waits >= VALU_TO_MFMA:
                    break
                if prev.startswith("v_") and not prev.startswith("v_mfma"):
                    ops = _operands(prev)
                    if ops and _regs(ops[0]) & srcs:
                        problems.append(f"VALU write {prev!r} -> {ins!r} after {waits} wait states")
                        break
                waits += _wait(prev)
        elif not ins.startswith(("v_mfma", "s_nop")):
            reads = set().union(*[_regs(o) for o in _operands(ins)[1:]]) if _operands(ins) else set()
            if not any(r.startswith("a") for r in reads):
                continue
            waits = 0
            for back in range(1, 40):
                if k - back < 0 or waits >= MFMA_TO_READ:
                    break
                prev = body[k - back]
                if prev.startswith("v_mfma") and _regs(_operands(prev)[0]) & reads:
                    problems.append(f"MFMA {prev!r} read by {ins!r} after {waits} wait states")
                    break
                waits += _wait(prev)
    return problems


def asm_of_mlp(out_dir):
    """Device-only gfx950 assembly of mlp.hip with the library's flags."""
    src = os.path.join(_build.CSRC, "mlp.hip")
    out = os.path.join(out_dir, "mlp.s")
    flags = [f for f in _build.HIPCC_FLAGS if f not in ("-shared", "-fPIC")]
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    cmd = [hipcc, *flags, "--cuda-device-only", "-S", "-I", _build.INCLUDE, "-I", _build.CSRC, src,
           "-o", out]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc -S failed:\n" + res.stderr[-4000:])
    return open(out).read()


def kernels(asm, pattern):
    return [n for n in re.findall(r"^(_Z[^:\s]+):", asm, re.M) if re.search(pattern, n)]
