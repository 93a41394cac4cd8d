"""Static check of the inline-asm MFMAs in the built device code.

The weight-stationary conv and the flash attention issue their MFMAs as
inline asm (so that weights can sit in AGPRs and the MFMA order is the
kernel's own). The compiler's hazard recognizer does not model those
instructions: an instruction it places after one -- a register copy made
by the register allocator, a VALU op -- may read the MFMA's result
registers before the MFMA has written them, or overwrite its SrcC while
the MFMA still reads it. CDNA3/CDNA4 need N + 3 independent wait states
between an N-pass XDL write and a VALU, memory or LDS access of the same
VGPRs (one more is counted here on top); a dependent MFMA reading exactly
the previous MFMA's result as SrcC is interlocked in hardware and exempt.

`scan(asm_text)` returns every access inside that window, in layout order
(fall-through; a kernel whose MFMAs sit right before a branch keeps its
own padding). The build runs it on the sources that hold asm MFMAs and
refuses to link on a finding.
"""
import re
import sys

_FUNC = re.compile(r"^([A-Za-z_.$][\w.$]*):[^\n]*\n(.*?)^\.Lfunc_end", re.S | re.M)
_VRANGE = re.compile(r"^([va])\[(\d+):(\d+)\]$")
_VONE = re.compile(r"^([va])(\d+)$")
# instructions whose first operand is read, not written
_NO_DST = ("buffer_store", "global_store", "flat_store", "scratch_store", "ds_write", "ds_store", "s_")


def _regs(tok):
    tok = tok.strip(",")
    m = _VRANGE.match(tok)
    if m:
        return {(m.group(1), r) for r in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = _VONE.match(tok)
    return {(m.group(1), int(m.group(2)))} if m else set()


def _passes(op):
    if "32x32" in op:
        return 8
    if "16x16" in op:
        return 4
    return 2


def _wait_states(line):
    m = re.match(r"s_nop\s+(\d+)", line)
    return int(m.group(1)) + 1 if m else 1


def scan(text):
    findings = []
    for name, body in _FUNC.findall(text):
        lines = []
        for l in body.split("\n"):
            l = l.split(";")[0].strip()
            if l and not l.endswith(":") and not l.startswith("."):
                lines.append(l)
        for i, l in enumerate(lines):
            op = l.split()[0]
            if not (op.startswith("v_mfma") or op.startswith("v_smfmac")):
                continue
            ops = l.split()[1:]
            dst = _regs(ops[0])
            src_c = _regs(ops[3]) if len(ops) > 3 else set()
            need = _passes(op) + 4
            ws = 0
            for j in range(i + 1, len(lines)):
                if ws >= need:
                    break
                lj = lines[j]
                oj = lj.split()[0]
                toks = lj.split()[1:]
                if oj.startswith("v_mfma") or oj.startswith("v_smfmac"):
                    # another MFMA: its SrcC may be this result (interlocked
                    # when exactly the same registers); A/B may not
                    if toks and (_regs(toks[1]) | _regs(toks[2])) & dst:
                        findings.append((name, l, lj))
                    ws += 1
                    continue
                if oj.startswith(_NO_DST):
                    writes, reads = set(), set().union(*[_regs(t) for t in toks]) if toks else set()
                else:
                    writes = _regs(toks[0]) if toks else set()
                    reads = set().union(*[_regs(t) for t in toks[1:]]) if len(toks) > 1 else set()
                if reads & dst or writes & (dst | src_c):
                    findings.append((name, l, lj))
                ws += _wait_states(lj)
    return findings


# instructions that read M0 without naming it
_M0_IMPLICIT = ("s_movrel", "v_movrel", "s_sendmsg", "v_interp", "ds_gws", "s_cbranch_g_fork")


def scan_m0(text):
    """The patch loads set M0 (their LDS address) and leave it clobbered,
    which is sound only while nothing else in the kernel relies on M0:
    every mention of m0 must be a plain move into it or a save of it, and
    no instruction that reads M0 implicitly may appear."""
    findings = []
    for name, body in _FUNC.findall(text):
        for l in body.split("\n"):
            l = l.split(";")[0].strip()
            if not l or l.endswith(":") or l.startswith("."):
                continue
            op = l.split()[0]
            toks = [t.strip(",") for t in l.split()[1:]]
            if op.startswith(_M0_IMPLICIT):
                findings.append((name, l, "reads M0"))
            elif "m0" in toks and not (op == "s_mov_b32" and len(toks) == 2):
                findings.append((name, l, "uses M0"))
    return findings


_VMCNT = re.compile(r"vmcnt\((\d+)\)")


def scan_vmem(text):
    """Registers of an asm load in flight. The conv's stream loads are asm
    (hidden from the compiler's wait tracking) and land only by a later
    s_waitcnt vmcnt(n) of the kernel's own; the compiler, which takes the
    registers for written at issue, may place a copy or other access of
    them before that wait and so read (or overwrite) data not yet landed.
    Within each straight-line stretch of code (from a label to the next),
    every vector-memory instruction is counted in layout order; a wait
    with vmcnt(n) retires all but the last n; an access of a register that
    an unretired load writes is a finding (a load into the same registers
    included). Loads straight into LDS write no registers. A label starts
    afresh: code reached by a branch has its own waits on every path (the
    compiler's loads), and this check is about accesses placed between an
    asm load and its wait in the same stretch."""
    findings = []
    for name, body in _FUNC.findall(text):
        pending = []  # (registers, line) per vector-memory instruction in flight, oldest first
        for l in body.split("\n"):
            l = l.split(";")[0].strip()
            if l.endswith(":"):
                pending = []
                continue
            if not l or l.startswith("."):
                continue
            op = l.split()[0]
            toks = l.split()[1:]
            if op.startswith("s_waitcnt"):
                m = _VMCNT.search(l)
                if m:
                    n = int(m.group(1))
                    pending = pending[len(pending) - n:] if n < len(pending) else pending
                continue
            regs = set().union(*[_regs(t) for t in toks]) if toks else set()
            busy = set().union(*[r for r, _ in pending]) if pending else set()
            if regs & busy:
                findings.append((name, [ln for r, ln in pending if r & regs][0], l))
            if op.startswith(("buffer_", "global_", "flat_", "scratch_")):
                dst = set()
                if op.startswith(("buffer_load", "global_load", "flat_load", "scratch_load")) and " lds" not in " " + l:
                    dst = _regs(toks[0])
                pending.append((dst, l))
    return findings


if __name__ == "__main__":
    t = open(sys.argv[1]).read()
    bad = scan(t) + scan_m0(t) + scan_vmem(t)
    for f in bad:
        print("%s: %s  ->  %s" % f)
    sys.exit(1 if bad else 0)
