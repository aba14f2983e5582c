"""Scan of the gfx950 assembly hipcc writes for the library's kernels.

Matrix-core results (v_mfma_*) are not interlocked against the vector
instructions that read them: the compiler must leave enough independent
instructions (wait states, s_nop N counting N + 1) between a product and the
first read of its destination.  The scan walks every path out of every
product -- fall-through and taken branches alike -- to the first instruction
that reads one of its destination registers (a vector ALU, LDS or memory
instruction, or another product reading it as an A/B operand; the same
registers as the accumulator input of the next product in a chain is
forwarded by the hardware and not counted), and records the wait states in
between and whether the path took a branch.

It reads only assembly built here from this repository's sources.
"""
import functools
import os
import re
import subprocess
import tempfile

_BRANCHES = ("s_cbranch_scc0", "s_cbranch_scc1", "s_cbranch_vccz", "s_cbranch_vccnz", "s_cbranch_execz",
             "s_cbranch_execnz")
_VREG = re.compile(r"^v\[(\d+):(\d+)\]$|^v(\d+)$")


def _vregs(op):
    m = _VREG.match(op.strip())
    if not m:
        return set()
    if m.group(3) is not None:
        return {int(m.group(3))}
    return set(range(int(m.group(1)), int(m.group(2)) + 1))


def device_asm(src, flags, hipcc="/opt/rocm/bin/hipcc"):
    """The device assembly of one source file, compiled with the library's flags
    (compiled once per test session and source)."""
    return _device_asm(src, tuple(flags), hipcc, os.path.getmtime(src))


@functools.lru_cache(maxsize=None)
def _device_asm(src, flags, hipcc, _mtime):
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, "k.s")
        cmd = [hipcc] + [f for f in flags if f != "-fPIC"] + ["--cuda-device-only", "-S", src, "-o", out]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("hipcc -S failed on %s:\n%s" % (src, r.stderr[-4000:]))
        with open(out) as f:
            return f.read()


def kernels(asm):
    """(symbol, instruction lines) for every kernel in an assembly file."""
    lines = asm.splitlines()
    out = []
    for i, line in enumerate(lines):
        m = re.match(r"^(_Z\w+):", line)
        if not m:
            continue
        body = []
        for j in range(i + 1, len(lines)):
            body.append(lines[j].split(";")[0].strip())
            if body[-1].startswith("s_endpgm"):
                break
        out.append((m.group(1), body))
    return out


def _parse(line):
    if not line or line.startswith(".") or line.endswith(":"):
        return None
    parts = line.split(None, 1)
    ops = [o.strip() for o in parts[1].split(",")] if len(parts) > 1 else []
    return parts[0], ops


def mfma_reads(body, max_wait=24):
    """For every product in a kernel body: (opcode, wait states, took_branch)
    for the first read of its destination on each path out of it."""
    labels = {l[:-1]: i for i, l in enumerate(body) if re.match(r"^\.LBB\w+:$", l)}
    found = []
    for i, line in enumerate(body):
        p = _parse(line)
        if not p or not p[0].startswith("v_mfma"):
            continue
        op, ops = p
        dst = _vregs(ops[0])
        seen = set()
        stack = [(i + 1, 0, False)]
        while stack:
            j, d, branched = stack.pop()
            while j < len(body) and d <= max_wait:
                q = _parse(body[j])
                j += 1
                if q is None:
                    continue
                qop, qops = q
                if qop.startswith("s_endpgm"):
                    break
                if qop.startswith("v_mfma"):
                    reads = set().union(*[_vregs(o) for o in qops[1:3]]) if len(qops) >= 3 else set()
                    if len(qops) >= 4 and _vregs(qops[3]) != dst:
                        reads |= _vregs(qops[3])
                    writes = _vregs(qops[0])
                elif qop.startswith(("v_", "ds_", "global_", "buffer_", "flat_", "scratch_")):
                    stores = qop.startswith(("ds_write", "ds_store", "global_store", "buffer_store", "flat_store",
                                             "scratch_store"))
                    swaps = "permlane" in qop and "swap" in qop
                    first = 0 if (stores or swaps) else 1
                    reads = set().union(set(), *[_vregs(o) for o in qops[first:]])
                    writes = set() if stores else _vregs(qops[0]) if qops else set()
                else:
                    reads, writes = set(), set()
                if reads & dst:
                    found.append((op, d, branched))
                    break
                if writes & dst:
                    break  # overwritten before any read
                if qop in _BRANCHES or qop == "s_branch":
                    tgt = qops[0] if qops else None
                    if tgt in labels and (tgt, d) not in seen:
                        seen.add((tgt, d))
                        stack.append((labels[tgt] + 1, d + 1, True))
                    if qop == "s_branch":
                        break
                m = re.match(r"s_nop\s+(\d+)", body[j - 1])
                d += int(m.group(1)) + 1 if m else 1
    return found
