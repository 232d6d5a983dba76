"""Static check of the loads the kernels issue in inline asm.

Some coding loops issue their loads in asm and wait for them with an explicit
s_waitcnt, so that the wait does not also cover the stores issued after those
loads.  The compiler does not know such a load is still in flight: were it to
read, copy or reuse the destination register before the wait, the result
would be wrong on the GPU with no error.  This test compiles the kernels for
gfx950 and walks the generated code: from each asm load up to the wait that
covers it (counting, in issue order, the memory operations issued after the
load), no instruction may reference the load's destination registers, and
there may be no label or branch (so the walk is the execution order).
"""
import os
import re
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "lossless_compression_float_amd", "csrc", "uzip_kernels.hip")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

VMEM = re.compile(r"^\s*(buffer|global|flat|scratch)_(load|store|atomic)")
WAIT = re.compile(r"^\s*s_waitcnt\b(.*)")
VREG = re.compile(r"\bv(\d+)\b|\bv\[(\d+):(\d+)\]")
BRANCH = re.compile(r"^\s*(s_branch|s_cbranch\w*|s_setpc_b64|s_endpgm)\b")


def _regs(text):
    out = set()
    for a, lo, hi in VREG.findall(text):
        if a:
            out.add(int(a))
        else:
            out.update(range(int(lo), int(hi) + 1))
    return out


def check_asm(lines):
    """Returns a list of violations in one kernel's instruction lines."""
    bad = []
    pending = []  # [dest registers, memory operations issued after it, line]
    in_asm = False
    for n, raw in enumerate(lines):
        line = raw.split(";")[0] if not raw.strip().startswith(";;#ASM") else raw
        s = raw.strip()
        if s.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if s.startswith(";;#ASMEND"):
            in_asm = False
            continue
        if not s or s.startswith(";") or s.startswith("."):
            if s.startswith(".LBB") and pending:
                bad.append("label %s with asm loads in flight (from line %d)" % (s, pending[0][2]))
            continue
        body = line.strip()
        if not body:
            continue
        w = WAIT.match(body)
        if w:
            m = re.search(r"vmcnt\((\d+)\)", w.group(1))
            if m or w.group(1).strip() in ("0", ""):
                cnt = int(m.group(1)) if m else 0
                pending = [p for p in pending if p[1] < cnt]
            continue
        if BRANCH.match(body) and pending:
            bad.append("branch '%s' with asm loads in flight (from line %d)" % (body, pending[0][2]))
        if VMEM.match(body):
            is_asm_load = in_asm and "_load" in body.split()[0]
            operands = body.split(None, 1)[1] if " " in body else ""
            first, _, rest = operands.partition(",")
            refs = _regs(rest) if is_asm_load else _regs(operands)
            for p in pending:
                if p[0] & refs:
                    bad.append("line %d '%s' reads a register loaded at line %d" % (n, body, p[2]))
            for p in pending:
                p[1] += 1
            if is_asm_load:
                pending.append([_regs(first), 0, n])
            continue
        refs = _regs(body)
        for p in pending:
            if p[0] & refs:
                bad.append("line %d '%s' touches a register loaded at line %d" % (n, body, p[2]))
    if pending:
        bad.append("kernel ends with asm loads in flight")
    return bad


def count_asm_loads(lines):
    n, in_asm = 0, False
    for raw in lines:
        s = raw.strip()
        if s.startswith(";;#ASMSTART"):
            in_asm = True
        elif s.startswith(";;#ASMEND"):
            in_asm = False
        elif in_asm and VMEM.match(s) and "_load" in s.split()[0]:
            n += 1
    return n


def _kernels(asm_text):
    """(name, instruction lines) of every kernel in an assembly listing."""
    out = []
    cur = None
    for raw in asm_text.splitlines():
        m = re.match(r"^(_Z\w+):\s*(;.*)?$", raw)
        if m:
            cur = (m.group(1), [])
            out.append(cur)
            continue
        if cur is not None:
            if raw.startswith(".Lfunc_end"):
                cur = None
                continue
            cur[1].append(raw)
    return out


def test_checker_catches_a_read_before_the_wait():
    lines = [";;#ASMSTART", "buffer_load_dword v4, v1, s[0:3], 0 offen", ";;#ASMEND",
             "buffer_store_short v2, v3, s[4:7], 0 offen", "v_mov_b32_e32 v5, v4",
             ";;#ASMSTART", "s_waitcnt vmcnt(1)", ";;#ASMEND"]
    assert check_asm(lines)
    ok = [";;#ASMSTART", "buffer_load_dword v4, v1, s[0:3], 0 offen", ";;#ASMEND",
          "buffer_store_short v2, v3, s[4:7], 0 offen", ";;#ASMSTART", "s_waitcnt vmcnt(1)", ";;#ASMEND",
          "v_mov_b32_e32 v5, v4"]
    assert check_asm(ok) == []
    # a wait that leaves the load outstanding does not clear it
    short = [";;#ASMSTART", "buffer_load_dword v4, v1, s[0:3], 0 offen", ";;#ASMEND",
             ";;#ASMSTART", "s_waitcnt vmcnt(1)", ";;#ASMEND", "v_mov_b32_e32 v5, v4"]
    assert check_asm(short)
    branch = [";;#ASMSTART", "buffer_load_dword v[4:5], v1, s[0:3], 0 offen", ";;#ASMEND",
              "s_cbranch_scc1 .LBB0_3", ";;#ASMSTART", "s_waitcnt vmcnt(0)", ";;#ASMEND"]
    assert check_asm(branch)


@pytest.mark.timeout(600)
def test_kernels_never_touch_asm_loads_in_flight():
    inc = ["-I" + os.path.join(ROOT, "include"), "-I" + os.path.dirname(SRC)]
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, "k.s")
        subprocess.check_call([HIPCC, "-O3", "-std=c++17", "--offload-arch=gfx950", "--cuda-device-only", "-S",
                               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"] + inc +
                              ["-o", out, SRC], stderr=subprocess.DEVNULL)
        text = open(out).read()
    kernels = _kernels(text)
    assert any("k_encode" in k for k, _ in kernels)
    for name, lines in kernels:
        bad = check_asm(lines)
        assert not bad, "%s:\n  " % name + "\n  ".join(bad[:10])
        if "k_encode" in name:
            assert count_asm_loads(lines) > 0, name  # the check is not vacuous
