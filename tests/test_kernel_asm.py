"""Host-side checks of the gfx950 assembly the GEMV kernels compile to.

The staging kernels load their x range straight into LDS and only then issue
their weight ring; one explicit `s_waitcnt vmcnt(N)` (N = the ring's load
count) then waits for the x loads alone, relying on vector memory loads
completing in issue order.  The GEMV's per-unit staging kernels issue one x
load with each unit's first ring slot and wait for it just before the unit's
products; each of those waits is checked against the loads issued after its
x load.  The compiler does not track LDS writes made by
such loads, so nothing else guards that wait: it is only correct if at least
N vector memory loads are issued, in straight-line code, between the last x
load and the wait, and if no LDS read comes before it.  This test compiles
the kernel sources to assembly and checks that for every instantiation.

It also checks that the kernels hold no other inline assembly.  The compiler
puts the wait states an MFMA needs after a VALU op that writes one of its
operands only where it sees that op; an asm statement that writes a VGPR
hides it, and an operand built that way was once read stale.
"""
import os
import re
import shutil
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "bit_weight_only_03_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SOURCES = ["w4_gemv.hip", "w2t.hip", "w4_gemm.hip", "w16_gemv.hip", "w4_gemv_valu.hip"]

pytestmark = pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")


def compile_asm(src, out):
    # The library's own per-source flags, so the assembly checked is the one built.
    from bit_weight_only_03_amd.build import SOURCE_FLAGS
    cmd = [HIPCC, "-O3", "-std=c++17", "--offload-arch=gfx950", "--cuda-device-only", "-S",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *SOURCE_FLAGS.get(src, []),
           f"-I{CSRC}", "-o", out, os.path.join(CSRC, src)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    return out


@pytest.fixture(scope="module")
def asm_files():
    d = tempfile.mkdtemp(prefix="w4asm")
    try:
        with ThreadPoolExecutor(len(SOURCES)) as ex:
            outs = list(ex.map(lambda s: compile_asm(s, os.path.join(d, s + ".s")), SOURCES))
        yield {s: open(o).read() for s, o in zip(SOURCES, outs)}
    finally:
        shutil.rmtree(d, ignore_errors=True)


def functions(text):
    # Kernel symbols only (each ends at its .Lfunc_end label); data symbols
    # such as a file-scope device array have no function body.
    for m in re.finditer(r"^(_Z\w+):[ \t]*; @", text, re.M):
        end = text.index(".Lfunc_end", m.start())
        yield m.group(1), [l.strip() for l in text[m.start():end].split("\n") if l.strip()]


def is_vmem_load(line):
    return re.match(r"(buffer|global)_load", line) is not None


def check_x_wait(lines, expect=1):
    """Returns None if the function's explicit x waits are safe, else a
    reason.  A kernel has one such wait per wave chain it compiles: one, or
    three for the balanced plan (its extra waves and the two halves of its
    full waves run chains of different lengths, in separate straight-line
    blocks)."""
    waits = [i for i, l in enumerate(lines)
             if re.fullmatch(r"s_waitcnt vmcnt\(\d+\)", l) and lines[i - 1].startswith(";;#ASMSTART")]
    if len(waits) != expect:
        return f"{len(waits)} explicit vmcnt waits"
    prev = 0
    for w in waits:
        n = int(re.search(r"\((\d+)\)", lines[w]).group(1))
        # Walk back from the wait through straight-line code: the n most
        # recent vector memory loads on every path into the wait must be ring
        # loads.
        count = 0
        for line in reversed(lines[:w]):
            if count >= n:
                break
            if line.startswith(";"):
                continue
            if is_vmem_load(line):
                if " lds" in line:
                    return f"only {count} loads between the last x load and vmcnt({n})"
                count += 1
            elif line.endswith(":") or line.startswith(("s_cbranch", "s_branch", "s_setpc")):
                return f"control flow after only {count} of {n} ring loads ({line})"
        if count < n:
            return f"only {count} loads before vmcnt({n})"
        # No LDS read on any path from the chain's first x load (the first
        # after the previous wait) to its wait.  (Following branches, not the
        # layout: the compiler may place another chain's blocks in between.)
        xs = [i for i in range(prev, w) if is_vmem_load(lines[i]) and " lds" in lines[i]]
        if not xs:
            return f"no x load before vmcnt({n})"
        if any(lines[i].startswith("ds_read") for i in lines_on_paths(lines, xs[0], w)):
            return "an LDS read precedes the x wait"
        prev = w
    return None


def lines_on_paths(lines, a, b):
    """Indices of the lines on some control-flow path from line a to line b
    (not past b), following fall-through and branch targets."""
    labels = {l[:-1]: i for i, l in enumerate(lines) if l.endswith(":") and not l.startswith(";")}
    seen, stack, out = set(), [a], set()
    while stack:
        i = stack.pop()
        while i < len(lines) and i not in seen:
            seen.add(i)
            if i == b:
                break
            out.add(i)
            l = lines[i]
            if l.startswith(("s_cbranch", "s_branch")):
                target = l.split()[-1]
                if target in labels:
                    stack.append(labels[target])
                if l.startswith("s_branch"):
                    break
            elif l.startswith(("s_endpgm", "s_setpc")):
                break
            i += 1
    return out


def check_unit_x_waits(lines):
    """Per-unit x staging (the GEMV's PX kernels): the i-th explicit wait
    guards the i-th x load.  With loads completing in issue order, vmcnt(n)
    covers that load only if at least n vector memory loads were issued
    after it (and before the wait).  The loads and waits sit in straight-line
    code (only the LDS reads are under branches), so program order is issue
    order.  Returns None if every wait is safe, else a reason."""
    issued = []          # "x" or "w" per vector memory load, in program order
    xs = []              # positions of the x loads in `issued`
    w = 0
    for i, line in enumerate(lines):
        if is_vmem_load(line):
            if " lds" in line:
                xs.append(len(issued))
            issued.append("x" if " lds" in line else "w")
        m = re.fullmatch(r"s_waitcnt vmcnt\((\d+)\)", line)
        if m and lines[i - 1].startswith(";;#ASMSTART"):
            n = int(m.group(1))
            if w >= len(xs):
                return f"wait {w} before its x load"
            after = len(issued) - xs[w] - 1
            if after < n:
                return f"wait {w}: vmcnt({n}) with only {after} loads after its x load"
            w += 1
    if w != len(xs):
        return f"{len(xs)} x loads but {w} waits"
    return None


def test_x_wait_covers_the_x_loads(asm_files):
    checked = 0
    bad = []
    for src, text in asm_files.items():
        for name, lines in functions(text):
            if not any(is_vmem_load(l) and " lds" in l for l in lines):
                continue            # no LDS-direct x staging in this kernel
            checked += 1
            # The GEMV's per-unit x staging (template argument PX = true)
            # has one wait per x load; every other kernel one wait in all.
            # <BF16, SPG, UPW, TPW, MX, PX = true, BAL>
            px = re.search(r"kernelILb[01]ELi\d+ELi\d+ELi\d+ELb[01]ELb1E", name) is not None
            bal = re.search(r"kernelILb[01]ELi\d+ELi\d+ELi\d+ELb[01]ELb[01]ELb1E", name) is not None
            why = check_unit_x_waits(lines) if px else check_x_wait(lines, 3 if bal else 1)
            if why:
                bad.append(f"{src} {name}: {why}")
    # every 4-bit and staged ternary instantiation stages x this way
    assert checked >= 150, checked
    assert not bad, "\n".join(bad[:20])


def test_no_inline_asm_besides_the_x_wait(asm_files):
    bad = []
    for src, text in asm_files.items():
        for name, lines in functions(text):
            for i, l in enumerate(lines):
                if l.startswith(";;#ASMSTART"):
                    body = []
                    for m in lines[i + 1:]:
                        if m.startswith(";;#ASMEND"):
                            break
                        body.append(m)
                    if body and not (len(body) == 1 and re.fullmatch(r"s_waitcnt vmcnt\(\d+\)", body[0])):
                        bad.append(f"{src} {name}: {body}")
    assert not bad, "\n".join(bad[:10])


def test_x_wait_checker_on_synthetic_code():
    # The checker itself, on hand-written sequences: one x load, two ring
    # loads, the wait for them.
    head = ["buffer_load_dwordx4 v2, s[0:3], 0 offen lds",
            "buffer_load_dwordx4 v[4:7], v1, s[4:7], 0 offen",
            "buffer_load_dword v8, v1, s[8:11], 0 offen"]
    wait = [";;#ASMSTART", "s_waitcnt vmcnt(2)", ";;#ASMEND"]
    assert check_x_wait(head + wait) is None
    # an LDS read on the way to the wait
    assert "LDS read" in check_x_wait(head[:1] + ["ds_read_b128 v[10:13], v9"] + head[1:] + wait)
    # a block that is jumped over (another chain's) is not on the path...
    jumped = head[:1] + ["s_branch .LBB0_2", ".LBB0_1:", "ds_read_b128 v[10:13], v9", ".LBB0_2:"] + head[1:]
    assert check_x_wait(jumped + wait) is None
    # ...but one reached by a branch is
    taken = head[:1] + ["s_cbranch_execz .LBB0_1", "s_branch .LBB0_2", ".LBB0_1:",
                        "ds_read_b128 v[10:13], v9", ".LBB0_2:"] + head[1:]
    assert "LDS read" in check_x_wait(taken + wait)
    # too few ring loads after the x load
    assert check_x_wait(head[:2] + wait) is not None


def test_gemv_kernel_arguments_are_preloaded(asm_files):
    # The GEMV kernels take the fields every wave needs before its first
    # load as leading arguments, compiled as preloaded into SGPRs (the
    # build's per-source flags): the kernel descriptor must say so, and the
    # hot instantiations must reach their first buffer load from the
    # preloaded entry without waiting for a scalar load (later fields may be
    # loaded on the way, as long as nothing waits for them).
    want = {"w4_gemv.hip": ("w4_gemv_kernel", 14), "w16_gemv.hip": ("w16_", 14),
            "w2t.hip": ("w2t_gemv", 10), "w4_gemm.hip": ("w4_gemm_kernel", 14)}
    bad = []
    for src, (stem, min_len) in want.items():
        text = asm_files[src]
        descs = re.findall(r"\.amdhsa_kernel (\S+)\n(.*?)\.end_amdhsa_kernel", text, re.S)
        hits = [(n, b) for n, b in descs if stem in n]
        assert hits, src
        for name, body in hits:
            m = re.search(r"\.amdhsa_user_sgpr_kernarg_preload_length (\d+)", body)
            if not m or int(m.group(1)) < min_len:
                bad.append(f"{src} {name}: preload {m.group(1) if m else None}")
    # the hot 4-bit instantiations (qkv / o_proj, gate_up, down)
    for name, lines in functions(asm_files["w4_gemv.hip"]):
        if not re.search(r"w4_gemv_kernelILb0ELi4ELi5ELi[13]ELb0ELb1ELb0E|w4_gemv_kernelILb0ELi4ELi17ELi1ELb0ELb0ELb1E", name):
            continue
        # the preloaded entry is the first label after the compatibility block
        entry = next(i for i, l in enumerate(lines) if i > 0 and re.fullmatch(r"\.LBB\d+_0:", l))
        first = next(i for i in range(entry, len(lines)) if is_vmem_load(lines[i]))
        pending = False
        for l in lines[entry:first]:
            if l.startswith("s_load"):
                pending = True
            elif pending and l.startswith("s_waitcnt") and "lgkmcnt" in l:
                bad.append(f"{name}: waits for a scalar load before its first buffer load")
                break
    assert not bad, "\n".join(bad[:10])
