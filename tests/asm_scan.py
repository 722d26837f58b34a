"""Static check of compiled kernels: registers that an inline-asm load is still writing.

Several kernels issue LDS reads (and loads) from inline asm and wait for them in a
later asm statement, to keep the compiler from draining direct global->LDS copies.
The compiler treats such an asm's outputs as ready when the asm ends, so it could read
or copy one of those registers before the s_waitcnt that makes it valid.  This module
reads the gfx950 assembly of a kernel and reports every instruction that touches a
register an asm-issued LDS read or VMEM load may still be writing, counting outstanding
operations in issue order per counter (lgkmcnt: LDS reads and writes; vmcnt: VMEM loads,
stores and direct-to-LDS copies) the way s_waitcnt does.  The scan is straight-line; a
loop body (from its header label to a backward branch) is scanned twice, so operations
issued late in one iteration are tracked into the next.  Loads the compiler issued
itself are counted but not reported: it orders their uses on its own.
"""
import re


def _regs(tok):
    m = re.match(r"v\[(\d+):(\d+)\]$", tok) or re.match(r"v(\d+)$", tok)
    if not m:
        return frozenset()
    a = int(m.group(1))
    b = int(m.group(2)) if m.lastindex == 2 else a
    return frozenset(range(a, b + 1))


def _trim(queue, n):
    del queue[:max(0, len(queue) - n)]


def _scan_lines(lines, vm, lg, found):
    in_asm = False
    for ln in lines:
        s = ln.strip()
        if s.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if s.startswith(";;#ASMEND"):
            in_asm = False
            continue
        if not s or s.startswith((";", ".")):
            continue
        parts = s.split(None, 1)
        op = parts[0]
        args = [a.strip() for a in parts[1].split(";")[0].split(",")] if len(parts) > 1 else []
        if op == "s_waitcnt":
            m = re.search(r"vmcnt\((\d+)\)", parts[1])
            if m:
                _trim(vm, int(m.group(1)))
            m = re.search(r"lgkmcnt\((\d+)\)", parts[1])
            if m:
                _trim(lg, int(m.group(1)))
            continue
        if op.startswith("s_"):
            continue
        live = set()
        for q in (vm, lg):
            for regs, from_asm in q:
                if from_asm:
                    live |= regs
        use = set()
        for a in args:
            use |= _regs(a.split()[0]) if a else set()
        if use & live:
            found.append(s)
        if op.startswith(("global_load", "buffer_load")):
            vm.append((frozenset() if "lds" in op else _regs(args[0]), in_asm))
        elif op.startswith(("global_store", "buffer_store", "global_atomic", "buffer_atomic")):
            vm.append((frozenset(), False))
        elif op.startswith("ds_read"):
            lg.append((_regs(args[0]), in_asm))
        elif op.startswith("ds_"):
            lg.append((frozenset(), False))


def kernels(asm_text):
    """Names of the kernel entry points in a gfx950 assembly listing."""
    return re.findall(r"^\s*\.amdhsa_kernel\s+(\S+)", asm_text, re.M)


def scan_kernel(asm_text, name):
    """Instructions of kernel `name` that touch a register an asm-issued load may still write."""
    start = re.search(r"^" + re.escape(name) + r":", asm_text, re.M).start()
    body = asm_text[start:asm_text.index("s_endpgm", start)].splitlines()
    labels = {}
    for i, ln in enumerate(body):
        m = re.match(r"(\.LBB\w+):", ln)
        if m:
            labels[m.group(1)] = i
    found = []
    _scan_lines(body, [], [], found)
    for i, ln in enumerate(body):
        m = re.match(r"\s*s_(?:cbranch_\w+|branch)\s+(\.LBB\w+)", ln)
        if m and labels.get(m.group(1), i) < i:
            vm, lg = [], []
            loop = body[labels[m.group(1)]:i + 1]
            _scan_lines(loop, vm, lg, [])
            _scan_lines(loop, vm, lg, found)
    return found
