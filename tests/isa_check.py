"""Static check of the GEMM kernels' weight loads in gfx950 assembly.

The weight tiles are fetched with inline-asm vector loads that the compiler's
wait-count analysis does not track, so nothing but the kernel's own explicit
vmcnt waits protects their destination registers.  For every non-LDS global
load in every gemm_kernel this follows each control-flow path from the load
and requires that no instruction reads or writes the destination registers
before a wait that provably covers the load: `s_waitcnt vmcnt(k)` with at
least k vector-memory loads issued after it on that path (loads return in
issue order; stores are not counted, which only makes the check stricter).
A later load may write the same registers (in-order return), but must not
use them as its address.  Typical failures: a register copy the compiler
places at a loop's back edge, or epilogue code that reuses the registers of
a final, discarded prefetch before the last wait.
"""
import re
import sys

_LOAD = re.compile(r'\s*global_load_(dwordx4|dwordx2|ubyte|dword)\s+(v\[\d+:\d+\]|v\d+),')
_VMEM_LOAD = re.compile(r'(global|buffer|flat)_load_\w+')
_BRANCH = re.compile(r'(s_branch|s_cbranch_\w+)\s+(\.LBB\w+)')
_VMCNT = re.compile(r'vmcnt\((\d+)\)')


def _regs(op):
    m = re.match(r'v\[(\d+):(\d+)\]', op)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r'v(\d+)$', op)
    return {int(m.group(1))} if m else set()


def _vgprs(text):
    out = set()
    for tok in re.findall(r'v\[\d+:\d+\]|v\d+\b', text):
        out |= _regs(tok)
    return out


def _touches(ins, dest):
    parts = ins.split(None, 1)
    if len(parts) < 2:
        return False
    if _VMEM_LOAD.match(parts[0]) and 'lds' not in parts[0]:
        ops = parts[1].split(',', 1)  # a load may overwrite, but not read, the registers
        return bool(len(ops) > 1 and _vgprs(ops[1]) & dest)
    return bool(_vgprs(parts[1]) & dest)


def split_kernels(asm_text, pattern=r'gemm_kernel'):
    kernels, cur = {}, None
    for ln in asm_text.splitlines():
        m = re.match(r'^(_Z\w*' + pattern + r'\w*):', ln)
        if m:
            cur = m.group(1)
            kernels[cur] = []
            continue
        if cur is not None:
            kernels[cur].append(ln)
            if 's_endpgm' in ln:
                cur = None
    return kernels


def _hazard_from(body, labels, i, dest):
    """Depth-first over paths from instruction i; returns the offending
    instruction or None."""
    stack, seen = [(i + 1, 0)], set()
    while stack:
        j, after = stack.pop()
        while j < len(body):
            key = (j, min(after, 64))
            if key in seen:
                break
            seen.add(key)
            ins = body[j].split(';')[0].strip()
            if not ins or ins.startswith('.'):
                j += 1
                continue
            if ins.startswith('s_waitcnt'):
                m = _VMCNT.search(ins)
                if m and after >= int(m.group(1)):
                    break  # covered on this path
            if _touches(ins, dest):
                return ins
            if _VMEM_LOAD.match(ins):
                after += 1
            if ins.startswith('s_endpgm'):
                break
            mb = _BRANCH.match(ins)
            if mb and mb.group(2) in labels:
                tgt = labels[mb.group(2)]
                if mb.group(1) == 's_branch':
                    j = tgt + 1
                    continue
                stack.append((tgt + 1, after))
            j += 1
    return None


def find_hazards(asm_text):
    """Returns (number of kernels, list of hazard descriptions)."""
    kernels = split_kernels(asm_text)
    hazards = []
    for name, body in kernels.items():
        labels = {}
        for i, ln in enumerate(body):
            m = re.match(r'^(\.LBB\w+):', ln)
            if m:
                labels[m.group(1)] = i
        for i, ln in enumerate(body):
            m = _LOAD.match(ln)
            if not m or 'lds' in ln:
                continue
            bad = _hazard_from(body, labels, i, _regs(m.group(2)))
            if bad:
                hazards.append(f"{name}: '{ln.strip()}' then '{bad}' before a covering wait")
    return len(kernels), hazards


if __name__ == "__main__":
    n, hz = find_hazards(open(sys.argv[1]).read())
    print("\n".join(hz))
    print(f"{n} kernels, {len(hz)} hazards")
    sys.exit(1 if hz else 0)
