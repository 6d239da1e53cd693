"""Build-time check of the device code around the HBM -> LDS copies.

The kernels issue their HBM -> LDS copies (global_load_lds_dwordx4) as inline
asm, and the compiler applies none of its hazard rules to inline asm.  Two
rules of the gfx9 family (gfx950 included) concern these copies, and the
compiler enforces both for the copies it generates itself (it puts s_nop 4
after a v_readfirstlane that writes a copy's base, and s_nop 0 after an m0
write):

  * a VMEM instruction that reads an SGPR written by a VALU instruction
    (v_readlane / v_readfirstlane, a compare or a carry-out into an SGPR)
    needs 5 wait states between the two.  The compiler can restore a spilled
    SGPR from a VGPR lane with v_readlane right before a copy; the copy then
    reads a stale base address and faults;
  * a copy reads m0 (its LDS destination); an SALU write of m0 needs 1 wait
    state before it.  The copies' asm begins with s_nop 0 for this.

check_asm() scans the assembly the compiler emits for a source (hipcc -S) and
returns every copy that violates either rule on some path into it: the
straight-line code before it and, through branch targets, the code before
every branch that jumps to its block.  Wait states are counted as the
hardware counts them: one per instruction, N + 1 for s_nop N.
"""

import re

VALU_SGPR_WAIT = 5  # VALU writes SGPR -> VMEM reads that SGPR
M0_WAIT = 1         # SALU writes M0 -> LDS-DMA reads M0

_COPY = re.compile(r"^global_load_lds_dword\w*\s+v\d+,\s*s\[(\d+):(\d+)\]")
_COPY_ANY = re.compile(r"^global_load_lds_dword\w*\b")
_BRANCH = re.compile(r"^s_(c?branch\w*)\s+(\.\w+)")
_LABEL = re.compile(r"^(\.?[\w.$]+):")
_FUNC = re.compile(r"^([A-Za-z_][\w.$]*):")
_SREG = re.compile(r"^s(\d+)$|^s\[(\d+):(\d+)\]$")
# VOP3b forms: the second operand is an SGPR destination (carry or flag out)
_VOP3B = ("v_add_co_", "v_sub_co_", "v_subrev_co_", "v_addc_co_", "v_subb_co_", "v_subbrev_co_",
          "v_div_scale_", "v_mad_u64_u32", "v_mad_i64_i32")


def _sgprs(tok):
    m = _SREG.match(tok.strip())
    if not m:
        return set()
    if m.group(1) is not None:
        return {int(m.group(1))}
    return set(range(int(m.group(2)), int(m.group(3)) + 1))


def _operands(text):
    parts = text.split(None, 1)
    if len(parts) < 2:
        return parts[0], []
    return parts[0], [t.strip() for t in parts[1].split(",")]


def valu_sgpr_writes(text):
    """SGPRs a VALU instruction writes (empty for non-VALU instructions)."""
    op, ops = _operands(text)
    if not op.startswith("v_") or not ops:
        return set()
    out = _sgprs(ops[0])
    if op.startswith(_VOP3B) and len(ops) > 1:
        out |= _sgprs(ops[1])
    return out


def salu_writes_m0(text):
    op, ops = _operands(text)
    return op.startswith("s_") and bool(ops) and ops[0] == "m0"


def wait_states(text):
    op, ops = _operands(text)
    if op == "s_nop":
        return int(ops[0], 0) + 1
    return 1


def _functions(asm):
    """Split assembly text into (name, [entries]); an entry is ('label', name) or ('insn', text)."""
    funcs, cur, name = [], None, None
    for raw in asm.splitlines():
        line = raw.split(";", 1)[0].strip() if not raw.lstrip().startswith(";;#ASM") else ""
        if not line or line.startswith("."):
            lab = _LABEL.match(line) if line else None
            if lab and cur is not None:
                cur.append(("label", lab.group(1)))
            continue
        fm = _FUNC.match(line)
        if fm and not line.startswith("."):
            name, cur = fm.group(1), []
            funcs.append((name, cur))
            continue
        lab = _LABEL.match(line)
        if lab:
            if cur is not None:
                cur.append(("label", lab.group(1)))
            continue
        if cur is not None:
            cur.append(("insn", line))
    return funcs


def _scan_back(entries, pos, branches_to, hit, need, seen):
    """True if some path into entries[pos] has an instruction matching hit()
    fewer than `need` wait states before it."""
    stack = [(pos, 0)]
    while stack:
        p, used = stack.pop()
        if (p, used) in seen:
            continue
        seen.add((p, used))
        j = p - 1
        while j >= 0 and used < need:
            kind, text = entries[j]
            if kind == "label":
                for b in branches_to.get(text, ()):
                    stack.append((b + 1, used))  # the branch itself is examined next
                if j > 0 and entries[j - 1][0] == "insn":
                    op = entries[j - 1][1].split(None, 1)[0]
                    if op in ("s_branch", "s_endpgm", "s_setpc_b64"):
                        break  # no fall-through into this label
                j -= 1
                continue
            if hit(text):
                return True
            used += wait_states(text)
            j -= 1
    return False


def check_asm(asm):
    """Every copy that violates a rule, as (function, instruction, rule) tuples."""
    problems = []
    for name, entries in _functions(asm):
        branches_to = {}
        for i, (kind, text) in enumerate(entries):
            if kind == "insn":
                bm = _BRANCH.match(text)
                if bm:
                    branches_to.setdefault(bm.group(2), []).append(i)
        for i, (kind, text) in enumerate(entries):
            if kind != "insn" or not _COPY_ANY.match(text):
                continue
            m = _COPY.match(text)
            if m:
                regs = set(range(int(m.group(1)), int(m.group(2)) + 1))
                if _scan_back(entries, i, branches_to, lambda t: bool(valu_sgpr_writes(t) & regs),
                              VALU_SGPR_WAIT, set()):
                    problems.append((name, text, "SGPR base written by VALU < 5 wait states before"))
            if _scan_back(entries, i, branches_to, salu_writes_m0, M0_WAIT, set()):
                problems.append((name, text, "m0 written by SALU < 1 wait state before"))
    return problems
