"""Audit of the GEMM kernels' gfx950 assembly for the hardware wait states that inline assembly
must provide itself (the compiler pads only the instructions it generates and counts an inline
assembly statement as one instruction whatever it holds).

Checked along every control-flow path into the instruction (fall-through and branches):
  - an LDS-DMA copy (global_load_lds_*) with an SGPR base: at least 5 wait states since a VALU
    instruction last wrote one of those SGPRs, at least 1 since M0 was last written by the
    SALU (5 if the VALU wrote it);
  - an MFMA: at least 2 wait states since a VALU instruction (other than an MFMA) last wrote a
    VGPR of its A or B operand;
  - any other instruction reading an MFMA's result registers (accumulator reads, VALU, stores):
    at least passes + 3 wait states after that MFMA, with the passes of its shape (4 for
    16x16x32 bf16/f16, 8 for 32x32x16 bf16/f16, 16 for the 32x32x64 block-scaled MFMA with an
    8-bit operand and 8 without, half that for the 16x16x128 one; 16 for any other MFMA).
A wait state is one issued instruction; s_nop N counts N + 1.
"""
from __future__ import annotations

import re
from collections import defaultdict

_REG = re.compile(r"^([svam])(?:\[(\d+):(\d+)\]|(\d+))$")


def _regs(tok: str) -> set:
    """Registers named by one operand token: {('s', 4), ('s', 5)} for s[4:5], {('m', 0)} for m0."""
    tok = tok.strip().rstrip(",")
    if tok == "m0":
        return {("m", 0)}
    m = _REG.match(tok)
    if not m or m.group(1) == "m":
        return set()
    if m.group(4) is not None:
        return {(m.group(1), int(m.group(4)))}
    return {(m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1)}


def _parse(text: str):
    """Functions as lists of (mnemonic, operand tokens) and label -> index maps."""
    funcs = []
    cur = None
    for raw in text.splitlines():
        line = raw.split(";")[0].rstrip()
        s = line.strip()
        if not s:
            continue
        m = re.match(r"^([A-Za-z_.$][\w.$]*):$", s)
        if m:
            name = m.group(1)
            if not name.startswith("."):
                cur = {"name": name, "ins": [], "labels": {}}
                funcs.append(cur)
            elif cur is not None:
                cur["labels"][name] = len(cur["ins"])
            continue
        if cur is None or s.startswith("."):
            continue
        parts = s.split(None, 1)
        ops = [t.strip() for t in parts[1].split(",")] if len(parts) > 1 else []
        cur["ins"].append((parts[0], ops))
    return funcs


def _waits(ins) -> int:
    op, ops = ins
    if op == "s_nop":
        return int(ops[0], 0) + 1
    return 1


def _writes(ins) -> set:
    op, ops = ins
    if not ops or op.startswith(("s_cbranch", "s_branch", "s_waitcnt", "s_barrier", "s_nop")):
        return set()
    if op.startswith(("global_store", "buffer_store", "scratch_store", "flat_store", "ds_write", "global_load_lds")):
        return set()
    return _regs(ops[0])


def _min_since(f, i: int, hit, need: int) -> int:
    """Fewest wait states on any path from the last instruction satisfying hit(ins) to
    instruction i (need or more if none is closer than need)."""
    ins, labels = f["ins"], f["labels"]
    preds = f.setdefault("_preds", None)
    if preds is None:
        preds = defaultdict(list)
        for j, (op, ops) in enumerate(ins):
            if op.startswith(("s_branch", "s_cbranch")) and ops:
                if ops[0] in labels:
                    preds[labels[ops[0]]].append(j)
        starts = defaultdict(list)
        for name, idx in labels.items():
            starts[idx].append(name)
        f["_preds"] = preds
        f["_starts"] = starts
    starts = f["_starts"]
    best = need
    stack = [(i, 0)]
    seen = {}
    while stack:
        j, ws = stack.pop()
        while ws < best:
            if j in starts or j == 0:
                for b in preds.get(j, []):
                    if seen.get(b, 1 << 30) > ws:
                        stack.append((b + 1, ws))
                if j == 0:
                    break
                prev = ins[j - 1][0]
                if j in starts and prev in ("s_branch", "s_endpgm", "s_setpc_b64"):
                    break
            j -= 1
            if seen.get(j, 1 << 30) <= ws:
                break
            seen[j] = ws
            if hit(ins[j]):
                best = min(best, ws)
                break
            ws += _waits(ins[j])
    return best


def _passes(ins) -> int:
    """Passes of an MFMA: the block-scaled shapes run at half length when neither operand is
    8-bit (format codes cbsz / blgp: 0 E4M3, 1 E5M2, 2 E2M3, 3 E3M2, 4 E2M1)."""
    op, ops = ins
    if op.startswith("v_mfma_f32_16x16x32_"):
        return 4
    if op.startswith("v_mfma_f32_32x32x16_"):
        return 8
    if op.startswith("v_mfma_scale_f32_"):
        mods = " ".join(ops)
        codes = [int(m) for m in re.findall(r"(?:cbsz|blgp):(\d+)", mods)]
        narrow = len(codes) == 2 and min(codes) >= 2
        full = 8 if op.startswith("v_mfma_scale_f32_16x16x128") else 16
        return full // 2 if narrow else full
    return 16


def _reads(ins) -> set:
    """Registers an instruction reads (every operand but the destination; stores read all)."""
    op, ops = ins
    if op.startswith(("global_store", "buffer_store", "scratch_store", "flat_store", "ds_write")):
        toks = ops
    else:
        toks = ops[1:]
    r = set()
    for t in toks:
        r |= _regs(t)
    return r


def audit(text: str) -> list:
    """Violations as strings (empty when the assembly keeps every wait state above)."""
    out = []
    for f in _parse(text):
        for i, (op, ops) in enumerate(f["ins"]):
            if op.startswith("global_load_lds") and len(ops) >= 2 and ops[1] != "off":
                base = _regs(ops[1])
                w = _min_since(f, i, lambda x: x[0].startswith("v_") and bool(_writes(x) & base), 5)
                if w < 5:
                    out.append(f"{f['name']}: {op} #{i}: {w} wait states after a VALU write of its SGPR base")
                m0 = {("m", 0)}
                w = _min_since(f, i, lambda x: bool(_writes(x) & m0) and not x[0].startswith("v_"), 1)
                if w < 1:
                    out.append(f"{f['name']}: {op} #{i}: no wait state after the write of M0")
                w = _min_since(f, i, lambda x: bool(_writes(x) & m0) and x[0].startswith("v_"), 5)
                if w < 5:
                    out.append(f"{f['name']}: {op} #{i}: {w} wait states after a VALU write of M0")
            elif op.startswith("v_mfma") and len(ops) >= 3:
                src = _regs(ops[1]) | _regs(ops[2])
                src = {r for r in src if r[0] == "v"}
                if not src:
                    continue
                w = _min_since(f, i, lambda x: x[0].startswith("v_") and not x[0].startswith(("v_mfma", "v_dot"))
                               and bool(_writes(x) & src), 2)
                if w < 2:
                    out.append(f"{f['name']}: {op} #{i}: {w} wait states after a VALU write of its A/B VGPRs")
            if not op.startswith("v_mfma"):
                rd = {r for r in _reads((op, ops)) if r[0] in "va"}
                if not rd:
                    continue
                hit = lambda x: x[0].startswith("v_mfma") and bool(_writes(x) & rd)
                w = _min_since(f, i, hit, 19)
                if w < 19:
                    # the nearest MFMA writing what this reads: its shape sets the requirement
                    need = _min_need(f, i, rd)
                    if w < need:
                        out.append(f"{f['name']}: {op} #{i}: {w} wait states after an MFMA wrote what it reads "
                                   f"(needs {need})")
    return out


def _min_need(f, i: int, rd: set) -> int:
    """passes + 3 of the MFMA that last wrote any of rd on the fall-through path before i
    (the largest such requirement among the nearest writers, 19 if none is found nearby)."""
    ins = f["ins"]
    for j in range(i - 1, max(i - 200, -1), -1):
        op = ins[j][0]
        if op.startswith("v_mfma") and _writes(ins[j]) & rd:
            return _passes(ins[j]) + 3
    return 19
