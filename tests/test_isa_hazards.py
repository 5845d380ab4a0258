"""Hazards the compiler cannot see: the library issues its LDS copies and its
write-through output stores from inline assembly, which the compiler's
hazard recognizer does not look into.  This test compiles every kernel
source to gfx950 assembly with the library's own flags (no GPU needed) and
checks the three GFX9-family wait-state rules that apply to those
instructions:

  1. a buffer instruction reads no scalar register that a vector instruction
     wrote in the five instructions before it;
  2. an LDS copy (buffer_load ... lds) is not the instruction right after the
     write of M0 that it reads;
  3. no vector instruction overwrites the data registers of a store of more
     than 64 bits in the two instructions after it;

and the ordering rule of the write-through stores (`nt sc1`), whose vector
memory counts the compiler does not track: in each kernel no global or
buffer load follows them.
"""
import concurrent.futures as cf
import os
import re
import shutil
import subprocess

import pytest

from head_attention_sdpa_amd import build as hip_build


def _sregs(tok):
    m = re.match(r"s\[(\d+):(\d+)\]$", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"s(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def _vregs(tok):
    m = re.match(r"v\[(\d+):(\d+)\]$", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def _operands(instr):
    parts = instr.split(None, 1)
    return [o.strip().split()[0] for o in parts[1].split(",") if o.strip()] if len(parts) > 1 else []


def _instructions(asm_text):
    """Instructions of the assembly in order (labels, directives and comments
    dropped; the lines of an inline-assembly block are instructions too)."""
    out = []
    for line in asm_text.splitlines():
        t = line.strip()
        if not t or t.startswith((";", ".", "//")) or t.endswith(":"):
            continue
        out.append(t.split(";")[0].strip())
    return out


# scalar instructions whose first operand is not a destination
_NO_SCALAR_DEST = ("s_cmp", "s_bitcmp", "s_cbranch", "s_waitcnt", "s_nop", "s_barrier", "s_setprio",
                   "s_sleep", "s_branch", "s_endpgm")


def hazards(instrs):
    """List of (rule, index, text) for every violation in one instruction stream."""
    found = []
    after_asm_store = False
    for i, ins in enumerate(instrs):
        op = ins.split()[0]
        if op == "s_endpgm":
            after_asm_store = False
        if re.match(r"(global|buffer)_store\w*\b.*\bnt sc1\b", ins):
            after_asm_store = True
        elif after_asm_store and re.match(r"(global|buffer)_load", op):
            found.append(("load after a write-through store", i, ins))
        if op.startswith("buffer_"):
            # the latest writer of each scalar operand among the five
            # instructions before must not be a vector instruction
            pending = set().union(*(_sregs(o) for o in _operands(ins)))
            for j in range(i - 1, max(-1, i - 6), -1):
                prev = instrs[j]
                ops = _operands(prev)
                if not ops or prev.split()[0].startswith(_NO_SCALAR_DEST):
                    continue
                written = _sregs(ops[0]) & pending
                if written and prev.startswith("v_"):
                    found.append(("vector-written scalar register read by a buffer instruction", i, ins))
                    break
                pending -= written
            if ins.rstrip().endswith(" lds") and i > 0 and re.match(r"s_\w+\s+m0\b", instrs[i - 1]):
                found.append(("M0 written right before an LDS copy", i, ins))
        if re.match(r"(global|buffer)_store_dword(x3|x4)\b", op):
            ops = _operands(ins)
            data = _vregs(ops[1]) if op.startswith("global") else _vregs(ops[0])
            for j in range(i + 1, min(len(instrs), i + 3)):
                nxt = instrs[j]
                if nxt.startswith("v_") and _operands(nxt) and _vregs(_operands(nxt)[0]) & data:
                    found.append(("store data overwritten within two instructions", i, ins))
    return found


def test_rules_catch_the_patterns():
    """The checker itself: each rule fires on a minimal bad sequence and not on
    the fixed one."""
    bad = ["v_readfirstlane_b32 s26, v45", "s_mov_b32 m0, s3", "s_nop 0",
           "buffer_load_dwordx4 v35, s[24:27], 0 offen lds"]
    assert [h[0] for h in hazards(bad)] == ["vector-written scalar register read by a buffer instruction"]
    ok = ["v_readfirstlane_b32 s26, v45", "s_mov_b32 s26, s26", "s_mov_b32 m0, s3", "s_nop 0",
          "buffer_load_dwordx4 v35, s[24:27], 0 offen lds"]
    assert hazards(ok) == []
    assert [h[0] for h in hazards(["s_mov_b32 m0, s3", "buffer_load_dwordx4 v1, s[4:7], 0 offen lds"])] == \
        ["M0 written right before an LDS copy"]
    st = ["global_store_dwordx4 v[8:9], v[4:7], off nt sc1", "s_or_b64 exec, exec, s[0:1]",
          "v_or_b32_e32 v4, 16, v134"]
    assert [h[0] for h in hazards(st)] == ["store data overwritten within two instructions"]
    assert hazards(st[:1] + ["s_nop 1"] + st[1:]) == []
    ld = ["global_store_dword v[2:3], v1, off nt sc1", "global_load_dword v5, v[6:7], off", "s_endpgm"]
    assert [h[0] for h in hazards(ld)] == ["load after a write-through store"]
    assert hazards(ld[:1] + ["s_endpgm"] + ld[1:]) == []


@pytest.mark.skipif(shutil.which(hip_build.hipcc()) is None and not os.path.exists(hip_build.hipcc()),
                    reason="hipcc not available")
def test_library_kernels_have_no_hidden_hazards(tmp_path):
    srcs = [s for s in hip_build.sources() if s.endswith(".hip")]

    def to_asm(src):
        out = tmp_path / (os.path.basename(src) + ".s")
        cmd = [hip_build.hipcc(), *hip_build.COMMON, "--cuda-device-only", "-S", src, "-o", str(out)]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        return src, out.read_text()

    with cf.ThreadPoolExecutor(min(8, len(srcs))) as ex:
        results = list(ex.map(to_asm, srcs))
    problems, n_buffer = [], 0
    for src, text in results:
        instrs = _instructions(text)
        n_buffer += sum(1 for x in instrs if x.startswith("buffer_"))
        problems += [f"{os.path.basename(src)}: {rule}: {ins}" for rule, _, ins in hazards(instrs)]
    assert n_buffer > 100, "no buffer instructions found: the assembly was not parsed"
    assert not problems, "\n".join(problems[:20])
