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

and the ordering rule of the write-through stores (`nt sc1`), which the
compiler does not count among its vector memory operations: on no path from
such a store is there a load that returns data to registers (the compiler
would wait for it with a count that misses the store), and every vector
memory wait on such a path is vmcnt(0), which no uncounted store can
confuse (the LDS copies after a store are only waited for that way).

"Before" and "after" follow the control flow: the instructions before a
branch target include the branches that jump to it (loop back-edges too),
and the instructions after a branch include its target.
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


def _program(lines):
    """Instructions in order plus the label -> instruction index map.  Labels,
    directives and comments are dropped; the lines of an inline-assembly
    block are instructions too.  Each kernel ends at s_endpgm."""
    instrs, labels = [], {}
    for line in lines:
        t = line.split(";")[0].split("//")[0].strip()
        if not t:
            continue
        if t.endswith(":"):
            labels[t[:-1]] = len(instrs)
            continue
        if t.startswith("."):
            continue
        instrs.append(t)
    return instrs, labels


_UNCONDITIONAL = ("s_branch", "s_endpgm", "s_setpc_b64")


def _edges(instrs, labels):
    """Successor and predecessor lists of every instruction."""
    succ = [[] for _ in instrs]
    for i, ins in enumerate(instrs):
        op = ins.split()[0]
        if op not in _UNCONDITIONAL and i + 1 < len(instrs):
            succ[i].append(i + 1)
        if op == "s_branch" or op.startswith("s_cbranch"):
            target = ins.split()[1]
            assert target in labels, f"branch to an unknown label: {ins}"
            succ[i].append(labels[target])
        assert op != "s_setpc_b64", "indirect jump: the checker cannot follow it"
    pred = [[] for _ in instrs]
    for i, ss in enumerate(succ):
        for j in ss:
            pred[j].append(i)
    return succ, pred


# scalar instructions whose first operand is not a destination
_NO_SCALAR_DEST = ("s_cmp", "s_bitcmp", "s_cbranch", "s_waitcnt", "s_nop", "s_barrier", "s_setprio",
                   "s_sleep", "s_branch", "s_endpgm")


def _vector_writer_within(instrs, pred, i, pending, depth):
    """Does a vector instruction write one of `pending` (scalar registers) on
    some path of at most `depth` instructions ending right before i, with no
    scalar instruction rewriting it in between?"""
    for j in pred[i]:
        prev = instrs[j]
        ops = _operands(prev)
        left = pending
        if ops and not prev.split()[0].startswith(_NO_SCALAR_DEST):
            written = _sregs(ops[0]) & pending
            if written and prev.startswith("v_"):
                return True
            left = pending - written
        if left and depth > 1 and _vector_writer_within(instrs, pred, j, left, depth - 1):
            return True
    return False


def _store_data_overwritten(instrs, succ, i, data, depth):
    for j in succ[i]:
        nxt = instrs[j]
        if nxt.startswith("v_") and _operands(nxt) and _vregs(_operands(nxt)[0]) & data:
            return True
        if depth > 1 and _store_data_overwritten(instrs, succ, j, data, depth - 1):
            return True
    return False


def _write_through(ins):
    return re.match(r"(global|buffer)_store\w*\b.*\bnt sc1\b", ins) is not None


def hazards(lines):
    """List of (rule, index, text) for every violation in a stream of
    assembly lines (instructions and labels)."""
    instrs, labels = _program(lines)
    succ, pred = _edges(instrs, labels)
    found = []
    # instructions reachable from a write-through store
    after_store, todo = set(), [i for i, ins in enumerate(instrs) if _write_through(ins)]
    while todo:
        i = todo.pop()
        for j in succ[i]:
            if j not in after_store:
                after_store.add(j)
                todo.append(j)
    for i, ins in enumerate(instrs):
        op = ins.split()[0]
        if i in after_store:
            if re.match(r"(global|buffer)_load", op) and not ins.rstrip().endswith(" lds"):
                found.append(("register load after a write-through store", i, ins))
            m = re.search(r"vmcnt\((\d+)\)", ins)
            if op == "s_waitcnt" and m and int(m.group(1)) != 0:
                found.append(("counted vector memory wait after a write-through store", i, ins))
        if op.startswith("buffer_"):
            pending = set().union(*(_sregs(o) for o in _operands(ins)))
            if pending and _vector_writer_within(instrs, pred, i, pending, 5):
                found.append(("vector-written scalar register read by a buffer instruction", i, ins))
            if ins.rstrip().endswith(" lds") and any(re.match(r"s_\w+\s+m0\b", instrs[j]) for j in pred[i]):
                found.append(("M0 written right before an LDS copy", i, ins))
        if re.match(r"(global|buffer)_store_dword(x3|x4)\b", op):
            ops = _operands(ins)
            data = _vregs(ops[1]) if op.startswith("global") else _vregs(ops[0])
            if _store_data_overwritten(instrs, succ, i, data, 2):
                found.append(("store data overwritten within two instructions", i, ins))
    return found


def _rules(lines):
    return [h[0] for h in hazards(lines)]


def test_rules_catch_the_patterns():
    """The checker itself: each rule fires on a minimal bad sequence and not on
    the fixed one, along straight-line code and across branches."""
    bad = ["v_readfirstlane_b32 s26, v45", "s_mov_b32 m0, s3", "s_nop 0",
           "buffer_load_dwordx4 v35, s[24:27], 0 offen lds"]
    assert _rules(bad) == ["vector-written scalar register read by a buffer instruction"]
    ok = ["v_readfirstlane_b32 s26, v45", "s_mov_b32 s26, s26", "s_mov_b32 m0, s3", "s_nop 0",
          "buffer_load_dwordx4 v35, s[24:27], 0 offen lds"]
    assert _rules(ok) == []
    # loop-carried: the vector write sits at the latch, the copy at the loop head
    loop = [".LBB0_1:", "s_mov_b32 m0, s3", "s_nop 0", "buffer_load_dwordx4 v35, s[24:27], 0 offen lds",
            "s_add_i32 s4, s4, 1", "s_cmp_lt_i32 s4, 8", "v_readfirstlane_b32 s26, v45",
            "s_cbranch_scc1 .LBB0_1", "s_endpgm"]
    assert _rules(loop) == ["vector-written scalar register read by a buffer instruction"]
    # the write at the end of an if-block, the copy at the join
    join = ["s_cbranch_scc0 .LBB0_2", "v_readfirstlane_b32 s26, v45", ".LBB0_2:", "s_mov_b32 m0, s3",
            "s_nop 0", "buffer_load_dwordx4 v35, s[24:27], 0 offen lds", "s_endpgm"]
    assert _rules(join) == ["vector-written scalar register read by a buffer instruction"]
    assert _rules(["s_mov_b32 m0, s3", "buffer_load_dwordx4 v1, s[4:7], 0 offen lds"]) == \
        ["M0 written right before an LDS copy"]
    # a label between them does not separate them (a branch instruction does)
    assert _rules(["s_cbranch_scc1 .LBB0_3", "s_mov_b32 m0, s3", ".LBB0_3:",
                   "buffer_load_dwordx4 v1, s[4:7], 0 offen lds", "s_endpgm"]) == \
        ["M0 written right before an LDS copy"]
    assert _rules(["s_mov_b32 m0, s3", "s_branch .LBB0_3", ".LBB0_3:",
                   "buffer_load_dwordx4 v1, s[4:7], 0 offen lds", "s_endpgm"]) == []
    st = ["global_store_dwordx4 v[8:9], v[4:7], off nt sc1", "s_or_b64 exec, exec, s[0:1]",
          "v_or_b32_e32 v4, 16, v134"]
    assert _rules(st) == ["store data overwritten within two instructions"]
    assert _rules(st[:1] + ["s_nop 1"] + st[1:]) == []
    st_br = ["global_store_dwordx4 v[8:9], v[4:7], off nt sc1", "s_cbranch_scc1 .LBB0_4", "s_endpgm",
             ".LBB0_4:", "v_or_b32_e32 v4, 16, v134", "s_endpgm"]
    assert _rules(st_br) == ["store data overwritten within two instructions"]
    ld = ["global_store_dword v[2:3], v1, off nt sc1", "global_load_dword v5, v[6:7], off", "s_endpgm"]
    assert _rules(ld) == ["register load after a write-through store"]
    assert _rules(ld[:1] + ["s_endpgm"] + ld[1:]) == []
    # an LDS copy after the store, waited for with vmcnt(0): allowed; with a count: not
    cp = ["global_store_dword v[2:3], v1, off nt sc1", "s_mov_b32 m0, s3", "s_nop 0",
          "buffer_load_dwordx4 v1, s[4:7], 0 offen lds", "s_waitcnt vmcnt(0)", "s_endpgm"]
    assert _rules(cp) == []
    assert _rules(cp[:4] + ["s_waitcnt vmcnt(1) lgkmcnt(0)", "s_endpgm"]) == \
        ["counted vector memory wait after a write-through store"]
    # a store inside a loop reaches the loop head again
    back = [".LBB0_5:", "s_waitcnt vmcnt(2)", "global_store_dword v[2:3], v1, off nt sc1",
            "s_cbranch_scc1 .LBB0_5", "s_endpgm"]
    assert _rules(back) == ["counted vector memory wait after a write-through store"]


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
        instrs, _ = _program(text.splitlines())
        n_buffer += sum(1 for x in instrs if x.startswith("buffer_"))
        problems += [f"{os.path.basename(src)}: {rule}: {ins}" for rule, _, ins in hazards(text.splitlines())]
    assert n_buffer > 100, "no buffer instructions found: the assembly was not parsed"
    assert not problems, "\n".join(problems[:20])
