"""Static check of the built library's gfx950 code: no instruction other than an MFMA
reads or overwrites a register that an MFMA wrote fewer than LIMIT wait states before
it.

The tiled LM-head kernel and the MFMA-rate probe issue MFMAs as inline asm, whose
result latency the compiler does not know: if it places a register copy of an
accumulator (or any other read of it) right after the MFMA that writes it, the copy
takes the stale value and the logits of that 16 x 16 block come out wrong,
differently from run to run. This scans the code
objects embedded in libmtpv.so (unbundled from its .hip_fatbin section, disassembled
with llvm-objdump), as a dataflow over each function's basic blocks: a block is entered
with the worst case over every path into it (fall-through, forward jumps and loop back
edges), counting one wait state per instruction and N + 1 per s_nop N; MFMAs reading
an accumulator that an earlier MFMA wrote are left to the hardware's interlock.
LIMIT = 18 is above the wait states a 16x16 MFMA result needs before a VALU read or
write, so the check is strict. Only the kernels with inline-asm MFMAs are scanned:
where the compiler's MFMA builtins are used, its hazard recognizer inserts the wait
states from each MFMA's own latency. No GPU is needed.
"""
import os
import re
import struct
import subprocess
import tempfile

import pytest

import mtp_draft_verification_amd as mv

LLVM = "/opt/rocm/llvm/bin"
LIMIT = 18
MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"
REG = re.compile(r"\b([av])\[(\d+):(\d+)\]|\b([av])(\d+)\b")


def _regs(text):
    out = set()
    for m in REG.finditer(text):
        if m.group(1):
            out |= {(m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1)}
        else:
            out.add((m.group(4), int(m.group(5))))
    return out


def _code_objects(lib_path, tmp):
    """The gfx950 code objects of every offload bundle in the library's .hip_fatbin."""
    fat = os.path.join(tmp, "fatbin.bin")
    subprocess.run([os.path.join(LLVM, "llvm-objcopy"), "--dump-section", f".hip_fatbin={fat}", lib_path,
                    os.path.join(tmp, "copy.so")], check=True, capture_output=True)
    data = open(fat, "rb").read()
    objs = []
    start = data.find(MAGIC)
    while start >= 0:
        n = struct.unpack_from("<Q", data, start + len(MAGIC))[0]
        pos = start + len(MAGIC) + 8
        for _ in range(n):
            off, size, tlen = struct.unpack_from("<QQQ", data, pos)
            triple = data[pos + 24:pos + 24 + tlen].decode()
            pos += 24 + tlen
            if "gfx950" in triple and size > 0:
                path = os.path.join(tmp, f"co{len(objs)}.o")
                open(path, "wb").write(data[start + off:start + off + size])
                objs.append(path)
        start = data.find(MAGIC, start + 1)
    return objs


ADDR = re.compile(r"//\s*([0-9A-Fa-f]+):")


def _parse(disasm):
    """Functions of the listing: name -> [(address, instruction text)]."""
    fns, fn = {}, None
    for line in disasm.splitlines():
        m = re.match(r"^[0-9a-f]+ <(.+)>:", line)
        if m:
            fn = m.group(1)
            fns[fn] = []
            continue
        s = line.split("//")[0].strip()
        a = ADDR.search(line)
        if s and fn is not None and a:
            fns[fn].append((int(a.group(1), 16), s))
    return fns


def _target(addr, op, args):
    """Branch target of s_branch / s_cbranch_* (signed dword offset from the next word)."""
    imm = int(args.split(",")[0].strip(), 0)
    if imm >= 1 << 15:
        imm -= 1 << 16
    return addr + 4 + 4 * imm


def _step(state, ins, flagged=None, fn=None):
    """One instruction through the state {register: wait states since an MFMA wrote it}
    (only registers closer than LIMIT are kept); flags the early reads when asked."""
    s = ins
    op = s.split()[0]
    args = s[len(op):]
    if op.startswith("s_nop"):
        n = int(args.strip(), 0) + 1 if args.strip() else 1
        return {r: w + n for r, w in state.items() if w + n < LIMIT}
    parts = [p.strip() for p in args.split(",")]
    out = {r: w + 1 for r, w in state.items() if w + 1 < LIMIT}
    if op.startswith("v_mfma"):
        for r in _regs(parts[0]):
            out[r] = 0
        return out
    if flagged is not None and state and parts and parts[0]:
        touched = set().union(*(_regs(p) for p in parts))  # sources and destination
        hit = [state[r] for r in touched if r in state]
        if hit:
            flagged.append((fn, s, min(hit)))
    return out


def _join(a, b):
    out = dict(a)
    for r, w in b.items():
        out[r] = min(w, out.get(r, w))
    return out


def _scan(disasm, only=None):
    """(function, instruction, wait states) of every early read in the listing: a
    dataflow over each function's basic blocks, every block entered with the worst
    case over its predecessors (fall-through, jumps and loop back edges). only: a
    predicate on function names (None: every function)."""
    flagged = []
    for fn, code in _parse(disasm).items():
        if not code or (only is not None and not only(fn)):
            continue
        index = {a: i for i, (a, _) in enumerate(code)}
        starts, succ = {0}, {}
        for i, (a, s) in enumerate(code):
            op = s.split()[0]
            if op == "s_branch" or op.startswith("s_cbranch"):
                t = index.get(_target(a, op, s[len(op):]))
                succ[i] = ([t] if t is not None else []) + ([i + 1] if op != "s_branch" and i + 1 < len(code) else [])
                starts.update(x for x in succ[i])
                if i + 1 < len(code):
                    starts.add(i + 1)
            elif op in ("s_setpc_b64", "s_endpgm"):
                succ[i] = []
                if i + 1 < len(code):
                    starts.add(i + 1)
        starts = sorted(starts)
        block_of = {}
        blocks = []
        for j, b0 in enumerate(starts):
            b1 = starts[j + 1] if j + 1 < len(starts) else len(code)
            blocks.append((b0, b1))
            block_of[b0] = j
        def out_edges(j):
            b0, b1 = blocks[j]
            last = b1 - 1
            nxt = succ.get(last, [b1] if b1 < len(code) else [])
            return [block_of[x] for x in nxt if x in block_of]
        state_in = {0: {}}
        work = [0]
        while work:
            j = work.pop()
            st = dict(state_in[j])
            for i in range(*blocks[j]):
                st = _step(st, code[i][1])
            for k in out_edges(j):
                new = _join(state_in[k], st) if k in state_in else st
                if k not in state_in or new != state_in[k]:
                    state_in[k] = new
                    work.append(k)
        for j, st in state_in.items():
            for i in range(*blocks[j]):
                st = _step(st, code[i][1], flagged, fn)
    return flagged


def _tools_present():
    return all(os.path.exists(os.path.join(LLVM, t)) for t in ("llvm-objcopy", "llvm-objdump"))


CSRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "mtp_draft_verification_amd", "csrc")


def _asm_mfma_kernels():
    """Kernels defined in the sources that issue MFMAs as inline asm (whose result
    latency the compiler does not see). Kernels that use the compiler's MFMA builtins
    get their wait states from its hazard recognizer, which knows each MFMA's latency
    on every path, and are left to it."""
    names = set()
    for f in sorted(os.listdir(CSRC)):
        if not f.endswith(".hip"):
            continue
        src = open(os.path.join(CSRC, f)).read()
        if 'asm volatile("v_mfma' in src:
            names |= set(re.findall(r"__global__[^;{]*?\bvoid\s+(\w+)\s*\(", src))
    return names


@pytest.mark.skipif(not _tools_present(), reason="ROCm llvm tools not found")
def test_no_early_reads_of_mfma_results():
    lib_path = mv.LIB_PATH
    if not os.path.exists(lib_path):
        pytest.skip("library not built")
    kernels = _asm_mfma_kernels()
    assert {"head_tile_kernel", "mfma_kernel"} <= kernels, kernels
    tags = [f"{len(k)}{k}" for k in kernels]  # as the names appear in mangled symbols
    only = lambda fn: any(t in fn for t in tags)
    with tempfile.TemporaryDirectory() as tmp:
        objs = _code_objects(lib_path, tmp)
        assert objs, "no gfx950 code object in the library"
        flagged, n_mfma = [], 0
        for o in objs:
            res = subprocess.run([os.path.join(LLVM, "llvm-objdump"), "-d", "--mcpu=gfx950", o],
                                 check=True, capture_output=True, text=True)
            n_mfma += sum(len(re.findall(r"\bv_mfma", "\n".join(s for _, s in code)))
                          for fn, code in _parse(res.stdout).items() if only(fn))
            flagged += _scan(res.stdout, only)
    assert n_mfma > 1000  # every instance of the tiled kernel is in there
    assert not flagged, flagged[:5]


def _listing(lines, base=0x1000):
    """A planted listing in llvm-objdump's form: every instruction with its address
    (MFMAs take 8 bytes, the rest 4)."""
    out, a = ["%016x <k>:" % base], base
    for s in lines:
        out.append("\t%s // %012X: 0" % (s, a))
        a += 8 if s.startswith("v_mfma") else 4
    return "\n".join(out) + "\n"


MFMA = "v_mfma_f32_16x16x32_bf16 a[4:7], v[2:5], v[6:9], a[4:7]"


def test_scan_flags_a_copy_right_after_an_mfma():
    """The scanner on planted listings: a copy one instruction after the MFMA that
    writes its source is flagged, and so is an overwrite of its destination; the same
    copy after four s_nop 7 or a chained MFMA is not, nor code after an unconditional
    branch that nothing else reaches. A read at a loop head right after the MFMA at
    the loop's end is flagged through the back edge, and so is one at a jump target."""
    bad = [MFMA, "s_add_i32 s0, s0, 1", "v_accvgpr_read_b32 v10, a5"]
    assert [f[1] for f in _scan(_listing(bad))] == ["v_accvgpr_read_b32 v10, a5"]
    overwrite = [MFMA, "s_add_i32 s0, s0, 1", "v_accvgpr_write_b32 a6, 0"]
    assert [f[1] for f in _scan(_listing(overwrite))] == ["v_accvgpr_write_b32 a6, 0"]
    assert _scan(_listing([MFMA] + ["s_nop 7"] * 4 + ["v_accvgpr_read_b32 v10, a5"])) == []
    assert _scan(_listing([MFMA, "s_add_i32 s0, s0, 1", MFMA])) == []
    # s_branch over the read: the read is unreachable (the branch lands on s_endpgm)
    assert _scan(_listing([MFMA, "s_branch 1", "v_accvgpr_read_b32 v10, a5", "s_endpgm"])) == []
    # loop: head reads a5, the body ends with the MFMA and branches back to the head
    loop = ["s_mov_b32 s0, 4", "v_accvgpr_read_b32 v10, a5", "s_add_i32 s0, s0, -1", MFMA,
            "s_cmp_lg_u32 s0, 0", "s_cbranch_scc1 65530", "s_endpgm"]
    # the branch at 0x1018 goes back 6 dwords from the next word (0x101c) to 0x1004
    assert [f[1] for f in _scan(_listing(loop))] == ["v_accvgpr_read_b32 v10, a5"]
    looped_safe = loop[:4] + ["s_nop 7"] * 4 + loop[4:]
    looped_safe[-2] = "s_cbranch_scc1 65526"  # four more words back
    assert _scan(_listing(looped_safe)) == []
    # forward jump from right after the MFMA to a read
    jump = [MFMA, "s_cbranch_scc1 1", "s_nop 7", "v_accvgpr_read_b32 v10, a5", "s_endpgm"]
    assert [f[1] for f in _scan(_listing(jump))] == ["v_accvgpr_read_b32 v10, a5"]
