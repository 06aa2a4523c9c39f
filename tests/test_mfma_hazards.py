"""Static check of the built library's gfx950 code: no instruction other than an MFMA
reads or overwrites a register that an MFMA wrote fewer than LIMIT wait states before
it.

Several kernels issue MFMAs as inline asm, whose result latency the compiler does not
know: if it places a register copy of an accumulator (or any other read of it) right
after the MFMA that writes it, the copy takes the stale value and the logits of that
16 x 16 block come out wrong, differently from run to run. This scans the code
objects embedded in libmtpv.so (unbundled from its .hip_fatbin section, disassembled
with llvm-objdump), through each function in address order along the fall-through
path (the window restarts after an unconditional branch; a block entered only by a
jump is checked from its own start), counting one wait state per instruction and
N + 1 per s_nop N; MFMAs reading an accumulator that an earlier MFMA wrote are left to
the hardware's interlock. LIMIT = 18 is above the wait states a 16x16 MFMA result
needs before a VALU read or write, so the check is strict. No GPU is needed.
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


def _scan(disasm):
    """(function, instruction, wait states) of every early read in the listing."""
    flagged, fn, recent = [], None, []
    for line in disasm.splitlines():
        m = re.match(r"^[0-9a-f]+ <(.+)>:", line)
        if m:
            fn, recent = m.group(1), []
            continue
        s = line.split("//")[0].strip()
        if not s or fn is None:
            continue
        op = s.split()[0]
        args = s[len(op):]
        if op.startswith("s_nop"):
            n = int(args.strip(), 0) + 1 if args.strip() else 1
            recent = [(d, w + n) for d, w in recent if w + n < LIMIT]
            continue
        parts = [p.strip() for p in args.split(",")]
        if op.startswith("v_mfma"):
            recent = [(d, w + 1) for d, w in recent if w + 1 < LIMIT]
            recent.append((_regs(parts[0]), 0))
            continue
        if recent and parts and parts[0]:
            touched = set().union(*(_regs(p) for p in parts))  # sources and destination
            for d, w in recent:
                if touched & d:
                    flagged.append((fn, s, w))
                    break
        recent = [(d, w + 1) for d, w in recent if w + 1 < LIMIT]
        if op in ("s_branch", "s_setpc_b64", "s_endpgm"):
            recent = []  # what follows is entered by a jump, not by falling through
    return flagged


def _tools_present():
    return all(os.path.exists(os.path.join(LLVM, t)) for t in ("llvm-objcopy", "llvm-objdump"))


@pytest.mark.skipif(not _tools_present(), reason="ROCm llvm tools not found")
def test_no_early_reads_of_mfma_results():
    lib_path = mv.LIB_PATH
    if not os.path.exists(lib_path):
        pytest.skip("library not built")
    with tempfile.TemporaryDirectory() as tmp:
        objs = _code_objects(lib_path, tmp)
        assert objs, "no gfx950 code object in the library"
        flagged, n_mfma = [], 0
        for o in objs:
            res = subprocess.run([os.path.join(LLVM, "llvm-objdump"), "-d", "--mcpu=gfx950", o],
                                 check=True, capture_output=True, text=True)
            n_mfma += res.stdout.count("v_mfma")
            flagged += _scan(res.stdout)
    assert n_mfma > 1000  # the tiled, streaming and fp32-head kernels are in there
    assert not flagged, flagged[:5]


def test_scan_flags_a_copy_right_after_an_mfma():
    """The scanner on planted listings: a copy one instruction after the MFMA that
    writes its source is flagged, and so is an overwrite of its destination; the same
    copy after four s_nop 7, a chained MFMA, or code after an unconditional branch are
    not."""
    bad = """0000000000001000 <k>:
	v_mfma_f32_16x16x32_bf16 a[4:7], v[2:5], v[6:9], a[4:7]
	s_add_i32 s0, s0, 1
	v_accvgpr_read_b32 v10, a5
"""
    good = bad.replace("\ts_add_i32 s0, s0, 1\n", "\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n")
    chained = bad.replace("\tv_accvgpr_read_b32 v10, a5\n",
                          "\tv_mfma_f32_16x16x32_bf16 a[4:7], v[2:5], v[6:9], a[4:7]\n")
    overwrite = bad.replace("v_accvgpr_read_b32 v10, a5", "v_accvgpr_write_b32 a6, 0")
    jumped = bad.replace("\ts_add_i32 s0, s0, 1\n", "\ts_branch 3\n")
    assert [f[1] for f in _scan(bad)] == ["v_accvgpr_read_b32 v10, a5"]
    assert [f[1] for f in _scan(overwrite)] == ["v_accvgpr_write_b32 a6, 0"]
    assert _scan(good) == []
    assert _scan(chained) == []
    assert _scan(jumped) == []
