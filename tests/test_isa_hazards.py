"""Wait states around inline asm in the library's gfx950 device assembly.

An MFMA that reads a VGPR as a source operand needs two wait states (issued
instructions, or s_nop cycles) after a VALU instruction that wrote that VGPR.
The compiler inserts them after the instructions it generates itself, but an
instruction written as inline asm is opaque to it: an inline-asm VALU result
fed straight into an MFMA can leave too few, and the MFMA then reads the
register's old contents. The test compiles every kernel source that holds an
MFMA to assembly with the library's own flags and checks, for each MFMA, the
last writer of each source register before it, along straight-line code and
along the branches into its block. A second scan checks the inline-asm LDS
copies: the scalar write of M0 (the copy's LDS address) needs one wait state
before the copy. Runs on the CPU (hipcc cross-compiles); skipped where hipcc
is absent.
"""
from __future__ import annotations

import os
import re
import shutil
import subprocess
from collections import defaultdict
from concurrent.futures import ThreadPoolExecutor

import pytest

from w4a16_grouped_gemm_amd import build

NEED = 2  # wait states between a VALU write of a VGPR and an MFMA read of it
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

_REG = re.compile(r"\bv\[(\d+):(\d+)\]|\bv(\d+)\b")


def _vgprs(text: str) -> list[int]:
    out = []
    for m in _REG.finditer(text):
        if m.group(3) is not None:
            out.append(int(m.group(3)))
        else:
            out.extend(range(int(m.group(1)), int(m.group(2)) + 1))
    return out


def _wait_states(inst: str) -> int:
    op = inst.split()[0]
    return int(inst.split()[1].rstrip(","), 0) + 1 if op == "s_nop" else 1


def _valu_dsts(inst: str) -> list[int]:
    """VGPRs a VALU instruction (not an MFMA) writes: its first operand."""
    op = inst.split()[0]
    if (not op.startswith("v_") or op.startswith(("v_mfma", "v_cmp", "v_readlane", "v_readfirstlane", "v_accvgpr"))
            or op == "v_nop"):
        return []
    return _vgprs(inst[len(op):].split(",")[0])


def _functions(asm: str):
    """[(name, [("label", name) | ("inst", text)])] for each function of an assembly file."""
    funcs, cur = [], None
    for line in asm.splitlines():
        s = line.split(";")[0].strip()
        if not s:
            continue
        if s.endswith(":") and not s.startswith("."):
            cur = (s[:-1], [])
            funcs.append(cur)
        elif cur is None:
            continue
        elif s.startswith(".Lfunc_end"):
            cur = None
        elif s.endswith(":"):
            cur[1].append(("label", s[:-1]))
        elif not s.startswith("."):
            cur[1].append(("inst", s))
    return funcs


def _writes_m0(inst: str) -> bool:
    op = inst.split()[0]
    return op.startswith("s_") and inst[len(op):].split(",")[0].strip() == "m0"


def m0_too_close(asm: str):
    """(function, copy) for each LDS DMA copy (global_load_lds_*) whose M0, the
    LDS address it writes to, was set by the instruction right before it: a
    scalar write of M0 needs one wait state before such a copy reads it."""
    found = []
    for name, body in _functions(asm):
        prev = None
        for kind, v in body:
            if kind == "label":
                prev = None
                continue
            if v.split()[0].startswith("global_load_lds") and prev is not None and _writes_m0(prev):
                found.append((name, v))
            prev = v
    return found


def short_distances(asm: str):
    """(function, wait states, writer, mfma) for each MFMA source written by a
    VALU instruction fewer than NEED wait states before it."""
    found = []
    for name, body in _functions(asm):
        insts, block_of, into = [], {}, defaultdict(list)
        for kind, v in body:
            if kind == "label":
                block_of[len(insts)] = v
            else:
                insts.append(v)
                op = v.split()[0]
                if op.startswith("s_cbranch") or op == "s_branch":
                    into[v.split()[-1]].append(len(insts) - 1)

        def back(j, dist, srcs):
            """Writers of srcs within reach going back from instruction j,
            which lies dist wait states before the MFMA."""
            hits = []
            while j >= 0 and dist < NEED:
                if srcs.intersection(_valu_dsts(insts[j])):
                    return hits + [(dist, insts[j])]
                dist += _wait_states(insts[j])
                if j in block_of:  # the branches into this block
                    for b in into.get(block_of[j], []):
                        hits += back(b - 1, dist + 1, srcs)
                    if j > 0 and insts[j - 1].split()[0] == "s_branch":
                        return hits
                j -= 1
            return hits

        for i, inst in enumerate(insts):
            op = inst.split()[0]
            if not op.startswith("v_mfma"):
                continue
            srcs = set()
            for operand in inst[len(op):].split(",")[1:4]:
                srcs.update(_vgprs(operand))
            hits = []
            j = i - 1
            if i in block_of:
                for b in into.get(block_of[i], []):
                    hits += back(b - 1, 1, srcs)
                if i > 0 and insts[i - 1].split()[0] == "s_branch":
                    j = -1
            hits += back(j, 0, srcs)
            found += [(name, d, w, inst) for d, w in hits]
    return found


def test_scanner_flags_a_short_distance():
    """The scan itself: an inline-asm VALU write one instruction before the MFMA
    that reads it is flagged, at the fall-through and across a branch; two wait
    states (s_nop 1, or two instructions) are not."""
    head = "k:\n"
    mfma = "\tv_mfma_f32_16x16x32_bf16 v[0:3], v[4:7], v[8:11], v[12:15]\n"
    tail = ".Lfunc_end0:\n"
    asm_write = "\t;;#ASMSTART\n\tv_and_or_b32 v11, v20, s4, v21\n\t;;#ASMEND\n"
    assert len(short_distances(head + asm_write + "\tv_lshrrev_b32_e32 v30, 4, v31\n" + mfma + tail)) == 1
    assert len(short_distances(head + asm_write + mfma + tail)) == 1
    assert short_distances(head + asm_write + "\ts_nop 1\n" + mfma + tail) == []
    assert short_distances(head + asm_write + "\tv_mov_b32 v30, 0\n\tv_mov_b32 v31, 0\n" + mfma + tail) == []
    # an unrelated register, and the C operand
    assert short_distances(head + "\tv_mov_b32 v40, 0\n" + mfma + tail) == []
    assert len(short_distances(head + "\tv_mov_b32 v13, 0\n" + mfma + tail)) == 1
    # across a branch into the MFMA's block; an s_branch ends the fall-through
    branchy = (head + asm_write + "\ts_cbranch_scc1 .LBB0_2\n\tv_mov_b32 v30, 0\n\tv_mov_b32 v31, 0\n"
               "\ts_branch .LBB0_3\n.LBB0_2:\n" + mfma + ".LBB0_3:\n\ts_endpgm\n" + tail)
    assert len(short_distances(branchy)) == 1


def test_scanner_flags_an_m0_write_right_before_a_copy():
    copy = "\tglobal_load_lds_dwordx4 v[2:3], off\n"
    assert len(m0_too_close("k:\n\ts_mov_b32 m0, s4\n" + copy + ".Lfunc_end0:\n")) == 1
    assert m0_too_close("k:\n\ts_mov_b32 m0, s4\n\ts_nop 0\n" + copy + ".Lfunc_end0:\n") == []
    assert m0_too_close("k:\n\ts_mov_b32 s5, s4\n" + copy + ".Lfunc_end0:\n") == []


def _lds_dma_sources() -> list[str]:
    return [s for s in build.sources() if "global_load_lds" in open(s).read()]


def _mfma_sources() -> list[str]:
    return [s for s in build.sources() if "mfma" in open(s).read()]


_ASM_CACHE: dict[str, str] = {}


def _device_asm(srcs: list[str], tmp_dir) -> dict[str, str]:
    """gfx950 assembly of each source, compiled with the library's flags."""
    flags = [f for f in build.FLAGS if f not in ("-shared", "-fPIC")]

    def compile_one(src):
        out = os.path.join(str(tmp_dir), os.path.basename(src) + ".s")
        cmd = [HIPCC, *flags, "--cuda-device-only", "-S", "-I", os.path.join(build.ROOT, "include"), "-I",
               os.path.join(build.PKG, "csrc"), src, "-o", out]
        res = subprocess.run(cmd, capture_output=True, text=True)
        assert res.returncode == 0, res.stderr[-2000:]
        return src, open(out).read()

    todo = [s for s in srcs if s not in _ASM_CACHE]
    if todo:
        with ThreadPoolExecutor(max_workers=min(4, len(todo))) as ex:
            _ASM_CACHE.update(dict(ex.map(compile_one, todo)))
    return {s: _ASM_CACHE[s] for s in srcs}


needs_hipcc = pytest.mark.skipif(not shutil.which(HIPCC) and not os.path.exists(HIPCC), reason="hipcc not found")


@needs_hipcc
def test_no_short_valu_to_mfma_distance(tmp_path):
    srcs = _mfma_sources()
    assert srcs
    bad = []
    for src, asm in _device_asm(srcs, tmp_path).items():
        assert "v_mfma" in asm, src
        bad += [(os.path.basename(src),) + h for h in short_distances(asm)]
    assert not bad, "\n".join(f"{s} {n[:60]}: {d} wait state(s): {w} -> {m}" for s, n, d, w, m in bad[:10])


@needs_hipcc
def test_m0_set_a_wait_state_before_each_lds_copy(tmp_path):
    srcs = _lds_dma_sources()
    assert srcs
    bad = []
    for src, asm in _device_asm(srcs, tmp_path).items():
        assert "global_load_lds" in asm, src
        bad += [(os.path.basename(src),) + h for h in m0_too_close(asm)]
    assert not bad, "\n".join(f"{s} {n[:60]}: {c}" for s, n, c in bad[:10])
