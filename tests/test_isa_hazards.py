"""Wait-state rules around the hand-scheduled assembly blocks, the use of M0, and the cache
policy of the cache streams (CPU only).

The GQA kernel issues some DPP arithmetic as inline assembly. The compiler
inserts the wait states gfx950 needs between dependent instructions of the
code it generates, but not across the boundary of an assembly block. This
test compiles the kernels to gfx950 assembly and scans it linearly for the
rules that apply to those blocks. The rules are the CDNA wait-state
requirements as AMD documents them (the "Manually Inserted Wait States
(NOPs)" table of the CDNA3 / CDNA4 instruction-set reference guides) and as
LLVM's AMDGPU hazard recognizer enforces them for gfx940 / gfx950 code:

* a VALU instruction writes a VGPR, then a DPP instruction reads it as its
  lane-shuffled operand (src0): at least 2 wait states in between;
* a VALU instruction writes a VGPR, then v_permlane16/32_swap (new in CDNA4)
  reads it: at least 2 wait states;
* a dot-product instruction (v_dot2c_f32_bf16) writes a VGPR, then another
  VALU instruction reads it: at least 3 wait states; none are needed when the
  reader is the same dot instruction accumulating into that register.

``s_nop N`` counts N + 1 wait states, any other instruction one. The scan
ignores branches (it follows program order), which covers every block the
assembly helpers emit: each one opens and closes with its own wait states.

M0: the direct-to-LDS copies are assembly blocks that write M0 (the LDS
address) and issue the copy right after. The compiler must not read M0 for
anything of its own in these kernels; the scan checks that every instruction
naming M0 is one of those writes, that each write is followed at once by its
copy, and that no instruction that reads M0 implicitly appears elsewhere.
"""

from __future__ import annotations

import functools
import os
import re
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mla_kv_cache_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

pytestmark = pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")


@functools.lru_cache(maxsize=None)
def _assembly_of(src: str) -> tuple[str, ...]:
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, os.path.basename(src) + ".s")
        cmd = [HIPCC, "-O3", "-std=c++17", "--offload-arch=gfx950", "--cuda-device-only", "-S",
               "-I", os.path.join(ROOT, "include"), "-I", CSRC,
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-o", out, src]
        subprocess.run(cmd, check=True, capture_output=True)
        with open(out) as f:
            return tuple(ln.split(";")[0].strip() for ln in f.read().splitlines())


def _assembly(src: str, tmp_path=None) -> list[str]:
    """The gfx950 assembly of one source, compiled once per test session."""
    return list(_assembly_of(src))


def _vregs(tok: str) -> set[str]:
    tok = tok.rstrip(",")
    m = re.match(r"v\[(\d+):(\d+)\]$", tok)
    if m:
        return {f"v{i}" for i in range(int(m.group(1)), int(m.group(2)) + 1)}
    return {tok} if re.match(r"v\d+$", tok) else set()


def _is_instr(t: str) -> bool:
    return bool(re.match(r"^[sv]_|^ds_|^global_|^buffer_|^flat_|^scratch_", t))


def _operands(t: str) -> list[str]:
    parts = t.replace(",", " ").split()
    return parts[1:]


def _dst_src(t: str):
    ops = _operands(t)
    if not ops:
        return set(), set()
    dst = _vregs(ops[0])
    src = set().union(*(_vregs(o) for o in ops[1:])) if len(ops) > 1 else set()
    return dst, src


def _violations(lines: list[str]) -> list[str]:
    bad = []
    ins = [t for t in lines if _is_instr(t)]
    for i, t in enumerate(ins):
        op = t.split()[0]
        dst, src = _dst_src(t)
        reads = src | (dst if op.startswith(("v_dot2c", "v_fmac", "v_mac")) else set())
        need = 0
        if "_dpp" in op or " row_" in t or "quad_perm" in t:
            # The lane-shuffled operand is src0; the other operands (and a
            # v_dot2c accumulator) are read through the ordinary path, where a
            # back-to-back dependent v_dot2c measured correct.
            need = 2
            ops = _operands(t)
            reads = _vregs(ops[1]) if len(ops) > 1 else set()
        if op.startswith(("v_permlane16_swap", "v_permlane32_swap")):
            need = 2
            reads = reads | dst
        if need:
            ws, j = 0, i - 1
            while j >= 0 and ws < need:
                p = ins[j]
                if p.startswith("s_nop"):
                    ws += int(p.split()[1], 0) + 1
                else:
                    if p.startswith("v_") and _dst_src(p)[0] & reads:
                        bad.append(f"{p}  ->  {t}  ({ws} wait states, need {need})")
                        break
                    ws += 1
                j -= 1
        if op.startswith("v_dot2c_f32_bf16"):
            ws, j = 0, i + 1
            while j < len(ins) and ws < 3:
                n = ins[j]
                if n.startswith("s_nop"):
                    ws += int(n.split()[1], 0) + 1
                else:
                    nop_ = n.split()[0]
                    nd, ns = _dst_src(n)
                    chained = nop_.startswith("v_dot2c_f32_bf16") and nd == dst
                    if n.startswith("v_") and not chained and (ns | (nd if nop_.startswith("v_dot2c") else set())) & dst:
                        bad.append(f"{t}  ->  {n}  ({ws} wait states, need 3)")
                        break
                    ws += 1
                j += 1
    return bad


# Instructions that read M0 without naming it (gfx9 family).
_M0_IMPLICIT = ("s_movrel", "v_movrel", "s_sendmsg", "ds_gws", "v_interp", "ds_ordered_count",
                "ds_append", "ds_consume", "s_ttracedata")


def _is_lds_copy(t: str) -> bool:
    op = t.split()[0]
    return ((op.startswith("buffer_load") and (t.endswith(" lds") or " lds " in t))
            or op.startswith(("global_load_lds", "scratch_load_lds")))


def _m0_violations(lines: list[str]) -> list[str]:
    bad = []
    ins = [t for t in lines if _is_instr(t)]
    for i, t in enumerate(ins):
        op = t.split()[0]
        m0_write = re.match(r"s_mov_b32 m0, s\d+$", t) is not None
        if re.search(r"\bm0\b", t) and not m0_write:
            bad.append(f"names m0: {t}")
        if m0_write and not (i + 1 < len(ins) and _is_lds_copy(ins[i + 1])):
            bad.append(f"m0 write not followed by its copy: {t}")
        if _is_lds_copy(t) and not (i > 0 and re.match(r"s_mov_b32 m0, s\d+$", ins[i - 1])):
            bad.append(f"copy without its m0 write: {t}")
        if op.startswith(_M0_IMPLICIT):
            bad.append(f"reads m0 implicitly: {t}")
    return bad


@pytest.mark.parametrize("name", ["gqa_decode.hip", "gqa_mma16.hip", "gqa_matrix.hip", "mla_decode.hip", "lse_merge.hip", "mla_absorb.hip"])
def test_m0_is_only_used_by_the_copy_blocks(name, tmp_path):
    lines = _assembly(os.path.join(CSRC, name), tmp_path)
    bad = _m0_violations(lines)
    assert not bad, f"{len(bad)} M0 uses outside the copy blocks, first: " + "; ".join(bad[:5])


def test_m0_scanner_catches_planted_uses():
    lines = [
        "s_mov_b32 m0, s4",
        "buffer_load_dwordx4 v1, s[8:11], s12 offen lds",
        "s_mov_b32 m0, s5",                      # not followed by a copy
        "v_mov_b32 v2, v3",
        "global_load_lds_dwordx4 v4, off",       # no m0 write right before
        "v_readlane_b32 s6, v7, m0",             # the compiler reading m0
        "s_movrels_b32 s1, s2",                  # implicit reader
    ]
    assert len(_m0_violations(lines)) == 4


@pytest.mark.parametrize("name", ["gqa_decode.hip", "mla_decode.hip", "lse_merge.hip"])
def test_assembly_respects_wait_states(name, tmp_path):
    lines = _assembly(os.path.join(CSRC, name), tmp_path)
    assert any(_is_instr(t) for t in lines)
    bad = _violations(lines)
    assert not bad, f"{len(bad)} wait-state violations, first: " + "; ".join(bad[:5])


def test_scanner_catches_planted_hazards():
    # A DPP read right after a VALU write, a permlane right after a write, and a
    # dot result read one instruction later must be reported; a dot chain
    # accumulating into one register, followed by enough wait states, must not.
    lines = [
        "v_mov_b32 v1, v2",
        "v_max_f32_dpp v3, v1, v1 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf",
        "s_nop 4",
        "v_mov_b32 v5, v6",
        "v_permlane16_swap_b32 v7, v5",
        "s_nop 4",
        "v_dot2c_f32_bf16 v9, v10, v11",
        "v_mov_b32 v12, v13",
        "v_mul_f32 v14, 2.0, v9",
        "s_nop 4",
        "v_dot2c_f32_bf16 v20, v21, v22",
        "v_dot2c_f32_bf16 v20, v23, v24",
        "s_nop 2",
        "v_mul_f32 v25, 2.0, v20",
    ]
    bad = _violations(lines)
    assert len(bad) == 3, bad


# Cache policy of the cache streams: every K, V and latent copy (the
# direct-to-LDS copies and the V register loads) carries the non-temporal
# policy, which the decode kernels' streaming rate depends on. The scan
# counts, per kernel source, the copies that carry `nt` and fails on any
# that does not.
@pytest.mark.parametrize("name,min_copies", [("gqa_decode.hip", 2), ("gqa_mma16.hip", 1), ("gqa_matrix.hip", 1),
                                             ("mla_decode.hip", 1)])
def test_cache_streams_are_non_temporal(name, min_copies, tmp_path):
    lines = _assembly(os.path.join(CSRC, name), tmp_path)
    copies = [t for t in lines if _is_instr(t) and _is_lds_copy(t)]
    assert len(copies) >= min_copies, name
    plain = [t for t in copies if " nt" not in t]
    assert not plain, plain[:4]
    if name == "gqa_decode.hip":  # the V rows of the position-per-lane kernel go to registers
        vloads = [t for t in lines if t.startswith("buffer_load_dwordx4 v[") and "offen" in t]
        assert vloads and all(" nt" in t for t in vloads), [t for t in vloads if " nt" not in t][:4]
