"""The built device code keeps the wait state gfx940-class parts need between
a transcendental instruction (exp, log, rcp, rsq, sqrt, sin, cos) and a VALU
instruction that reads its result. The compiler inserts it for the
instructions it generates, but not for the inside of inline asm blocks: an
asm v_fma_mix_f32 scheduled right after a v_exp_f32 whose result it read got
the register's previous contents (wrong attention rows for a few bit pairs,
depending on scheduling). This test disassembles the library's own gfx950
code objects (the objects of this build, under the package's _build folder)
and fails on any such adjacency."""

import os
import re
import shutil
import subprocess

import pytest

from bit_kv_cache_groupwise_amd import build as B

LLVM = os.path.join(B.ROCM, "llvm", "bin")
TRANS = re.compile(r"^\s*(v_(?:exp|log|rcp|rcp_iflag|rsq|sqrt|sin|cos)_f(?:16|32))\w*\s+v(\d+)\b")
INSN = re.compile(r"^\s*([a-z_0-9]+)\s+(.*?)\s*(?://.*)?$")
TRANS_OP = re.compile(r"^v_(?:exp|log|rcp|rcp_iflag|rsq|sqrt|sin|cos)_f(?:16|32)")


def _reads(operands: str, reg: int) -> bool:
    """Whether VGPR `reg` is among the source operands (all but the first)."""
    srcs = operands.split(",")[1:]
    for op in srcs:
        op = op.strip()
        m = re.match(r"^-?\|?v(\d+)\b", op)
        if m and int(m.group(1)) == reg:
            return True
        m = re.match(r"^-?v\[(\d+):(\d+)\]", op)
        if m and int(m.group(1)) <= reg <= int(m.group(2)):
            return True
    return False


def hazards(disasm_lines):
    """(trans instruction, next instruction) pairs where a non-transcendental
    VALU instruction reads the transcendental's result in the next slot."""
    out = []
    prev = None
    for line in disasm_lines:
        m = INSN.match(line)
        if not m or line.startswith(("Disassembly", " ", "\t\t")) and not line.startswith("\t"):
            continue
        op, operands = m.group(1), m.group(2)
        if not (op.startswith(("v_", "s_", "ds_", "global_", "buffer_", "flat_", "scratch_"))):
            continue
        if prev is not None and op.startswith("v_") and not TRANS_OP.match(op) and _reads(operands, prev[1]):
            out.append((prev[0], line.strip()))
        t = TRANS.match(line)
        prev = (line.strip(), int(t.group(2))) if t else None
    return out


def _device_code(obj, tmp):
    fat = os.path.join(tmp, "fat.bin")
    co = os.path.join(tmp, "dev.co")
    subprocess.run([os.path.join(LLVM, "llvm-objcopy"), "--dump-section", f".hip_fatbin={fat}", obj,
                    os.path.join(tmp, "host.o")], check=True, capture_output=True)
    subprocess.run([os.path.join(LLVM, "clang-offload-bundler"), "--unbundle", "--type=o", f"--input={fat}",
                    f"--targets=hipv4-amdgcn-amd-amdhsa--{B.ARCH}", f"--output={co}"], check=True, capture_output=True)
    r = subprocess.run([os.path.join(LLVM, "llvm-objdump"), "-d", f"--mcpu={B.ARCH}", co], check=True,
                       capture_output=True, text=True)
    return r.stdout.splitlines()


def test_scanner_flags_a_planted_adjacency():
    lines = ["\tv_exp_f32_e32 v0, v0", "\tv_fma_mix_f32 v149, v1, v0, v149 op_sel:[1,0,0] op_sel_hi:[1,0,0]",
             "\tv_rcp_f32_e32 v4, v3", "\ts_nop 0", "\tv_mul_f32_e32 v5, v4, v4",
             "\tv_sqrt_f32_e32 v8, v9", "\tv_add_f32_e32 v10, v11, v12",
             "\tv_exp_f32_e32 v20, v20", "\tv_pk_mul_f32 v[30:31], v[19:20], v[2:3]"]
    found = hazards(lines)
    assert [f[1].split()[0] for f in found] == ["v_fma_mix_f32", "v_pk_mul_f32"]


@pytest.mark.parametrize("obj", [u[1] for u in B.units() if u[3]])
def test_no_instruction_reads_a_transcendental_result_in_the_next_slot(obj, tmp_path):
    path = os.path.join(B.BUILD, obj)
    if not os.path.exists(path) or not os.path.exists(os.path.join(LLVM, "llvm-objdump")):
        pytest.skip("library objects not built here")
    found = hazards(_device_code(path, str(tmp_path)))
    assert not found, f"{obj}: {len(found)} reads of a transcendental result in the next slot, e.g. {found[:3]}"
