"""The stream kernel's record hold (head_dim 256, explicit partitions) keeps up to
kHoldRecs partial records per wave in accumulator registers that it addresses by
number in inline asm, outside the compiler's register allocation.  That is sound
only while the compiler's own code never touches those registers and the kernel
allocates the whole AGPR file.  This checks both on the built library's gfx950
code object (disassembled with the ROCm LLVM tools): every instruction naming an
AGPR at or above kHoldBase is one of the hold's reads or writes, each hold
register is written and read, and the kernel metadata allocates 256 AGPRs."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "gqa_aware_paged_amd", "libpagedattn.so")
HEADER = os.path.join(ROOT, "gqa_aware_paged_amd", "csrc", "pa_stream.h")
LLVM = "/opt/rocm/llvm/bin"
KERNELS = [f"_ZN2pa23pa_phase1_stream_kernelILi256ENS_{t}ELi4ELb1EEEvNS_10DecodeArgsE"
           for t in ("3F16", "4BF16")]


def header_constant(name):
    text = open(HEADER).read()
    m = re.search(rf"constexpr int {name} = ([^;]+);", text)
    assert m, name
    return m.group(1)


def hold_layout():
    recs = int(header_constant("kHoldRecs"))
    stride = int(header_constant("kHoldStride"))
    base = 256 - recs * stride
    assert header_constant("kHoldBase") == "256 - kHoldRecs * kHoldStride"
    return recs, stride, base


@pytest.fixture(scope="module")
def code_object(tmp_path_factory):
    tools = [os.path.join(LLVM, t) for t in ("llvm-objcopy", "clang-offload-bundler",
                                             "llvm-objdump", "llvm-readelf")]
    if not os.path.exists(LIB):
        pytest.skip("libpagedattn.so is not built")
    if not all(os.path.exists(t) for t in tools):
        pytest.skip("ROCm LLVM tools not found")
    d = tmp_path_factory.mktemp("co")
    fatbin, co = str(d / "fatbin"), str(d / "gfx950.co")
    subprocess.run([tools[0], f"--dump-section=.hip_fatbin={fatbin}", LIB, str(d / "lib.so")],
                   check=True)
    subprocess.run([tools[1], "--unbundle", "--type=o", f"--input={fatbin}",
                    "--targets=hipv4-amdgcn-amd-amdhsa--gfx950", f"--output={co}"], check=True)
    yield co, tools
    shutil.rmtree(d, ignore_errors=True)


AGPR = re.compile(r"\ba\[(\d+):(\d+)\]|\ba(\d+)\b")


def agprs(operands):
    out = []
    for m in AGPR.finditer(operands):
        if m.group(3) is not None:
            out.append(int(m.group(3)))
        else:
            out.extend(range(int(m.group(1)), int(m.group(2)) + 1))
    return out


@pytest.mark.parametrize("kernel", KERNELS, ids=["f16", "bf16"])
def test_hold_registers_outside_compiler_allocation(code_object, kernel):
    co, tools = code_object
    recs, stride, base = hold_layout()
    dis = subprocess.run([tools[2], "-d", f"--disassemble-symbols={kernel}", co],
                         check=True, capture_output=True, text=True).stdout
    written, read, n_insts = set(), set(), 0
    for line in dis.splitlines():
        code = line.split("//")[0].strip()
        if not code or code.endswith(">:") or " " not in code:
            continue
        n_insts += 1
        op, operands = code.split(None, 1)
        regs = agprs(operands)
        high = [r for r in regs if r >= base]
        if not high:
            continue
        if op == "v_accvgpr_write_b32" and len(regs) == 1:
            written.add(regs[0])
        elif op == "v_accvgpr_read_b32" and len(regs) == 1:
            read.add(regs[0])
        else:
            pytest.fail(f"{kernel}: compiler code uses hold register(s) {high}: {code}")
    assert n_insts > 1000, "kernel not found in the code object"
    hold = set(range(base, base + recs * stride))
    assert written == hold and read == hold

    notes = subprocess.run([tools[3], "--notes", co], check=True, capture_output=True,
                           text=True).stdout
    blocks = re.split(r"\n\s+- \.agpr_count:", notes)
    mine = [b for b in blocks if f".name:           {kernel}" in b]
    assert len(mine) == 1
    assert int(mine[0].split()[0]) == 256
