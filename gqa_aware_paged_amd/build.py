"""Build libpagedattn.so for gfx950 with hipcc (in-tree, no JIT cache)."""
from __future__ import annotations

import collections
import os
import re
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "pagedattn.hip")
DEPS = [SRC, os.path.join(PKG, "csrc", "pa_kernels.h"), os.path.join(PKG, "csrc", "pa_prefill.h"),
        os.path.join(PKG, "csrc", "pa_stream.h"),
        os.path.join(ROOT, "include", "pagedattn.h")]
SO = os.path.join(PKG, "libpagedattn.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-fvisibility=hidden",
    # packed-fp32 VALU forms are kept out of the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def command(out: str = SO):
    return [HIPCC, *FLAGS, "-I", os.path.join(ROOT, "include"), SRC, "-o", out]


LLVM = "/opt/rocm/llvm/bin"
STREAM_H = os.path.join(PKG, "csrc", "pa_stream.h")
# the explicit-partition stream kernels at head_dim 256, which hold records in AGPRs
HOLD_KERNELS = [f"_ZN2pa23pa_phase1_stream_kernelILi256ENS_{t}ELi4ELb1EEEvNS_10DecodeArgsE"
                for t in ("3F16", "4BF16")]
_AGPR = re.compile(r"\ba\[(\d+):(\d+)\]|\ba(\d+)\b")


def hold_layout():
    """(first hold AGPR, hold register count) restated from pa_stream.h."""
    text = open(STREAM_H).read()
    recs = int(re.search(r"constexpr int kHoldRecs = (\d+);", text).group(1))
    stride = int(re.search(r"constexpr int kHoldStride = (\d+);", text).group(1))
    return 256 - recs * stride, recs * stride


def hold_register_problems(lib: str = SO) -> list:
    """Checks the gfx950 code object of `lib` (disassembled with the ROCm LLVM tools)
    for what the stream kernel's record hold assumes: no compiler-generated instruction
    names an AGPR of the hold, every hold register is written and read the same number
    of times, and the kernel allocates all 256 AGPRs.  Returns the problems found."""
    base, n = hold_layout()
    tools = {t: os.path.join(LLVM, t) for t in ("llvm-objcopy", "clang-offload-bundler",
                                                "llvm-objdump", "llvm-readelf")}
    problems = []
    with tempfile.TemporaryDirectory() as d:
        fatbin, co = os.path.join(d, "fatbin"), os.path.join(d, "gfx950.co")
        subprocess.run([tools["llvm-objcopy"], f"--dump-section=.hip_fatbin={fatbin}", lib,
                        os.path.join(d, "lib.so")], check=True)
        subprocess.run([tools["clang-offload-bundler"], "--unbundle", "--type=o", f"--input={fatbin}",
                        "--targets=hipv4-amdgcn-amd-amdhsa--gfx950", f"--output={co}"], check=True)
        notes = subprocess.run([tools["llvm-readelf"], "--notes", co], check=True,
                               capture_output=True, text=True).stdout
        for kernel in HOLD_KERNELS:
            dis = subprocess.run([tools["llvm-objdump"], "-d", f"--disassemble-symbols={kernel}", co],
                                 check=True, capture_output=True, text=True).stdout
            written, read, insts = collections.Counter(), collections.Counter(), 0
            for line in dis.splitlines():
                code = line.split("//")[0].strip()
                if not code or code.endswith(">:") or " " not in code:
                    continue
                insts += 1
                op, operands = code.split(None, 1)
                regs = []
                for m in _AGPR.finditer(operands):
                    if m.group(3) is not None:
                        regs.append(int(m.group(3)))
                    else:
                        regs.extend(range(int(m.group(1)), int(m.group(2)) + 1))
                if not any(r >= base for r in regs):
                    continue
                if op == "v_accvgpr_write_b32" and len(regs) == 1:
                    written[regs[0]] += 1
                elif op == "v_accvgpr_read_b32" and len(regs) == 1:
                    read[regs[0]] += 1
                else:
                    problems.append(f"{kernel}: compiler code names a hold AGPR: {code}")
            hold = set(range(base, base + n))
            if insts < 1000:
                problems.append(f"{kernel}: not found in the code object")
            elif set(written) != hold or set(read) != hold:
                problems.append(f"{kernel}: hold registers not all written and read")
            elif len(set(written.values())) != 1 or len(set(read.values())) != 1:
                problems.append(f"{kernel}: uneven writes or reads of the hold registers")
            block = [b for b in re.split(r"\n\s+- \.agpr_count:", notes)
                     if f".name:           {kernel}" in b]
            if len(block) != 1 or int(block[0].split()[0]) != 256:
                problems.append(f"{kernel}: the kernel does not allocate all 256 AGPRs")
    return problems


def build(verbose: bool = False) -> str:
    tmp = SO + ".tmp"
    cmd = command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed to build libpagedattn.so")
    # the record hold's registers lie outside the compiler's allocation: a build in
    # which the compiler's own code reaches them is rejected, not installed
    if all(os.path.exists(os.path.join(LLVM, t)) for t in ("llvm-objcopy", "clang-offload-bundler",
                                                            "llvm-objdump", "llvm-readelf")):
        problems = hold_register_problems(tmp)
        if problems:
            os.remove(tmp)
            raise RuntimeError("libpagedattn.so rejected:\n" + "\n".join(problems))
    elif verbose:
        print("ROCm LLVM tools not found: the record-hold register check is skipped", flush=True)
    os.replace(tmp, SO)
    return SO


def is_stale() -> bool:
    if not os.path.exists(SO):
        return True
    t = os.path.getmtime(SO)
    return any(os.path.getmtime(d) > t for d in DEPS)


if __name__ == "__main__":
    print(build(verbose=True))
