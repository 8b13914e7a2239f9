"""The stream kernel's record hold (head_dim 256, explicit partitions) keeps up to
kHoldRecs partial records per wave in accumulator registers that it addresses by
number in inline asm, outside the compiler's register allocation.  That is sound
only while the compiler's own code never touches those registers and the kernel
allocates the whole AGPR file.  The build rejects a library that breaks either
(gqa_aware_paged_amd.build.hold_register_problems, on the gfx950 code object
disassembled with the ROCm LLVM tools); this runs the same check on the library in
the tree, so a library built some other way is covered too."""
import os

import pytest

from gqa_aware_paged_amd import build

TOOLS = ("llvm-objcopy", "clang-offload-bundler", "llvm-objdump", "llvm-readelf")


def test_hold_registers_outside_compiler_allocation():
    if not os.path.exists(build.SO):
        pytest.skip("libpagedattn.so is not built")
    if not all(os.path.exists(os.path.join(build.LLVM, t)) for t in TOOLS):
        pytest.skip("ROCm LLVM tools not found")
    base, n = build.hold_layout()
    assert base + n == 256 and n > 0
    assert build.hold_register_problems() == []
