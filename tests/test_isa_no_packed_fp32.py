"""The build disables packed fp32 arithmetic (hipcc -Xclang -target-feature
-Xclang -packed-fp32-ops): no kernel of the library may contain a packed fp32
add, multiply or fma. Checked in the gfx950 code objects the build produced
(CPU only, disassembled with the toolchain's llvm-objdump)."""

import glob
import os
import subprocess

import pytest

from test_merge_isa import BUILD, _disassemble, _tool

PACKED = ("v_pk_add_f32", "v_pk_mul_f32", "v_pk_fma_f32")


def _objects():
    """The built objects that carry device code (a .hip_fatbin section); the
    host-only ABI layer has none."""
    tool = _tool("llvm-objdump")
    out = []
    for path in sorted(glob.glob(os.path.join(BUILD, "*.hip.o"))):
        if tool:
            heads = subprocess.run([tool, "-h", path], capture_output=True, text=True).stdout
            if ".hip_fatbin" not in heads:
                continue
        out.append(path)
    return out


@pytest.mark.parametrize("obj", [os.path.basename(p) for p in _objects()] or ["none"])
def test_no_packed_fp32_instructions(obj, tmp_path):
    path = os.path.join(BUILD, obj)
    if not os.path.exists(path) or not all(_tool(t) for t in ("llvm-objcopy",
                                                              "clang-offload-bundler",
                                                              "llvm-objdump")):
        pytest.skip("the library's objects or the ROCm LLVM tools are absent")
    kernels = _disassemble(path, tmp_path)
    assert kernels, "no kernel in the code object"
    found = {name: sorted({i.split()[0] for i in ins if i.split() and i.split()[0] in PACKED})
             for name, ins in kernels.items()}
    found = {k: v for k, v in found.items() if v}
    assert not found, f"packed fp32 instructions in {obj}: {found}"
