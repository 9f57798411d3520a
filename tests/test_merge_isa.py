"""The in-launch merge's hand-off between workgroups, checked in the code the
build produced (CPU only: the gfx950 code objects of the selecting decodes
are disassembled with the toolchain's llvm-objdump).

The split partials pass between workgroups of one launch (the last split of
a (request, KV head) to finish merges them). The kernels rely on this
instruction sequence, and a toolchain that lowered the accesses differently
must fail the build check rather than merge stale partials:
- the partials are written with agent-scope stores (global_store ... sc1:
  written through the chiplet's cache);
- the writer waits for its stores (s_waitcnt vmcnt(0)) before the
  arrival counter's atomic add;
- the merging workgroup reads the partials with agent-scope loads
  (global_load ... sc1: past the chiplet's cache) after the add;
- no whole-cache write-back or invalidation (buffer_wbl2 / buffer_inv) is
  emitted (the accesses above are the only ones that need to be coherent).
"""

import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BUILD = os.path.join(ROOT, "sparse_long_context_page_amd", "_build")
OBJECTS = ("ps_select_decode.hip.o", "ps_select_topdelta_decode.hip.o")
LLVM = "/opt/rocm/llvm/bin"
TARGET = "hipv4-amdgcn-amd-amdhsa--gfx950"


def _tool(name):
    path = os.path.join(LLVM, name)
    return path if os.path.exists(path) else shutil.which(name)


def _disassemble(obj, tmp_path):
    fat = tmp_path / "fatbin.bin"
    co = tmp_path / "device.co"
    subprocess.run([_tool("llvm-objcopy"), f"--dump-section=.hip_fatbin={fat}", obj, os.devnull],
                   check=True, capture_output=True)
    subprocess.run([_tool("clang-offload-bundler"), "--unbundle", "--type=o", f"--input={fat}",
                    f"--targets={TARGET}", f"--output={co}"], check=True, capture_output=True)
    out = subprocess.run([_tool("llvm-objdump"), "-d", "--mcpu=gfx950", str(co)], check=True,
                         capture_output=True, text=True).stdout
    kernels, name = {}, None
    for line in out.splitlines():
        m = re.match(r"^[0-9a-f]+ <(\S+)>:$", line)
        if m:
            name = m.group(1)
            kernels[name] = []
        elif name and line.strip():
            kernels[name].append(line.split("//")[0].strip())
    return kernels


@pytest.mark.parametrize("obj", OBJECTS)
def test_merge_handoff_instructions(obj, tmp_path):
    path = os.path.join(BUILD, obj)
    if not os.path.exists(path) or not all(_tool(t) for t in ("llvm-objcopy",
                                                              "clang-offload-bundler",
                                                              "llvm-objdump")):
        pytest.skip("the library's objects or the ROCm LLVM tools are absent")
    kernels = {k: v for k, v in _disassemble(path, tmp_path).items() if "decode" in k}
    assert kernels, "no decode kernel in the code object"
    for name, ins in kernels.items():
        ops = [i.split()[0] if i.split() else "" for i in ins]
        adds = [n for n, op in enumerate(ops) if op == "global_atomic_add"]
        assert adds, f"{name}: no arrival counter"
        first_add = adds[0]
        stores_sc1 = [n for n, i in enumerate(ins)
                      if ops[n].startswith("global_store") and i.endswith(" sc1")]
        loads_sc1 = [n for n, i in enumerate(ins)
                     if ops[n].startswith("global_load") and i.endswith(" sc1")]
        assert len([n for n in stores_sc1 if n < first_add]) >= 3, \
            f"{name}: partials not written with agent-scope stores before the count"
        assert any(i == "s_waitcnt vmcnt(0)" for i in ins[:first_add]), \
            f"{name}: no wait for the stores before the count"
        assert any(n > first_add for n in loads_sc1), \
            f"{name}: partials not read with agent-scope loads after the count"
        assert not any(op in ("buffer_wbl2", "buffer_inv") for op in ops), \
            f"{name}: whole-cache write-back or invalidation emitted"
