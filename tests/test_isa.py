"""Instruction-level checks of the built library's gfx950 code objects (no GPU).

The library's device code is disassembled with the ROCm LLVM tools and
checked for two classes of instruction that must not appear:

* FLAT memory instructions.  Every table, staging buffer and scratch array
  of the kernels lives in LDS and is addressed through the LDS array itself,
  so that accesses compile to DS instructions.  A FLAT access whose address
  came from an LDS offset (for instance after a pointer went through an
  integer) lands outside the shared aperture and faults the GPU with a memory
  aperture violation; one such fault hit an early version of the scan.
* Packed FP32 arithmetic (v_pk_add_f32, v_pk_mul_f32, v_pk_fma_f32): the
  build switches the feature off for all device code.
"""
import os
import re
import shutil
import subprocess
import tempfile

import pytest

from approximate_nearest_neighbour_amd import binding as B

LLVM = "/opt/rocm/llvm/bin"
TARGET = "hipv4-amdgcn-amd-amdhsa--gfx950"
MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"


def tool(name):
    p = os.path.join(LLVM, name)
    if not os.path.exists(p):
        pytest.skip(f"{name} not installed")
    return p


@pytest.fixture(scope="module")
def disassembly():
    """{kernel symbol: [instruction mnemonics]} over every code object in the
    library's .hip_fatbin section (one offload bundle per translation unit)."""
    lib = B.LIB_PATH
    if not os.path.exists(lib):
        pytest.skip("libivfpq.so not built")
    tmp = tempfile.mkdtemp()
    try:
        fat = os.path.join(tmp, "all.fatbin")
        subprocess.run([tool("llvm-objcopy"), f"--dump-section=.hip_fatbin={fat}", lib,
                        os.path.join(tmp, "discard.so")], check=True, capture_output=True)
        blob = open(fat, "rb").read()
        starts = [m.start() for m in re.finditer(re.escape(MAGIC), blob)]
        assert starts, "no offload bundle in the library"
        kernels = {}
        for n, s in enumerate(starts):
            end = starts[n + 1] if n + 1 < len(starts) else len(blob)
            part = os.path.join(tmp, f"b{n}.fatbin")
            open(part, "wb").write(blob[s:end])
            co = os.path.join(tmp, f"b{n}.co")
            r = subprocess.run([tool("clang-offload-bundler"), "--unbundle", "--type=o",
                                f"--input={part}", f"--targets={TARGET}", f"--output={co}"],
                               capture_output=True)
            if r.returncode != 0 or not os.path.exists(co) or os.path.getsize(co) == 0:
                continue
            dis = subprocess.run([tool("llvm-objdump"), "-d", "--no-show-raw-insn", co],
                                 check=True, capture_output=True, text=True).stdout
            name = None
            for line in dis.splitlines():
                m = re.match(r"^[0-9a-f]+ <(.+)>:$", line)
                if m:
                    name = m.group(1)
                    kernels.setdefault(name, [])
                    continue
                m = re.match(r"^\s+([a-z_][a-z0-9_]*)", line)
                if m and name:
                    kernels[name].append(m.group(1))
        return kernels
    finally:
        shutil.rmtree(tmp, ignore_errors=True)


def test_code_objects_found(disassembly):
    names = " ".join(disassembly)
    for k in ("scan_items_kernel", "coarse_mfma_kernel", "flat_gemm_kernel", "encode_kernel",
              "merge_items_kernel"):
        assert k in names, k
    # the scan kernels read their tables with DS instructions
    scan = [v for n, v in disassembly.items() if "scan_items_kernel" in n]
    assert scan and all(any(i.startswith("ds_read") for i in ins) for ins in scan)


def test_no_flat_memory_instructions(disassembly):
    bad = {n: sorted({i for i in ins if re.match(r"flat_(load|store|atomic)", i)})
           for n, ins in disassembly.items()}
    bad = {n: v for n, v in bad.items() if v}
    assert not bad, f"FLAT memory instructions in {len(bad)} kernels: {list(bad.items())[:3]}"


def test_no_packed_fp32_arithmetic(disassembly):
    bad = {n: sorted({i for i in ins if re.match(r"v_pk_(add|mul|fma)_f32", i)})
           for n, ins in disassembly.items()}
    bad = {n: v for n, v in bad.items() if v}
    assert not bad, f"packed FP32 instructions in {len(bad)} kernels: {list(bad.items())[:3]}"
