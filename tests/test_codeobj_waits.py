"""Host-side check of the built library's gfx950 code (no GPU needed).

Every direct global->LDS copy (global_load_lds_*, or buffer_load_* ... lds)
takes its LDS address from M0.  On gfx950 such a copy needs one wait state after an SALU write of M0;
without it the copy can take the previous M0 and land its row in the previous
copy's slot.  The copies are issued from inline asm, which the compiler does not
look into, so the asm carries the wait state itself.  This test disassembles
every gfx950 code object in libsparse_attn.so (llvm-objdump from the ROCm
toolchain) and checks that each copy is preceded by `s_nop` right after the
instruction that sets M0.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "sparse_latent_attention_02_amd", "libsparse_attn.so")
LLVM = "/opt/rocm/llvm/bin"
TARGET = "hipv4-amdgcn-amd-amdhsa--gfx950"


def _tool(name):
    p = os.path.join(LLVM, name)
    return p if os.path.exists(p) else shutil.which(name)


def gfx950_instructions(tmp_path):
    """Instruction mnemonics + operands of every gfx950 code object in the library, in order."""
    objcopy, bundler, objdump = _tool("llvm-objcopy"), _tool("clang-offload-bundler"), _tool("llvm-objdump")
    if not (objcopy and bundler and objdump):
        pytest.skip("ROCm LLVM tools not found")
    if not os.path.exists(LIB):
        from sparse_latent_attention_02_amd import build
        build.build()
    fat = tmp_path / "fatbin.bin"
    subprocess.run([objcopy, f"--dump-section=.hip_fatbin={fat}", LIB], check=True)
    data = fat.read_bytes()
    starts = [m.start() for m in re.finditer(re.escape(b"__CLANG_OFFLOAD_BUNDLE__"), data)]
    assert starts, "no offload bundle in the library"
    out = []
    for i, s0 in enumerate(starts):
        part = tmp_path / f"b{i}.bin"
        part.write_bytes(data[s0: starts[i + 1] if i + 1 < len(starts) else len(data)])
        co = tmp_path / f"co{i}.o"
        subprocess.run([bundler, "--unbundle", "--type=o", f"--input={part}", f"--targets={TARGET}",
                        f"--output={co}"], check=True)
        text = subprocess.run([objdump, "-d", "--mcpu=gfx950", str(co)], check=True, capture_output=True,
                              text=True).stdout
        for line in text.splitlines():
            ins = line.split("//")[0].strip()
            if ins and not ins.endswith(":") and not ins.startswith("Disassembly"):
                out.append(ins)
    return out


def test_every_lds_copy_waits_after_setting_m0(tmp_path):
    ins = gfx950_instructions(tmp_path)
    copies = [i for i, x in enumerate(ins)
              if x.startswith("global_load_lds") or (x.startswith("buffer_load") and x.split()[-1] == "lds")]
    assert len(copies) > 100, "the attention kernels' copies are missing from the disassembly"
    bad = []
    for i in copies:
        prev, prev2 = ins[i - 1], ins[i - 2]
        if not (prev.startswith("s_nop") and "m0" in prev2.split(",")[0]):
            bad.append((prev2, prev, ins[i]))
    assert not bad, f"{len(bad)} of {len(copies)} copies lack the M0 wait state, e.g. {bad[:3]}"
