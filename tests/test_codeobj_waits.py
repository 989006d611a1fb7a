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
from codeobj import disassemble, instruction_lines


def test_every_lds_copy_waits_after_setting_m0(tmp_path):
    ins = instruction_lines(disassemble(tmp_path))
    copies = [i for i, x in enumerate(ins)
              if x.startswith("global_load_lds") or (x.startswith("buffer_load") and x.split()[-1] == "lds")]
    assert len(copies) > 100, "the attention kernels' copies are missing from the disassembly"
    bad = []
    for i in copies:
        prev, prev2 = ins[i - 1], ins[i - 2]
        if not (prev.startswith("s_nop") and "m0" in prev2.split(",")[0]):
            bad.append((prev2, prev, ins[i]))
    assert not bad, f"{len(bad)} of {len(copies)} copies lack the M0 wait state, e.g. {bad[:3]}"
