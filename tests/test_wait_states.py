"""Host-side check of the built library's gfx950 code (no GPU needed): every
instruction that uses the result of an MFMA, a transcendental, a DPP source or a
v_readlane comes after the wait states the hardware needs, on every
control-flow path (see wait_states.py for the rules).

The decode kernel's score product once ended in a branch (the next stages'
index fetch) whose taken side read the accumulators four to six wait states
after the last MFMA, where eight are needed, with no s_nop from the compiler; a
change elsewhere in the kernel that shortened that side to two gave wrong scores
for the last stage of every query.  The first tests pin the checker on
hand-written code of each shape.
"""
from codeobj import disassemble
from wait_states import MFMA_WAITS, functions, short_waits

HEAD = "0000000000001000 <kern>:\n"


def code(*lines):
    """objdump-style text of one function from (instruction, branch target offset or None)."""
    out, addr = [HEAD], 0x1000
    for ins, tgt in lines:
        note = f" <kern+0x{tgt:x}>" if tgt is not None else ""
        out.append(f"\t{ins:56s} // {addr:012X}: 00000000{note}\n")
        addr += 8
    return "".join(out)


def test_checker_flags_an_mfma_result_read_through_a_branch():
    text = code(("v_mfma_f32_16x16x32_bf16 a[0:3], v[4:7], v[8:11], a[0:3]", None),
                ("s_cbranch_vccnz 2", 0x20),
                ("v_mov_b32_e32 v1, 0", None),
                ("s_nop 7", None),
                ("v_accvgpr_read_b32 v2, a3", None),
                ("s_endpgm", None))
    assert [f[0] for f in functions(text)] == ["kern"]
    found = short_waits(text)
    assert len(found) == 1
    name, rule, _, consumer, waits, need = found[0]
    assert (name, rule, waits, need) == ("kern", "mfma", 1, 8) and consumer.startswith("v_accvgpr_read_b32")
    padded = text.replace("s_cbranch_vccnz 2  ", "s_nop 6            ")
    assert short_waits(padded) == []


def test_checker_lets_accumulator_chains_through_and_flags_operand_reuse():
    chain = code(("v_mfma_f32_16x16x32_bf16 a[0:3], v[4:7], v[8:11], a[0:3]", None),
                 ("v_mfma_f32_16x16x32_bf16 a[0:3], v[12:15], v[8:11], a[0:3]", None),
                 ("s_nop 7", None),
                 ("v_accvgpr_read_b32 v2, a3", None),
                 ("s_endpgm", None))
    assert short_waits(chain) == []
    srcab = chain.replace("a[0:3], v[12:15], v[8:11], a[0:3]", "v[16:19], a[0:3], v[8:11], v[16:19]")
    assert [f[1] for f in short_waits(srcab)] == ["mfma"]


def test_checker_rules_for_vector_alu_producers():
    cases = [
        # (producer, consumer, rule, wait states needed)
        ("v_exp_f32_e32 v2, v1", "v_add_f32_e32 v3, v2, v1", "trans -> valu", 1),
        ("v_add_u32_e32 v1, 7, v1", "v_mov_b32_dpp v2, v1 row_shr:1 row_mask:0xf bank_mask:0xf", "valu -> dpp", 2),
        ("v_add_f32_e32 v1, v1, v1", "v_permlane32_swap_b32_e32 v1, v2", "valu -> permlane swap", 2),
        ("v_readfirstlane_b32 s0, v1", "v_mov_b32_e32 v0, s0", "readlane sgpr -> valu", 2),
        ("v_readfirstlane_b32 s4, v1", "v_readlane_b32 s5, v1, s4", "readlane sgpr -> lane select", 4),
    ]
    for prod, cons, rule, need in cases:
        bare = code((prod, None), (cons, None), ("s_endpgm", None))
        assert rule in [f[1] for f in short_waits(bare)], (prod, cons)
        nops = code((prod, None), (f"s_nop {need - 1}", None), (cons, None), ("s_endpgm", None))
        assert rule not in [f[1] for f in short_waits(nops)], (prod, cons)
    # a result overwritten in between is no longer the one read
    over = code(("v_exp_f32_e32 v2, v1", None), ("v_mov_b32_e32 v2, 0", None),
                ("v_add_f32_e32 v3, v2, v1", None), ("s_endpgm", None))
    assert short_waits(over, only="trans") == []


def test_every_result_waits_long_enough(tmp_path):
    texts = disassemble(tmp_path)
    n_mfma, found = 0, []
    for text in texts:
        for _, ins in functions(text):
            n_mfma += sum(1 for _, op, _, _ in ins if op in MFMA_WAITS)
        found += short_waits(text)
    assert n_mfma > 1000, "the attention kernels' MFMAs are missing from the disassembly"
    assert not found, f"{len(found)} short waits, e.g. {found[:3]}"
