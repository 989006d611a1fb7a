"""Host-side check of the built library's gfx950 code (no GPU needed): every
instruction that touches an MFMA's result registers comes after the wait states
the matrix unit needs, on every control-flow path (see mfma_waits.py).

The decode kernel's score product once ended in a branch (the next stages'
index fetch) whose taken side read the accumulators four to six wait states
after the last MFMA, with no s_nop from the compiler; a change elsewhere in the
kernel that shortened that side to two gave wrong scores for the last stage of
every query.  The first two tests pin the checker on hand-written code of that
shape.
"""
from codeobj import disassemble
from mfma_waits import REQUIRED, functions, short_waits

SHORT = """
0000000000001000 <kern>:
	v_mfma_f32_16x16x32_bf16 a[0:3], v[4:7], v[8:11], a[0:3]  // 000000001000: D3B58000 04021104
	s_cbranch_vccnz 2                                         // 000000001008: BF870002 <kern+0x14>
	v_mov_b32_e32 v1, 0                                       // 00000000100C: 7E020280
	s_nop 7                                                   // 000000001010: BF800007
	v_accvgpr_read_b32 v2, a3                                 // 000000001014: D3D84002 18000103
	s_endpgm                                                  // 00000000101C: BF810000
"""


def test_checker_flags_a_read_reached_through_a_branch():
    assert [f[0] for f in functions(SHORT)] == ["kern"]
    found = short_waits(SHORT)
    assert len(found) == 1
    name, mfma, consumer, waits, need = found[0]
    assert name == "kern" and consumer.startswith("v_accvgpr_read_b32") and waits == 1 and need == 8


def test_checker_passes_enough_wait_states_and_accumulator_chains():
    padded = SHORT.replace("s_cbranch_vccnz 2 ", "s_nop 6           ")
    assert short_waits(padded) == []
    chain = """
0000000000002000 <chain>:
	v_mfma_f32_16x16x32_bf16 a[0:3], v[4:7], v[8:11], a[0:3]  // 000000002000: D3B58000 04021104
	v_mfma_f32_16x16x32_bf16 a[0:3], v[12:15], v[8:11], a[0:3] // 000000002008: D3B58000 0402110C
	s_nop 7                                                   // 000000002010: BF800007
	v_accvgpr_read_b32 v2, a3                                 // 000000002014: D3D84002 18000103
	s_endpgm                                                  // 00000000201C: BF810000
"""
    assert short_waits(chain) == []
    srcab = chain.replace("v[12:15], v[8:11], a[0:3] //", "a[0:3], v[8:11], v[16:19] //")
    assert len(short_waits(srcab)) == 1


def test_every_mfma_result_waits_long_enough(tmp_path):
    texts = disassemble(tmp_path)
    n_mfma, found = 0, []
    for text in texts:
        for _, ins in functions(text):
            n_mfma += sum(1 for _, op, _, _ in ins if op in REQUIRED)
        found += short_waits(text)
    assert n_mfma > 1000, "the attention kernels' MFMAs are missing from the disassembly"
    assert not found, f"{len(found)} short waits after MFMAs, e.g. {found[:3]}"
