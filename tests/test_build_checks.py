"""The build's device-code checks, on synthetic disassembly (CPU only).

build.py disassembles the gfx950 code it has just compiled and refuses a
library in which, in a forward bias instance (these write M0 from inline
assembly without the compiler saving it), a value could live in M0 across
another instruction that touches M0, or one of those instances uses scratch.
These tests plant each violation in a small listing in llvm-objdump's format
and require the checker to report it, so that a clean build means something.
"""

from tiled_attention_forward_amd import build


def _listing(*instrs, name="kern"):
    lines = [f"0000000000001000 <{name}>:"]
    addr = 0x1000
    for ins in instrs:
        lines.append(f"\t{ins:<60}// {addr:012X}: BF800000")
        addr += 4
    return "\n".join(lines) + "\n"


LOAD = "buffer_load_dwordx4 v78, s[16:19], 0 offen lds"


def test_write_then_load_is_clean():
    lst = _listing("s_mov_b32 m0, s29", "s_nop 0", LOAD, "s_add_i32 m0, s29, 0x2000", LOAD,
                   "s_endpgm")
    assert build.m0_discipline_problems(lst) == []


def test_value_kept_across_an_asm_statement_is_caught():
    # compiler sets M0 for a load it issues later; an asm statement's own
    # write + load sits in between
    lst = _listing("s_mov_b32 m0, s3", "s_mov_b32 m0, s29", "s_nop 0", LOAD, LOAD, "s_endpgm")
    probs = build.m0_discipline_problems(lst)
    assert len(probs) == 1 and "without its own write" in probs[0]


def test_load_without_write_in_its_block_is_caught():
    lst = _listing("s_mov_b32 m0, s3", "s_cbranch_scc1 1", "v_add_f32 v1, v2, v3", LOAD,
                   "s_endpgm")
    assert len(build.m0_discipline_problems(lst)) == 1
    # the write before a branch target does not reach a load after it
    lst = _listing("s_mov_b32 m0, s3", "s_branch 0", LOAD, "s_endpgm")
    assert len(build.m0_discipline_problems(lst)) == 1


def test_rule_applies_to_the_inline_assembly_instances():
    # one M0 value kept for two loads: a violation in a bias instance (whose
    # asm writes M0 unseen by the compiler), the compiler's own business in
    # any other kernel
    body = ("s_mov_b32 m0, s3", LOAD, LOAD, "s_endpgm")
    asm_kernel = "_ZN2fa12_GLOBAL__N_113fa_fwd_kernelIDF16bLi128ELi64ELi1ELb1ELb1ELb0ELb0ELi1ELi0ELi1EEEvNS0_6ParamsE"
    other = "_ZN2fa12_GLOBAL__N_118fa_bwd_dkdv_kernelIDF16_Li256ELb0ELb0ELb0EEEvNS0_9BwdParamsE"
    assert len(build.m0_discipline_problems(_listing(*body, name=asm_kernel),
                                            only=build._ASM_INSTANCE)) == 1
    assert build.m0_discipline_problems(_listing(*body, name=other), only=build._ASM_INSTANCE) == []
    assert len(build.m0_discipline_problems(_listing(*body, name=other))) == 1


def test_read_by_name_is_caught():
    lst = _listing("s_mov_b32 m0, s3", "s_mov_b32 s5, m0", "s_endpgm")
    assert any("by name" in p for p in build.m0_discipline_problems(lst))


def test_other_implicit_readers_are_checked():
    for ins in ("s_sendmsg sendmsg(MSG_DEALLOC_VGPRS)", "v_movrels_b32 v0, v1",
                "global_load_lds_dwordx4 v[2:3], off"):
        assert len(build.m0_discipline_problems(_listing("v_nop", ins, "s_endpgm"))) == 1
        assert build.m0_discipline_problems(_listing("s_mov_b32 m0, 0", ins, "s_endpgm")) == []


def test_scratch_in_an_asm_instance_is_caught():
    bias = "_ZN2fa12_GLOBAL__N_113fa_fwd_kernelIDF16bLi128ELi64ELi1ELb1ELb1ELb0ELb0ELi1ELi0EEEvNS0_6ParamsE"
    nobias = "_ZN2fa12_GLOBAL__N_113fa_fwd_kernelIDF16bLi128ELi64ELi1ELb1ELb0ELb0ELb0ELi1ELi0EEEvNS0_6ParamsE"
    fp32 = "_ZN2fa12_GLOBAL__N_113fa_fwd_kernelIfLi64ELi64ELi1ELb1ELb1ELb0ELb0ELi1ELi0EEEvNS0_6ParamsE"

    def notes(name, size):
        return f"    .name:           {name}\n    .private_segment_fixed_size: {size}\n"

    assert build.asm_instance_scratch_problems(notes(bias, 0)) == []
    assert len(build.asm_instance_scratch_problems(notes(bias, 16))) == 1
    # instances without the asm loads may spill (fp32 stages through registers)
    assert build.asm_instance_scratch_problems(notes(nobias, 16) + notes(fp32, 12)) == []
