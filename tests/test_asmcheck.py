"""Pins for the build-time LDS-DMA wait-state check (CPU only): small
listings in the compiler's assembly syntax with known answers."""

from exact_tiled_attention_16_amd import asmcheck

COPY = "\tbuffer_load_dwordx4 v209, s[8:11], 0 offen lds\n"


def _check(body):
    return asmcheck.check_text(body)


def test_five_wait_states_after_a_vector_write_pass():
    text = ("\tv_readfirstlane_b32 s8, v100\n"
            "\ts_and_b32 s9, s7, 0xffff\n\ts_mov_b32 s10, s41\n\ts_mov_b32 s11, 0x20000\n"
            "\ts_mov_b32 m0, s6\n\ts_nop 0\n" + COPY)
    assert _check(text) == []
    assert _check("\tv_readfirstlane_b32 s8, v100\n\ts_mov_b32 m0, s6\n\ts_nop 4\n" + COPY) == []


def test_vector_write_of_a_descriptor_sgpr_too_close_is_reported():
    text = "\tv_readfirstlane_b32 s8, v100\n\ts_mov_b32 m0, s6\n\ts_nop 0\n" + COPY
    p = _check(text)
    assert len(p) == 1 and "s[8]" in p[0] and "2 wait states" in p[0]
    # A spill restore by v_readlane counts as a vector ALU write too.
    p = _check("\tv_readlane_b32 s11, v254, 59\n\ts_nop 2\n" + COPY)
    assert len(p) == 1 and "s[11]" in p[0]


def test_a_later_scalar_write_hides_the_vector_write():
    text = ("\tv_readfirstlane_b32 s10, v98\n\ts_lshl_b32 s10, s10, 7\n"
            "\ts_mov_b32 m0, s2\n\ts_nop 0\n" + COPY)
    assert _check(text) == []


def test_m0_needs_one_wait_state():
    p = _check("\ts_mov_b32 m0, s6\n" + COPY)
    assert len(p) == 1 and "M0" in p[0]
    assert _check("\ts_mov_b32 m0, s6\n\ts_nop 0\n" + COPY) == []


def test_block_start_inside_the_window_is_reported():
    p = _check("\ts_nop 1\n.LBB3_24:\n\ts_nop 0\n" + COPY)
    assert len(p) == 1 and "block start" in p[0]
    assert _check(".LBB3_24:\n\ts_nop 4\n" + COPY) == []


def test_comments_and_directives_are_skipped_and_copies_counted():
    text = ("\t;;#ASMSTART\n\ts_nop 4\n" + COPY + "\t;;#ASMEND\n"
            "\t.p2align 2\n\ts_nop 0\n\tbuffer_load_dwordx4 v214, s[8:11], 0 offen lds\n"
            "\tbuffer_load_dwordx4 v1, s[4:7], 0 offen\n")
    assert asmcheck.copies(text) == 2
    assert _check(text) == []


_META = """amdhsa.kernels:
  - .agpr_count:     0
    .name:           _ZN2fa12_GLOBAL__N_110fwd_kernelILi128EEEvv
    .private_segment_fixed_size: {a}
    .vgpr_count:     242
  - .agpr_count:     0
    .name:           _ZN2fa12_GLOBAL__N_114bwd_kv3_kernelILi128EEEvv
    .private_segment_fixed_size: {b}
    .vgpr_count:     179
"""


def test_scratch_kernels_lists_only_kernels_with_a_private_segment():
    assert asmcheck.scratch_kernels(_META.format(a=0, b=0)) == []
    assert asmcheck.scratch_kernels(_META.format(a=388, b=0)) == [
        ("_ZN2fa12_GLOBAL__N_110fwd_kernelILi128EEEvv", 388)]
    assert [k for k, _ in asmcheck.scratch_kernels(_META.format(a=0, b=24))] == [
        "_ZN2fa12_GLOBAL__N_114bwd_kv3_kernelILi128EEEvv"]
