"""The build's scan for registers of transposing LDS reads still in flight.

The tiled kernel issues these reads from inline assembly, so the compiler does
not wait for them; the build refuses code in which an instruction touches a
read's registers before a wait covers it.  LDS operations complete in order:
an lgkmcnt(N) wait covers a read followed by at least N later LDS operations.
"""
from tile_planned_generator_amd.build import scan_transposing_reads


def kernel(*lines):
    return "_ZN2dg1kE:\n" + "\n".join("\t" + l for l in lines) + "\n"


def test_use_before_any_wait_is_flagged():
    bad = scan_transposing_reads(kernel("ds_read_b64_tr_b16 v[10:11], v1 offset:0",
                                        "v_mfma_f32_16x16x32_f16 v[0:3], v[10:13], v[20:23], v[0:3]"))
    assert len(bad) == 1


def test_wait_with_enough_later_lds_operations_covers_the_read():
    asm = kernel("ds_read_b64_tr_b16 v[10:11], v1 offset:0",
                 "ds_read_b128 v[20:23], v2",
                 "ds_read_b128 v[24:27], v2 offset:1024",
                 "s_waitcnt lgkmcnt(2)",
                 "v_mfma_f32_16x16x32_f16 v[0:3], v[10:13], v[20:23], v[0:3]")
    assert scan_transposing_reads(asm) == []


def test_wait_with_too_few_later_lds_operations_does_not():
    asm = kernel("ds_read_b64_tr_b16 v[10:11], v1 offset:0",
                 "ds_read_b128 v[20:23], v2",
                 "s_waitcnt lgkmcnt(2)",
                 "v_and_b32_e32 v11, v11, v5")
    assert len(scan_transposing_reads(asm)) == 1


def test_scalar_loads_do_not_count_as_later_lds_operations():
    # a scalar load after the read raises the counter but is not an LDS operation
    asm = kernel("ds_read_b64_tr_b8 v[10:11], v1 offset:0",
                 "s_load_dwordx4 s[0:3], s[4:5], 0x0",
                 "s_waitcnt lgkmcnt(1)",
                 "v_and_b32_e32 v10, v10, v5")
    assert len(scan_transposing_reads(asm)) == 1


def test_full_wait_and_unrelated_registers():
    asm = kernel("ds_read_b64_tr_b16 v[10:11], v1 offset:0",
                 "v_add_u32_e32 v12, v13, v14",          # other registers: fine
                 "v_mov_b32_e32 v10, 0",                 # overwrites a pending destination
                 "s_waitcnt lgkmcnt(0)",
                 "v_and_b32_e32 v10, v10, v5")           # after the wait: fine
    bad = scan_transposing_reads(asm)
    assert len(bad) == 1 and "v_mov_b32" in bad[0]


def test_state_resets_per_kernel():
    asm = kernel("ds_read_b64_tr_b16 v[10:11], v1 offset:0") + kernel("v_and_b32_e32 v10, v10, v5")
    assert scan_transposing_reads(asm) == []
