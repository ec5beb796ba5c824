"""The build's check of the expert GEMMs' untracked loads, on small synthetic
assembly listings: it must pass a weight load consumed by an MFMA after a wait
that lands it and an LDS read used after lgkmcnt(0), and catch each way the
invariant can break (a use -- the MFMA included -- before the wait, a wait whose
count leaves the load in flight, a copy, a spill, a reload into a pending
register, a path that skips the wait, a load still pending at the end)."""
import pytest

from combine_moe_route_topk_amd.isa_check import check_asm, check_kernel

LOAD = [";;#ASMSTART", "global_load_dwordx4 v[10:13], v[2:3], off", ";;#ASMEND"]
MFMA = ["v_mfma_i32_32x32x32_i8 v[20:35], v[40:43], v[10:13], v[20:35]"]
WAIT0 = ["s_waitcnt vmcnt(0)"]
END = ["s_endpgm"]


def bad(lines):
    return check_kernel("k", lines)


def test_consumed_by_mfma_after_its_wait_is_clean():
    assert bad(LOAD + ["v_add_u32_e32 v5, v6, v7"] + WAIT0 + MFMA + ["v_mov_b32_e32 v10, 0"] + END) == []
    assert bad(LOAD + ["v_add_u32_e32 v5, v6, v7"] + MFMA + END)  # no wait: the MFMA reads early


def test_wait_counts():
    """vmcnt(N) lands a load only with N vector-memory instructions issued after
    it; the DMA into LDS and stores count too."""
    LOAD2 = [";;#ASMSTART", "global_load_dwordx4 v[14:17], v[2:3], off offset:1024", ";;#ASMEND"]
    assert bad(LOAD + LOAD2 + ["s_waitcnt vmcnt(1)"] + MFMA + WAIT0 + END) == []
    assert bad(LOAD + ["s_waitcnt vmcnt(1)"] + MFMA + WAIT0 + END)
    assert bad(LOAD + LOAD2 + ["s_waitcnt vmcnt(2)"] + MFMA + WAIT0 + END)
    assert bad(LOAD + ["global_load_lds_dwordx4 v[4:5], off"] + ["s_waitcnt vmcnt(1)"] + MFMA
               + WAIT0 + END) == []
    assert bad(LOAD + ["global_store_dwordx4 v[4:5], v[50:53], off"] + ["s_waitcnt vmcnt(1)"] + MFMA
               + WAIT0 + END) == []
    # a join keeps the smaller count: the path without the second load decides
    lines = LOAD + ["s_cbranch_scc1 .LBB0_2"] + LOAD2 + [".LBB0_2:", "s_waitcnt vmcnt(1)"] + MFMA \
        + WAIT0 + END
    assert bad(lines)


def test_touch_before_consumption():
    assert bad(LOAD + ["v_add_u32_e32 v11, v6, v7"] + MFMA + END)
    assert bad(LOAD + ["v_mov_b32_e32 v50, v12"] + MFMA + END)          # a copy reads it early
    assert bad(LOAD + ["scratch_store_dword off, v13, s0"] + MFMA + END)  # a spill


def test_mfma_writing_a_pending_register():
    assert bad(LOAD + ["v_mfma_i32_32x32x32_i8 v[10:25], v[40:43], v[44:47], v[10:25]"] + END)


def test_reload_before_consumption_and_address_clobber():
    assert bad(LOAD + LOAD + MFMA + END)
    assert bad(LOAD + [";;#ASMSTART", "global_load_dwordx4 v[60:63], v[12:13], off", ";;#ASMEND"]
               + MFMA + ["v_mfma_i32_32x32x32_i8 v[20:35], v[40:43], v[60:63], v[20:35]"] + END)


def test_branch_that_skips_the_consumer():
    lines = LOAD + ["s_cbranch_scc1 .LBB0_2"] + MFMA + [".LBB0_2:", "v_mov_b32_e32 v10, 0"] + END
    assert bad(lines)


def test_pending_at_end_and_vmcnt_drain():
    assert bad(LOAD + END)
    assert bad(LOAD + ["s_waitcnt vmcnt(0)", "v_mov_b32_e32 v10, 0"] + END) == []


def test_indirect_control_flow_is_refused():
    assert bad(LOAD + ["s_setpc_b64 s[0:1]"] + MFMA + END)


def test_loop_carried_ring():
    # a two-buffer ring: each half of the loop waits for the older buffer with one
    # load in flight, consumes it and reloads it
    B = [";;#ASMSTART", "global_load_dwordx4 v[14:17], v[2:3], off offset:1024", ";;#ASMEND"]
    MB = ["v_mfma_i32_32x32x32_i8 v[20:35], v[40:43], v[14:17], v[20:35]"]
    ring = lambda n: LOAD + B + [".LBB0_1:", f"s_waitcnt vmcnt({n})"] + MFMA + LOAD \
        + [f"s_waitcnt vmcnt({n})"] + MB + B + ["s_cbranch_scc1 .LBB0_1"] + WAIT0 + END
    assert bad(ring(1)) == []
    assert bad(ring(2))  # two in flight: the consumed buffer may still be loading
    broken = LOAD + [".LBB0_1:", "v_mov_b32_e32 v10, 0"] + WAIT0 + MFMA + LOAD \
        + ["s_cbranch_scc1 .LBB0_1"] + WAIT0 + END
    assert bad(broken)


DS = [";;#ASMSTART", "ds_read_b128 v[40:43], v8", ";;#ASMEND"]
LGKM0 = ["s_waitcnt lgkmcnt(0)"]


def test_lds_read_used_after_lgkmcnt0_is_clean():
    assert bad(LOAD + DS + ["v_add_u32_e32 v5, v6, v7"] + LGKM0 + WAIT0 + MFMA + END) == []
    assert bad(DS + ["s_waitcnt vmcnt(0) lgkmcnt(0)", "v_mov_b32_e32 v50, v41"] + END) == []


def test_lds_read_touched_before_lgkmcnt0():
    assert bad(LOAD + DS + WAIT0 + MFMA + LGKM0 + END)                   # the MFMA reads it early
    assert bad(LOAD + DS + ["v_mov_b32_e32 v50, v41"] + LGKM0 + WAIT0 + MFMA + END)  # a planted copy
    assert bad(LOAD + DS + ["scratch_store_dwordx4 off, v[40:43], s0"] + LGKM0 + WAIT0 + MFMA + END)
    assert bad(LOAD + DS + ["s_waitcnt lgkmcnt(1)", "v_mov_b32_e32 v50, v41"] + LGKM0 + WAIT0 + MFMA
               + END)


def test_lds_read_reload_and_address_clobber():
    assert bad(DS + DS + LGKM0 + END)
    assert bad(DS + [";;#ASMSTART", "ds_read_b128 v[60:63], v41", ";;#ASMEND"] + LGKM0 + END)
    assert bad(LOAD + [";;#ASMSTART", "ds_read_b128 v[60:63], v11", ";;#ASMEND"] + LGKM0 + WAIT0 + MFMA
               + END)


def test_lds_read_on_a_path_that_skips_the_wait():
    lines = DS + ["s_cbranch_scc1 .LBB0_2"] + LGKM0 + [".LBB0_2:", "v_mov_b32_e32 v50, v40"] + END
    assert bad(lines)
    assert bad(DS + END)


@pytest.mark.parametrize("src,loads,reads", [("ffn_q8.hip", 6 * 16, 6 * 8), ("router.hip", 0, 20)])
def test_the_built_kernels_have_loads_to_check(src, loads, reads, tmp_path):
    """The real GEMMs, compiled to assembly: the untracked loads are there, and no
    violation (the expert GEMMs: six variants with weight loads and LDS fragment
    reads; the gate GEMM: LDS fragment reads)."""
    import os
    import subprocess
    from combine_moe_route_topk_amd import build as B
    from combine_moe_route_topk_amd.isa_check import check_asm
    if not os.path.exists(B.HIPCC):
        pytest.skip("needs hipcc")
    asm = str(tmp_path / "k.s")
    flags = [f for f in B.FLAGS if f not in ("-shared", "-fPIC")]
    subprocess.run([B.HIPCC, *flags, "--cuda-device-only", "-S", "-o", asm,
                    os.path.join(B.PKG, "csrc", src), "-I", os.path.join(B.ROOT, "include")],
                   check=True, capture_output=True)
    text = open(asm).read()
    assert text.count("global_load_dwordx4") >= loads
    assert text.count("ds_read_b128") >= reads
    assert check_asm(asm) == []


def test_listing_without_inline_markers_is_refused(tmp_path):
    """A kernel whose loads the check cannot see as inline assembly (no
    ;;#ASMSTART markers) must fail, not pass without tracking anything; the same
    kernel with the markers passes."""
    name = "_Z15ffn_gemm_kernelv"
    def listing(body):
        p = tmp_path / "k.s"
        p.write_text("\n".join([f"{name}:"] + body + [".Lfunc_end0:"]) + "\n")
        return str(p)
    plain = [l for l in LOAD if not l.startswith(";;#")]
    assert check_asm(listing(plain + WAIT0 + MFMA + END))
    assert check_asm(listing(LOAD + WAIT0 + MFMA + END)) == []


def test_a_planted_short_wait_in_the_expert_gemm_is_refused(tmp_path):
    """The real expert GEMM with its per-step wait loosened from vmcnt(6) to
    vmcnt(9) (the weight loads of the step could still be in flight at the MFMAs):
    the check must refuse the build."""
    import os
    import shutil
    import subprocess
    from combine_moe_route_topk_amd import build as B
    if not os.path.exists(B.HIPCC):
        pytest.skip("needs hipcc")
    src = open(os.path.join(B.PKG, "csrc", "ffn_q8.hip")).read()
    wait6 = "__builtin_amdgcn_s_waitcnt(0x0F76);  // vmcnt(6)"
    assert src.count(wait6) == 1
    for h in ("common.h", "sizes.h"):
        shutil.copy(os.path.join(B.PKG, "csrc", h), tmp_path / h)
    (tmp_path / "ffn_q8.hip").write_text(
        src.replace(wait6, "__builtin_amdgcn_s_waitcnt(0x0F79);  // vmcnt(9)"))
    asm = str(tmp_path / "k.s")
    flags = [f for f in B.FLAGS if f not in ("-shared", "-fPIC")]
    subprocess.run([B.HIPCC, *flags, "--cuda-device-only", "-S", "-o", asm,
                    str(tmp_path / "ffn_q8.hip"), "-I", os.path.join(B.ROOT, "include")],
                   check=True, capture_output=True)
    found = check_asm(asm)
    assert found and all("has landed" in f for f in found), found[:3]

