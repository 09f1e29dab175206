"""The grouped-GEMM kernels end inline-asm blocks with MFMAs; the compiler
does not insert the wait states an MFMA result needs before its own next
instruction reads it. These tests pin the checker on hand-made assembly and
then require the real kernels to be free of such hazards."""
import os
import shutil

import pytest

from mixture_experts_layer_25_amd import asmcheck

SNIPPET = """
_Zkernel:
\t;;#ASMSTART
\tv_mfma_f32_32x32x16_bf16 a[0:15], v[2:5], v[6:9], a[0:15]
\t;;#ASMEND
\tv_accvgpr_read_b32 v10, a3
\t;;#ASMSTART
\tv_mfma_f32_32x32x16_bf16 a[16:31], v[2:5], v[6:9], a[16:31]
\ts_nop 7
\ts_nop 7
\ts_nop 7
\t;;#ASMEND
\tv_accvgpr_read_b32 v11, a17
\t;;#ASMSTART
\tv_mfma_f32_32x32x16_bf16 v[32:47], v[2:5], v[6:9], v[32:47]
\ts_waitcnt lgkmcnt(0)
\t;;#ASMEND
\tv_add_u32_e32 v50, 1, v51
\tscratch_store_dwordx4 off, v[44:47], off
\t;;#ASMSTART
\tv_mfma_scale_f32_32x32x64_f8f6f4 v[64:79], v[2:9], v[10:13], v[64:79], v14, v15 blgp:4
\tds_read_b32 v16, v17 offset:256
\ts_waitcnt lgkmcnt(0)
\t;;#ASMEND
\tv_mov_b32_e32 v80, v79
"""


def test_checker_flags_reads_right_after_mfma_blocks():
    found = asmcheck.find_hazards(SNIPPET)
    # block 1: a3 read at once; block 2: padded by 24 wait states, fine;
    # block 3: the spill of v[44:47] within the window; block 4: an LDS read
    # after the MFMA is no padding, and v79 is read right after the block
    assert len(found) == 3
    assert "a3" in found[0] and "v[44:47]" in found[1] and "v79" in found[2]


BRANCHES = """
_Zkernel:
	;;#ASMSTART
	v_mfma_f32_16x16x32_bf16 v[2:5], v[6:9], v[10:13], v[2:5]
	;;#ASMEND
	s_cbranch_scc1 .LBB0_2
	s_branch .LBB0_3
.LBB0_1:
	v_mov_b32_e32 v20, v2
.LBB0_2:
	v_mov_b32_e32 v21, v3
	s_endpgm
.LBB0_3:
	v_mov_b32_e32 v22, v4
	s_endpgm
	v_mov_b32_e32 v23, v5
"""


def test_checker_follows_branches():
    # both branch targets are executed after the block (v3 and v4 read); the
    # block skipped by the unconditional branch (v2) and code after an
    # s_endpgm (v5) are not
    found = asmcheck.find_hazards(BRANCHES)
    assert sorted(found) == ["_Zkernel: v_mov_b32_e32 v21, v3", "_Zkernel: v_mov_b32_e32 v22, v4"]


@pytest.mark.skipif(not os.path.exists(asmcheck.HIPCC) and shutil.which("hipcc") is None,
                    reason="hipcc not available")
@pytest.mark.parametrize("name", asmcheck.SOURCES)
def test_gemm_kernels_have_no_mfma_result_hazards(name):
    src = os.path.join(os.path.dirname(asmcheck.__file__), "csrc", name)
    asm = asmcheck.compile_to_asm(src)
    assert "v_mfma" in asm
    assert asmcheck.find_hazards(asm) == []
