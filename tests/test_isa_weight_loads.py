"""CPU-only: the GEMM kernels' untracked weight loads are never touched
before their wait, checked on the gfx950 assembly hipcc produces here."""
import os
import shutil
import subprocess

import pytest

from isa_check import find_hazards

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# A loop whose back edge copies a pending load destination: the form the
# check exists to reject.
_BAD = """_Z11gemm_kernelBAD:
.LBB0_1:
	s_waitcnt vmcnt(4) lgkmcnt(0)
	s_barrier
	global_load_dwordx4 v[146:149], v[10:11], off
	v_cvt_scalef32_pk_f16_fp8 v182, v130, 1.0
	v_mov_b64_e32 v[130:131], v[146:147]
	s_cbranch_scc0 .LBB0_1
	s_endpgm
"""
_GOOD = _BAD.replace("\tv_mov_b64_e32 v[130:131], v[146:147]\n", "")

# The loop's exit path reuses the registers of a final, discarded prefetch
# before the wait that retires it.
_BAD_EXIT = """_Z11gemm_kernelEXIT:
.LBB1_1:
	s_waitcnt vmcnt(1) lgkmcnt(0)
	global_load_dwordx4 v[6:9], v[6:7], off
	global_load_lds_dwordx4 v[26:27], off
	s_cbranch_scc1 .LBB1_1
	v_accvgpr_read_b32 v10, a3
	v_mov_b32_e32 v6, v10
	s_waitcnt vmcnt(0)
	global_store_dwordx4 v[4:5], v[6:9], off
	s_endpgm
"""
_GOOD_EXIT = _BAD_EXIT.replace("\tv_mov_b32_e32 v6, v10\n\ts_waitcnt vmcnt(0)\n",
                               "\ts_waitcnt vmcnt(0)\n\tv_mov_b32_e32 v6, v10\n")

# vmcnt(1) with only one younger load does not cover the load; vmcnt(0) does.
_LOOSE_WAIT = """_Z11gemm_kernelLOOSE:
	global_load_dwordx4 v[6:9], v[2:3], off
	global_load_dwordx2 v[10:11], v[2:3], off
	s_waitcnt vmcnt(1)
	v_add_u32_e32 v12, v6, v10
	s_endpgm
"""


def test_checker_flags_planted_hazards():
    n, hz = find_hazards(_BAD)
    assert n == 1 and len(hz) == 1
    assert find_hazards(_GOOD) == (1, [])
    assert len(find_hazards(_BAD_EXIT)[1]) == 1
    assert find_hazards(_GOOD_EXIT) == (1, [])
    assert len(find_hazards(_LOOSE_WAIT)[1]) == 1
    assert find_hazards(_LOOSE_WAIT.replace("vmcnt(1)", "vmcnt(0)")) == (1, [])


@pytest.mark.skipif(not shutil.which(HIPCC) and not os.path.exists(HIPCC), reason="hipcc not available")
def test_gemm_weight_loads_waited(tmp_path):
    out = tmp_path / "gemm.s"
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
                    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                    "-I", os.path.join(ROOT, "include"), "--cuda-device-only", "-S",
                    os.path.join(ROOT, "block_draft_verification_amd", "csrc", "gemm.hip"), "-o", str(out)],
                   check=True, capture_output=True)
    n, hz = find_hazards(out.read_text())
    assert n >= 10, "no gemm kernels found in the assembly"
    assert not hz, "\n".join(hz[:10])


@pytest.mark.skipif(not shutil.which(HIPCC) and not os.path.exists(HIPCC), reason="hipcc not available")
@pytest.mark.parametrize("src", ["attention.hip", "misc.hip"])
def test_kernels_make_no_calls(tmp_path, src):
    """Device code is fully inlined: no out-of-line calls, in particular to the
    device library's id functions, which the inliner leaves alone in a file
    built with a different IEEE mode (attention.hip's flags)."""
    import sys
    sys.path.insert(0, ROOT)
    import __graft_entry__ as g
    out = tmp_path / (src + ".s")
    subprocess.run([HIPCC, *g.FLAGS, *g.SOURCE_FLAGS.get(src, []), "-I", g.CSRC, "--cuda-device-only", "-S",
                    os.path.join(g.CSRC, src), "-o", str(out)], check=True, capture_output=True)
    asm = out.read_text()
    assert "s_endpgm" in asm
    assert "s_swappc" not in asm and "__ockl_" not in asm
