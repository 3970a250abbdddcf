"""CPU checks of the compiled kernels' structure (hipcc cross-compiles for gfx950).

Every workgroup-wide barrier must execute in control flow that all lanes
follow together; a barrier inside a loop whose exit is exec-masked deadlocks
the workgroup.  No global->LDS DMA (inline assembly, outside the compiler's
hazard checks) may read a descriptor SGPR that a VALU instruction wrote
fewer than 5 wait states before.  Each checker must also flag known-bad
input, so a silent checker cannot pass.
"""
import os
import shutil
import subprocess

import pytest

from tests.asm_barrier_check import check_file
from tests.asm_hazard_check import check_file as check_hazards

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "communication_gemm_persistent_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
         "-packed-fp32-ops", "-Wno-unused-command-line-argument", "--cuda-device-only", "-S"]

pytestmark = pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")


def _asm(src_dir, name, out_dir):
    out = os.path.join(out_dir, name + ".s")
    subprocess.run([HIPCC, *FLAGS, os.path.join(src_dir, name), "-o", out], check=True,
                   capture_output=True)
    return out


@pytest.mark.parametrize("name", ["mk_kernels.hip", "mk_moe.hip", "mk_attn.hip"])
def test_no_barrier_in_divergent_loop(tmp_path, name):
    bad = check_file(_asm(CSRC, name, str(tmp_path)))
    assert not bad, f"barriers inside divergent loops: {bad}"


def test_checker_flags_merged_single_thread_regions(tmp_path):
    """Negative control: without the barrier that separates the lane-0 arrival
    from the next lane-0 counter fetch, the compiler builds a divergent loop."""
    src = tmp_path / "src"
    src.mkdir()
    for f in os.listdir(CSRC):
        txt = open(os.path.join(CSRC, f)).read()
        (src / f).write_text(txt.replace('#include "../../include/mk.h"',
                                         f'#include "{ROOT}/include/mk.h"'))
    dev = (src / "mk_device.h").read_text()
    before = "__device__ __forceinline__ uint32_t next_index(uint32_t *ctr, uint32_t *lds_word) {\n  __syncthreads();\n"
    assert before in dev
    dev = dev.replace(before, before.replace("  __syncthreads();\n", ""))
    (src / "mk_device.h").write_text(dev)
    assert check_file(_asm(str(src), "mk_kernels.hip", str(tmp_path))), \
        "checker missed the known-bad variant"


@pytest.mark.parametrize("name", ["mk_kernels.hip", "mk_moe.hip", "mk_attn.hip"])
def test_no_sgpr_hazard_at_lds_dma(tmp_path, name):
    bad = check_hazards(_asm(CSRC, name, str(tmp_path)))
    assert not bad, f"LDS DMAs reading a VALU-written SGPR too early: {bad[:5]}"


_HAZARD_ASM = """_Z1kv:
\tv_readlane_b32 s0, v250, 33
\tv_readlane_b32 s3, v250, 36
{between}\tbuffer_load_dwordx4 v32, s[0:3], 0 offen lds
\ts_endpgm
.Lfunc_end0:
"""


@pytest.mark.parametrize("between,flagged", [
    ("", True),                                             # descriptor read right after v_readlane
    ("\ts_mov_b32 m0, s5\n\ts_add_i32 s6, s6, 1\n", True),  # 2 wait states are not 5
    ("\ts_nop 4\n", False),                                 # the DMA helpers' own wait states
    ("\ts_add_i32 s6, s6, 1\n" * 5, False),                  # 5 other instructions
])
def test_hazard_checker_on_known_sequences(tmp_path, between, flagged):
    """The checker itself: a VALU write of a descriptor SGPR fewer than 5 wait
    states before an LDS DMA is flagged, and only then."""
    f = tmp_path / "k.s"
    f.write_text(_HAZARD_ASM.format(between=between))
    assert bool(check_hazards(str(f))) == flagged


def test_hazard_checker_sees_scalar_offsets(tmp_path):
    """A DMA's scalar offset written by a VALU instruction (v_readfirstlane)
    right before it is the same hazard as a descriptor."""
    f = tmp_path / "k.s"
    f.write_text("_Z1kv:\n\tv_readfirstlane_b32 s7, v3\n"
                 "\tbuffer_load_dwordx4 v32, s[8:11], s7 offen lds\n\ts_endpgm\n.Lfunc_end0:\n")
    assert check_hazards(str(f))


def test_hazard_checker_follows_branches_and_m0(tmp_path):
    """A descriptor written by v_readlane at the end of a block that branches
    to the DMA's block (not its fall-through predecessor), and M0 written by
    a VALU instruction right before the DMA, are both flagged; padded
    versions are not."""
    branch = ("_Z1kv:\n\tv_readlane_b32 s0, v250, 33\n\ts_branch .LBB0_2\n.LBB0_1:\n"
              "\ts_add_i32 s6, s6, 1\n" * 1 + "{pad}.LBB0_2:\n"
              "\tbuffer_load_dwordx4 v32, s[0:3], 0 offen lds\n\ts_endpgm\n.Lfunc_end0:\n")
    f = tmp_path / "b.s"
    f.write_text(branch.format(pad=""))
    assert check_hazards(str(f)), "the branch source's v_readlane is 2 wait states away"
    f.write_text(branch.replace("\ts_branch .LBB0_2\n", "\ts_nop 4\n\ts_branch .LBB0_2\n").format(pad=""))
    assert not check_hazards(str(f))
    m0 = "_Z1kv:\n\tv_readfirstlane_b32 m0, v3\n{pad}\tbuffer_load_dwordx4 v32, s[8:11], 0 offen lds\n\ts_endpgm\n.Lfunc_end0:\n"
    f.write_text(m0.format(pad=""))
    assert check_hazards(str(f))
    f.write_text(m0.format(pad="\ts_nop 4\n"))
    assert not check_hazards(str(f))
    carry = ("_Z1kv:\n\tv_add_co_u32_e64 v1, s[8:9], v2, v3\n"
             "\tbuffer_load_dwordx4 v32, s[8:11], 0 offen lds\n\ts_endpgm\n.Lfunc_end0:\n")
    f.write_text(carry)
    assert check_hazards(str(f)), "a carry-out written into the descriptor"
