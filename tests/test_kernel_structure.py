"""CPU checks of the compiled kernels' structure (hipcc cross-compiles for gfx950).

Every workgroup-wide barrier must execute in control flow that all lanes
follow together; a barrier inside a loop whose exit is exec-masked deadlocks
the workgroup.  No global->LDS DMA (inline assembly, outside the compiler's
hazard checks) may read a descriptor SGPR that a VALU instruction wrote
fewer than 5 wait states before.  No K loop (innermost MFMA loop) may move
spilled registers in its hot blocks.  Each checker must also flag known-bad
input, so a silent checker cannot pass.
"""
import os
import shutil
import subprocess

import pytest

from tests.asm_barrier_check import check_file
from tests.asm_hazard_check import check_file as check_hazards
from tests.asm_loop_check import mfma_loops, spill_counts

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


@pytest.fixture(scope="module")
def built(tmp_path_factory):
    """The library's sources compiled once per test session: name -> .s path."""
    d = str(tmp_path_factory.mktemp("asm"))
    return {n: _asm(CSRC, n, d) for n in ("mk_kernels.hip", "mk_moe.hip", "mk_attn.hip")}


@pytest.mark.parametrize("name", ["mk_kernels.hip", "mk_moe.hip", "mk_attn.hip"])
def test_no_barrier_in_divergent_loop(built, name):
    bad = check_file(built[name])
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
def test_no_sgpr_hazard_at_lds_dma(built, name):
    bad = check_hazards(built[name])
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


@pytest.mark.parametrize("name", ["mk_kernels.hip", "mk_moe.hip", "mk_attn.hip"])
def test_no_spill_traffic_in_k_loops(built, name):
    """A scratch access in a K loop's hot blocks costs a memory round trip
    every iteration (and its wait also waits for the DMAs in flight): none
    is allowed.  A scalar restored with v_readlane is one VALU instruction; a
    loop may have at most two (the slab-gated AllGather loop reloads its
    trip count), and asm_hazard_check keeps them away from the DMAs.  The
    error paths of the loop's bounded waits may spill."""
    loops = mfma_loops(built[name])
    assert loops, "no MFMA loop found"
    bad = [(f, n, sp[:3]) for f, n, sp in loops
           if any(x.startswith(("scratch_", "buffer_store_dword")) for x in sp) or len(sp) > 2]
    assert not bad, f"spill traffic in K loops: {bad[:4]}"


_LOOP_ASM = """_Z1kv:
.LBB0_1:
\tv_mfma_f32_32x32x16_bf16 v[0:15], v[16:19], v[20:23], v[0:15]
{hot}\ts_cbranch_scc0 .LBB0_3
.LBB0_2:
{cold}\ts_branch .LBB0_1
.LBB0_3:
\ts_cbranch_scc1 .LBB0_1
\ts_endpgm
.Lfunc_end0:
"""


@pytest.mark.parametrize("hot,cold,flagged", [
    ("", "", False),
    ("\tscratch_load_dword v30, off, off offset:4\n", "", True),
    ("\tv_readlane_b32 s12, v78, 37\n", "", True),
    ("", "\tscratch_load_dword v30, off, off offset:4\n", False),  # a block without MFMAs or DMAs
])
def test_loop_checker_on_known_loops(tmp_path, hot, cold, flagged):
    f = tmp_path / "k.s"
    f.write_text(_LOOP_ASM.format(hot=hot, cold=cold))
    loops = mfma_loops(str(f))
    assert loops and bool(any(sp for _, _, sp in loops)) == flagged


def test_spill_counts_bounded(built):
    """A regression guard on the register budget: the 8-wave tiles sit at the
    256-VGPR cap, and the few values they spill live outside the K loop
    (checked above); the GEMM-alone and transfer-alone AllGather variants
    spill nothing."""
    counts = {}
    for path in built.values():
        counts.update(spill_counts(path))
    assert len(counts) >= 10
    for k, (v, s_) in counts.items():
        assert v <= 32, (k, v)
        if "ag_gemm_kernel" in k and not k.endswith("Li0EEEvNS_8AgParamsE"):
            assert v == 0 and s_ == 0, (k, v, s_)
