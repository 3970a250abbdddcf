"""CPU checks of the compiled kernels' structure (hipcc cross-compiles for gfx950).

Every workgroup-wide barrier must execute in control flow that all lanes
follow together; a barrier inside a loop whose exit is exec-masked deadlocks
the workgroup.  The check also requires the checker to flag a known-bad
variant, so a silent checker cannot pass.
"""
import os
import shutil
import subprocess

import pytest

from tests.asm_barrier_check import check_file

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


@pytest.mark.parametrize("name", ["mk_kernels.hip", "mk_moe.hip"])
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
