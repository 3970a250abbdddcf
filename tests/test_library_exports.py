"""CPU checks of the C-ABI boundary: the library loads without a GPU and
exports every entry point include/mk.h declares."""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mk.h")
LIB = os.path.join(ROOT, "communication_gemm_persistent_amd", "libmk.so")


def declared():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(mk_[a-z_]+)\s*\(", txt)))


def test_header_declares_the_entry_points():
    names = declared()
    for want in ("mk_create", "mk_destroy", "mk_ag_gemm", "mk_gemm_rs", "mk_gemm_ar",
                 "mk_moe_dispatch_gemm", "mk_moe_dispatch_gemm_combine", "mk_ring_attention", "mk_mfma_ceiling", "mk_sync", "mk_status_string"):
        assert want in names


@pytest.mark.skipif(not os.path.exists(LIB), reason="libmk.so not built (run __graft_entry__.build())")
def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\bT (mk_[a-z_]+)\b", out))
    missing = [n for n in declared() if n not in exported]
    assert not missing, f"declared but not exported: {missing}"


@pytest.mark.skipif(not os.path.exists(LIB), reason="libmk.so not built (run __graft_entry__.build())")
def test_library_loads_and_binding_matches_header():
    from communication_gemm_persistent_amd import mk
    lib = mk.load()
    for n in declared():
        assert hasattr(lib, n)
    assert set(mk.EXPORTS) == set(declared())
    assert lib.mk_status_string(mk.MK_ERR_TIMEOUT).decode().startswith("MK_ERR_TIMEOUT")


@pytest.mark.skipif(not os.path.exists(LIB), reason="libmk.so not built (run __graft_entry__.build())")
def test_create_rejects_bad_arguments_without_a_gpu():
    import ctypes
    from communication_gemm_persistent_amd import mk
    lib = mk.load()
    h = ctypes.c_void_p()
    assert lib.mk_create(ctypes.byref(h), None) == mk.MK_ERR_INVALID
    assert lib.mk_destroy(None) == mk.MK_ERR_INVALID
    assert lib.mk_sync(None, None) == mk.MK_ERR_INVALID
    assert lib.mk_ag_gemm(None, None, 1, 0, None, None, None, None, 1, 8, 8, 0) == mk.MK_ERR_INVALID
