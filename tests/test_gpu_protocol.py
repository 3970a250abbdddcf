"""GPU tests of the launch protocol: bounded waits, error reporting, argument
validation and role control.

Failure handling is forced from the host: a handle with a tiny spin limit and
no land workgroups leaves the ready flags unset, so every wait expires by its
own bound and the launch completes normally with MK_ERR_TIMEOUT recorded.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle as O
from communication_gemm_persistent_amd import inputs as I
from tests.gpu_util import bits, dev_bf16, empty_bf16

pytestmark = pytest.mark.gpu


def _ag_buffers(d, rank=0):
    W = len(d["shards"])
    m_s, k = d["shards"][0].shape
    n = d["b"].shape[1]
    shards = [dev_bf16(s) for s in d["shards"]]
    bt = dev_bf16(I.transpose_bits(d["b"]))
    return shards, bt, empty_bf16((W * m_s, n)), empty_bf16((W * m_s, k))


def test_withheld_chunks_time_out_and_handle_recovers(mk):
    d = I.gen_ag(4, 256, 256, 128, I.INTEGER, config=500)
    shards, bt, c, ag = _ag_buffers(d)
    with mk.Handle(0, spin_timeout_ms=50) as h:
        h.set_roles(mk.OP_AG_GEMM, n_land=0)          # nobody lands the peers' chunks
        h.ag_gemm(shards, bt, c, ag, rank=0, flags=mk.F_STATIC_ROLES)
        with pytest.raises(mk.MkError) as ei:
            h.sync()
        assert ei.value.status == mk.MK_ERR_TIMEOUT
        h.sync()                                      # the error record was cleared
        h.set_roles(mk.OP_AG_GEMM)                    # defaults again
        h.ag_gemm(shards, bt, c, ag, rank=0)
        h.sync()
        O.assert_bits_equal(bits(c), O.ag_gemm(d["shards"], d["b"])["c"], "after recovery")


@pytest.mark.parametrize("combine", [False, True])
def test_moe_withheld_unit_times_out_and_handle_recovers(mk, monkeypatch, combine):
    """A MoE land unit that never lands (MK_TEST_MOE_WITHHOLD, a test-only
    knob read when the handle is created) leaves its route item's flag unset:
    the wave that checks a tile's item flags gives up at the spin limit, so
    does the combine's wait for the last tile, and the launch completes with
    MK_ERR_TIMEOUT recorded.  A second call on the handle reports it again;
    a handle without the knob then computes the right result."""
    from tests.test_gpu_moe import check_moe, run_moe
    from tests.test_gpu_moe_combine import run_combine
    S, T, H, N, E, E_loc, top_k = 2, 256, 64, 64, 8, 8, 2
    print(f"moe withheld unit, combine={combine}", flush=True)
    d = I.gen_moe(S, T, H, N, E, E_loc, I.INTEGER, config=470)
    run = run_combine if combine else run_moe
    monkeypatch.setenv("MK_TEST_MOE_WITHHOLD", "1")   # route item 0, second token part
    with mk.Handle(0, spin_timeout_ms=50) as h:
        for _ in range(2):
            with pytest.raises(mk.MkError) as ei:
                run(h, d, E, top_k, rank=0)
            assert ei.value.status == mk.MK_ERR_TIMEOUT
            h.sync()                                  # the error record was cleared
    monkeypatch.delenv("MK_TEST_MOE_WITHHOLD")
    with mk.Handle(0) as h:
        out = run_moe(h, d, E, top_k, rank=0)
        check_moe(d, out, top_k, 0, I.INTEGER)


def test_invalid_arguments_launch_nothing(mk):
    d = I.gen_ag(2, 64, 64, 64, I.FLOAT, config=501)
    shards, bt, c, ag = _ag_buffers(d)
    with mk.Handle(0) as h:
        lib = h.lib

        def call(**kw):
            a = dict(world=2, rank=0, m_s=64, n=64, k=64, flags=0,
                     shards=[s.data_ptr() for s in shards], bt=bt.data_ptr(), c=c.data_ptr(),
                     ag=ag.data_ptr())
            a.update(kw)
            arr = (ctypes.c_void_p * len(a["shards"]))(*a["shards"])
            return lib.mk_ag_gemm(h.h, None, a["world"], a["rank"], arr, a["bt"], a["c"], a["ag"],
                                  a["m_s"], a["n"], a["k"], a["flags"])

        assert call() == mk.MK_OK
        h.sync()
        assert call(k=60) == mk.MK_ERR_INVALID            # K not a multiple of 8
        assert call(n=12) == mk.MK_ERR_INVALID            # N not a multiple of 8
        assert call(world=17) == mk.MK_ERR_INVALID
        assert call(rank=2) == mk.MK_ERR_INVALID
        assert call(flags=0x80) == mk.MK_ERR_INVALID
        assert call(bt=bt.data_ptr() + 2) == mk.MK_ERR_INVALID   # misaligned
        pageable = np.zeros(64 * 64, np.uint16)
        assert call(shards=[shards[0].data_ptr(), pageable.ctypes.data]) == mk.MK_ERR_INVALID
        assert call(ag=0) == mk.MK_ERR_INVALID
        assert b"a_gathered" in lib.mk_last_error(h.h)


def test_short_buffers_are_rejected_before_launch(mk):
    # A raw hipMalloc gives an allocation whose extent is exactly known: a
    # buffer that starts inside it but ends past it must be refused with
    # MK_ERR_INVALID, and one that fits exactly must be accepted.
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipMalloc.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_size_t]
    hip.hipFree.argtypes = [ctypes.c_void_p]
    d = I.gen_ag(2, 64, 64, 64, I.INTEGER, config=502)
    shards, bt, c, _ = _ag_buffers(d)
    need = 2 * 64 * 64 * 2                      # a_gathered: [W*m_s, k] bf16
    raw = ctypes.c_void_p()
    assert hip.hipMalloc(ctypes.byref(raw), need) == 0
    try:
        with mk.Handle(0) as h:
            lib = h.lib
            arr = (ctypes.c_void_p * 2)(*[s.data_ptr() for s in shards])

            def call(ag):
                return lib.mk_ag_gemm(h.h, None, 2, 0, arr, bt.data_ptr(), c.data_ptr(), ag,
                                      64, 64, 64, 0)

            assert call(raw.value + 4096) == mk.MK_ERR_INVALID
            assert b"a_gathered is smaller than its shape" in lib.mk_last_error(h.h)
            assert call(raw.value) == mk.MK_OK
            h.sync()
            O.assert_bits_equal(bits(c), O.ag_gemm(d["shards"], d["b"])["c"], "exact-size a_gathered")
    finally:
        torch.cuda.synchronize()
        assert hip.hipFree(raw) == 0


def test_dynamic_roles_land_without_land_workgroups(mk):
    """With the default dynamic roles, compute workgroups land missing chunks
    themselves, so even n_land = 0 completes."""
    d = I.gen_ag(4, 256, 256, 128, I.INTEGER, config=505)
    shards, bt, c, ag = _ag_buffers(d)
    with mk.Handle(0, spin_timeout_ms=2000) as h:
        h.set_roles(mk.OP_AG_GEMM, n_land=0, n_compute=5)
        h.ag_gemm(shards, bt, c, ag, rank=0)
        h.sync()
        ref = O.ag_gemm(d["shards"], d["b"])
        O.assert_bits_equal(bits(ag), ref["a_gathered"], "a_gathered")
        O.assert_bits_equal(bits(c), ref["c"], "C")


def test_static_roles_give_identical_bits(mk):
    d = I.gen_ag(4, 512, 512, 256, I.FLOAT, config=506)
    shards, bt, c, ag = _ag_buffers(d)
    with mk.Handle(0) as h:
        h.ag_gemm(shards, bt, c, ag, rank=0)
        h.sync()
        dyn = bits(c)
        h.ag_gemm(shards, bt, c, ag, rank=0, flags=mk.F_STATIC_ROLES)
        h.sync()
        O.assert_bits_equal(bits(c), dyn, "static vs dynamic roles")


def test_roles_query_and_transfer_only_launch(mk):
    d = I.gen_ag(4, 256, 256, 128, I.FLOAT, config=502)
    shards, bt, c, ag = _ag_buffers(d)
    with mk.Handle(0) as h:
        assert h.get_roles(mk.OP_AG_GEMM) == (-1, -1, -1)
        h.set_roles(mk.OP_AG_GEMM, n_land=6, n_compute=0)   # transfer alone
        h.ag_gemm(shards, bt, c, ag, rank=0)
        h.sync()
        roles, grid = h.last_launch(mk.OP_AG_GEMM)
        assert roles == (6, 0, 0) and grid == 6
        O.assert_bits_equal(bits(ag), O.all_gather(d["shards"]), "a_gathered with no compute")
        h.set_roles(mk.OP_AG_GEMM, n_land=3, n_compute=9)
        h.ag_gemm(shards, bt, c, ag, rank=0)
        h.sync()
        assert h.last_launch(mk.OP_AG_GEMM) == ((3, 9, 0), 12)


def test_moe_keeps_at_least_one_land_workgroup(mk):
    S, T, H, N, E, E_loc, top_k = 2, 64, 32, 32, 8, 2, 2
    d = I.gen_moe(S, T, H, N, E, E_loc, I.FLOAT, config=503)
    from tests.test_gpu_moe import check_moe, run_moe
    with mk.Handle(0, spin_timeout_ms=5000) as h:
        h.set_roles(mk.OP_MOE, n_land=0, n_compute=3)
        out = run_moe(h, d, E, top_k)
        assert h.last_launch(mk.OP_MOE)[0][:2] == (1, 3)
        check_moe(d, out, top_k, 0, I.FLOAT)


def test_two_handles_interleaved_on_one_stream(mk):
    d = I.gen_ag(3, 128, 128, 64, I.INTEGER, config=504)
    shards, bt, c1, ag1 = _ag_buffers(d)
    _, _, c2, ag2 = _ag_buffers(d)
    ref = O.ag_gemm(d["shards"], d["b"])["c"]
    with mk.Handle(0) as h1, mk.Handle(0) as h2:
        for _ in range(5):
            h1.ag_gemm(shards, bt, c1, ag1, rank=0)
            h2.ag_gemm(shards, bt, c2, ag2, rank=0)
        h1.sync()
        h2.sync()
    O.assert_bits_equal(bits(c1), ref, "handle 1")
    O.assert_bits_equal(bits(c2), ref, "handle 2")


def test_mfma_ceiling_loop_runs(mk):
    """The measurement aid launches, completes and reports its FLOP count."""
    import torch
    h = mk.Handle(0)
    try:
        sink = torch.full((256,), float("nan"), dtype=torch.float32, device="cuda")
        flop = h.mfma_ceiling(4, sink)
        h.sync()
        props = torch.cuda.get_device_properties(0)
        assert flop == 2.0 * props.multi_processor_count * 4 * 4 * 8 * 32768
        assert torch.isfinite(sink[: min(256, 2 * props.multi_processor_count)]).all()
    finally:
        h.close()
