"""GPU test of mk_ag_gemm_noalloc (AllGather+GEMM with no handle and no
allocation, its control memory in the library's per-device array), through
the C ABI: two calls in a row, the second with a smaller input, each
compared with mk_ag_gemm on the same inputs (bit for bit: the same kernels
and schedule) and with the oracle.  Runs alone in a fresh process or after
the other tests."""
import numpy as np
import pytest
import torch

import oracle as O
from communication_gemm_persistent_amd import inputs as I
from tests.gpu_util import bits, dev_bf16, empty_bf16

pytestmark = pytest.mark.gpu


def _buffers(d):
    W = len(d["shards"])
    m_s, k = d["shards"][0].shape
    n = d["b"].shape[1]
    shards = [dev_bf16(s) for s in d["shards"]]
    bt = dev_bf16(I.transpose_bits(d["b"]))
    return shards, bt, empty_bf16((W * m_s, n)), empty_bf16((W * m_s, k))


@pytest.mark.parametrize("variant", [I.INTEGER, I.FLOAT])
def test_noalloc_matches_the_handle_entry_point(mk, variant):
    cases = [("ag_gemm_w8_8192x3584x8192", None), ("ag_gemm_w4_512x256x256", None),
             (None, (3, 300, 200, 72))]          # the second and third calls are smaller
    status = torch.full((2,), -1, dtype=torch.int32, device="cuda")
    with mk.Handle(0, spin_timeout_ms=10000) as h:
        for name, shape in cases:
            if name is not None:
                d = I.gen_workload(name, variant)
            else:
                W, m_s, n, k = shape
                d = I.gen_ag(W, m_s, n, k, variant, config=600)
            rank = 1 if name is None else 0
            print(f"noalloc {name or shape} variant={variant}", flush=True)
            shards, bt, c, ag = _buffers(d)
            status.fill_(-1)
            mk.ag_gemm_noalloc(shards, bt, c, ag, rank=rank, status=status)
            torch.cuda.synchronize()
            assert status.cpu().tolist() == [0, 0], "status of the launch"
            c_na, ag_na = bits(c), bits(ag)
            shards2, bt2, c2, ag2 = _buffers(d)
            h.ag_gemm(shards2, bt2, c2, ag2, rank=rank)
            h.sync()
            O.assert_bits_equal(c_na, bits(c2), "C: noalloc vs mk_ag_gemm")
            O.assert_bits_equal(ag_na, bits(ag2), "a_gathered: noalloc vs mk_ag_gemm")
            ref = O.ag_gemm(d["shards"], d["b"])
            O.assert_bits_equal(ag_na, ref["a_gathered"], "a_gathered vs oracle")
            if variant == I.INTEGER:
                O.assert_bits_equal(c_na, ref["c"], "C vs oracle")
            else:
                O.assert_close_bf16(c_na, ref["c"], "C vs oracle")


def test_noalloc_repeated_calls_without_status(mk):
    """Back-to-back calls on one stream reuse the array (cleared by each call)."""
    d = I.gen_ag(4, 256, 264, 136, I.INTEGER, config=601)
    shards, bt, c, ag = _buffers(d)
    for _ in range(10):
        mk.ag_gemm_noalloc(shards, bt, c, ag, rank=2)
    torch.cuda.synchronize()
    O.assert_bits_equal(bits(c), O.ag_gemm(d["shards"], d["b"])["c"], "C after 10 calls")


def test_noalloc_rejects_bad_arguments(mk):
    """Argument errors are returned by the C entry point before anything runs."""
    import ctypes
    d = I.gen_ag(2, 64, 64, 64, I.INTEGER, config=602)
    shards, bt, c, ag = _buffers(d)
    lib = mk.load()
    arr = (ctypes.c_void_p * 2)(*[s.data_ptr() for s in shards])
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    args = lambda world, rank, m_s, flags: (stream, world, rank, arr, ctypes.c_void_p(bt.data_ptr()),
                                            ctypes.c_void_p(c.data_ptr()), ctypes.c_void_p(ag.data_ptr()),
                                            m_s, 64, 64, flags, None)
    assert lib.mk_ag_gemm_noalloc(*args(2, 2, 64, 0)) == mk.MK_ERR_INVALID      # rank >= world
    assert lib.mk_ag_gemm_noalloc(*args(2, 0, 0, 0)) == mk.MK_ERR_INVALID      # m_s < 1
    assert lib.mk_ag_gemm_noalloc(*args(2, 0, 64, 0x2)) == mk.MK_ERR_INVALID   # a flag it does not take
    assert lib.mk_ag_gemm_noalloc(*args(2, 0, 64, 0)) == mk.MK_OK
    torch.cuda.synchronize()
    O.assert_bits_equal(bits(c), O.ag_gemm(d["shards"], d["b"])["c"], "C")
