"""GPU parity of AllGather+GEMM against the CPU oracle, through the C ABI."""
import os

import numpy as np
import pytest
import torch

import oracle as O
from communication_gemm_persistent_amd import inputs as I
from tests.gpu_util import bits, dev_bf16, empty_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def handle(mk):
    h = mk.Handle(0, spin_timeout_ms=10000)
    yield h
    h.close()


def run_ag(h, d, rank=0, where="hbm", flags=0, a_gathered=None):
    W = len(d["shards"])
    m_s, k = d["shards"][0].shape
    n = d["b"].shape[1]
    shards = [dev_bf16(s, "hbm" if q == rank else where) for q, s in enumerate(d["shards"])]
    bt = dev_bf16(I.transpose_bits(d["b"]))
    c = empty_bf16((W * m_s, n))
    ag = a_gathered if a_gathered is not None else empty_bf16((W * m_s, k))
    h.ag_gemm(shards, bt, c, ag, rank=rank, flags=flags)
    h.sync()
    return bits(c), bits(ag)


def check_full(d, c, ag, exact):
    ref = O.ag_gemm(d["shards"], d["b"])
    O.assert_bits_equal(ag, ref["a_gathered"], "a_gathered")
    if exact:
        O.assert_bits_equal(c, ref["c"], "C (integer inputs)")
    else:
        O.assert_close_bf16(c, ref["c"], "C")


@pytest.mark.parametrize("where", ["hbm", "host"])
@pytest.mark.parametrize("variant", [I.FLOAT, I.INTEGER])
def test_ag_gemm_w4_small_config(handle, where, variant):
    print(f"ag_gemm_w4_512x256x256 variant={variant} peers={where}", flush=True)
    d = I.gen_workload("ag_gemm_w4_512x256x256", variant)
    c, ag = run_ag(handle, d, rank=0, where=where)
    check_full(d, c, ag, exact=variant == I.INTEGER)


@pytest.mark.parametrize("shape", [(3, 1, 300, 200, 72), (2, 1, 1, 8, 8), (5, 4, 97, 136, 264),
                                   (1, 0, 130, 264, 64)])
@pytest.mark.parametrize("variant", [I.FLOAT, I.INTEGER])
def test_ag_gemm_ragged(handle, shape, variant):
    W, rank, m_s, n, k = shape
    print(f"ag ragged W={W} rank={rank} m_s={m_s} n={n} k={k} variant={variant}", flush=True)
    d = I.gen_ag(W, m_s, n, k, variant, config=200 + W)
    c, ag = run_ag(handle, d, rank=rank)
    check_full(d, c, ag, exact=variant == I.INTEGER)


@pytest.mark.parametrize("tile", ["256", "128"])
def test_ag_gemm_each_tile_shape(mk, tile):
    os.environ["MK_TILE"] = tile
    try:
        h = mk.Handle(0, spin_timeout_ms=10000)
    finally:
        del os.environ["MK_TILE"]
    try:
        for variant in (I.FLOAT, I.INTEGER):
            d = I.gen_ag(3, 290, 520, 200, variant, config=230)
            print(f"ag tile={tile} variant={variant}", flush=True)
            c, ag = run_ag(h, d, rank=2, where="host")
            check_full(d, c, ag, exact=variant == I.INTEGER)
    finally:
        h.close()


def test_ag_gemm_prelanded_equals_fused(handle, mk):
    """Fused (landing inside the kernel) and unfused (gathered A given) agree bit for bit."""
    d = I.gen_ag(4, 256, 512, 512, I.FLOAT, config=240)
    c_fused, ag = run_ag(handle, d, rank=1)
    pre = dev_bf16(O.all_gather(d["shards"]))
    c_pre, _ = run_ag(handle, d, rank=1, flags=mk.F_PRELANDED, a_gathered=pre)
    O.assert_bits_equal(c_fused, c_pre, "fused vs pre-landed")


def test_ag_gemm_role_counts_do_not_change_bits(handle, mk):
    d = I.gen_ag(4, 512, 512, 256, I.FLOAT, config=241)
    ref, _ = run_ag(handle, d, rank=0)
    for land, compute in [(1, 1), (3, 5), (64, 7), (2, 300)]:
        handle.set_roles(mk.OP_AG_GEMM, n_land=land, n_compute=compute)
        try:
            c, ag = run_ag(handle, d, rank=0)
            roles, grid = handle.last_launch(mk.OP_AG_GEMM)
            assert roles[:2] == (land, compute) and grid == land + compute
        finally:
            handle.set_roles(mk.OP_AG_GEMM)
        O.assert_bits_equal(c, ref, f"roles land={land} compute={compute}")


def test_ag_gemm_repeated_calls_reuse_flags(handle):
    """Epoch-valued flags and self-resetting counters: many calls in a row stay correct."""
    d = I.gen_ag(3, 128, 256, 128, I.INTEGER, config=242)
    W, (m_s, k), n = 3, d["shards"][0].shape, d["b"].shape[1]
    shards = [dev_bf16(s) for s in d["shards"]]
    bt = dev_bf16(I.transpose_bits(d["b"]))
    ref = O.ag_gemm(d["shards"], d["b"])["c"]
    c = empty_bf16((W * m_s, n))
    ag = empty_bf16((W * m_s, k))
    for _ in range(20):
        handle.ag_gemm(shards, bt, c, ag, rank=0)
    handle.sync()
    O.assert_bits_equal(bits(c), ref, "after 20 calls")


def _sample_rows(M, m_s, n_per_chunk=6, seed=0):
    g = np.random.default_rng(seed)
    rows = []
    for q in range(M // m_s):
        rows += [q * m_s, q * m_s + m_s - 1] + list(q * m_s + g.integers(0, m_s, n_per_chunk - 2))
    return np.array(sorted(set(rows)))


@pytest.mark.parametrize("variant", [I.FLOAT, I.INTEGER])
def test_ag_gemm_w8_full_size_sampled(handle, variant, mk):
    name = "ag_gemm_w8_8192x3584x8192"
    print(f"{name} variant={variant}", flush=True)
    d = I.gen_workload(name, variant)
    c, ag = run_ag(handle, d, rank=0)
    O.assert_bits_equal(ag, O.all_gather(d["shards"]), "a_gathered")
    assert not np.isnan(O.bf16_to_f64(c)).any(), "unwritten output elements"
    rows = _sample_rows(8192, 1024)
    ref = O.ag_gemm_rows(d["shards"], d["b"], rows)
    if variant == I.INTEGER:
        O.assert_bits_equal(c[rows], ref, "C rows (integer inputs)")
    else:
        O.assert_close_bf16(c[rows], ref, "C rows")
    if variant == I.FLOAT:
        # the same launch with A already gathered (GEMM alone) gives the same bits
        c_pre, _ = run_ag(handle, d, rank=0, flags=mk.F_PRELANDED, a_gathered=dev_bf16(ag))
        O.assert_bits_equal(c_pre, c, "fused vs pre-landed")


@pytest.mark.parametrize("shape", [(8, 1024, 512, 1024), (3, 300, 200, 72)])
def test_ag_gemm_new_data_in_the_same_buffers(handle, shape):
    """Consecutive calls on the same device buffers with different contents:
    no call may see data a previous call left in a cache."""
    W, m_s, n, k = shape
    shards = [torch.empty((m_s, k), dtype=torch.bfloat16, device="cuda") for _ in range(W)]
    bt = torch.empty((n, k), dtype=torch.bfloat16, device="cuda")
    c = empty_bf16((W * m_s, n))
    ag = empty_bf16((W * m_s, k))
    for call in range(4):
        d = I.gen_ag(W, m_s, n, k, I.INTEGER, config=250 + call)
        for q in range(W):
            shards[q].copy_(dev_bf16(d["shards"][q]))
        bt.copy_(dev_bf16(I.transpose_bits(d["b"])))
        handle.ag_gemm(shards, bt, c, ag, rank=call % W)
        handle.sync()
        ref = O.ag_gemm(d["shards"], d["b"])
        O.assert_bits_equal(bits(ag), ref["a_gathered"], f"a_gathered, call {call}")
        O.assert_bits_equal(bits(c), ref["c"], f"C, call {call}")
