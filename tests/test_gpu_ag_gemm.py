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


@pytest.mark.parametrize("tile", ["256", "128", "224"])
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


@pytest.mark.parametrize("variant", [I.FLOAT, I.INTEGER])
def test_ag_gemm_w8_full_size(handle, variant, mk):
    """The headline workload: every element of C and of the gathered A."""
    name = "ag_gemm_w8_8192x3584x8192"
    print(f"{name} variant={variant}", flush=True)
    d = I.gen_workload(name, variant)
    c, ag = run_ag(handle, d, rank=0)
    check_full(d, c, ag, exact=variant == I.INTEGER)
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


# K >= 2048 with K a multiple of 64 cuts the shards into K-slabs that land
# separately: tiles start after their first slab and check later ones in the
# K loop.  Shapes cover 8 full slabs, a partial last slab (K = 2112: 6 slabs
# of 320 and one of 192), and tiles spanning two land blocks (m_s = 300).
def _handle_with_env(mk, **env):
    old = {k: os.environ.get(k) for k in env}
    os.environ.update({k: str(v) for k, v in env.items()})
    try:
        return mk.Handle(0, spin_timeout_ms=10000)
    finally:
        for k, v in old.items():
            if v is None:
                del os.environ[k]
            else:
                os.environ[k] = v


@pytest.fixture(scope="module", params=["256", "224"])
def handle256(mk, request):
    """Handle on an 8-wave tile (256x256 or 256x224) with K-slab landing,
    whose K loop checks later slabs, and the per-XCD strided tile order."""
    h = _handle_with_env(mk, MK_TILE=request.param, MK_NO_SLABS="0", MK_TILE_MAP="2")
    yield h
    h.close()


@pytest.mark.parametrize("shape", [(4, 1, 256, 512, 4096), (3, 2, 512, 264, 2112),
                                   (2, 0, 300, 520, 2048)])
@pytest.mark.parametrize("variant", [I.FLOAT, I.INTEGER])
@pytest.mark.parametrize("tile", ["256", "default"])
def test_ag_gemm_k_slabs(handle, handle256, shape, variant, tile):
    W, rank, m_s, n, k = shape
    print(f"ag k-slabs W={W} rank={rank} m_s={m_s} n={n} k={k} variant={variant} tile={tile}",
          flush=True)
    d = I.gen_ag(W, m_s, n, k, variant, config=260 + W)
    h = handle256 if tile == "256" else handle
    for where in ("hbm", "host"):
        c, ag = run_ag(h, d, rank=rank, where=where)
        check_full(d, c, ag, exact=variant == I.INTEGER)


@pytest.mark.parametrize("roles", [(1, 1), (1, 40), (4, 3), (32, 224)])
@pytest.mark.parametrize("static", [False, True])
def test_ag_gemm_k_slabs_roles(handle256, mk, roles, static):
    """Few land workgroups (tiles then wait for later slabs inside the K loop)
    and static roles give the same bits."""
    print(f"ag k-slab roles={roles} static={static}", flush=True)
    d = I.gen_ag(4, 512, 512, 4096, I.INTEGER, config=270)
    ref = O.ag_gemm(d["shards"], d["b"])
    handle256.set_roles(mk.OP_AG_GEMM, n_land=roles[0], n_compute=roles[1])
    try:
        c, ag = run_ag(handle256, d, rank=3, flags=mk.F_STATIC_ROLES if static else 0)
    finally:
        handle256.set_roles(mk.OP_AG_GEMM)
    O.assert_bits_equal(ag, ref["a_gathered"], "a_gathered")
    O.assert_bits_equal(c, ref["c"], f"C roles={roles} static={static}")


@pytest.mark.parametrize("knobs", [dict(MK_TILE_MAP="1"), dict(MK_TILE_MAP="2", MK_HELP_EVERY="1"),
                                   dict(MK_NO_SLABS="0", MK_ITEM_KIB="32", MK_HELP_EVERY="3"),
                                   dict(MK_HELP_EAGER="1", MK_TILE="224", MK_LAND_SPLIT="0"),
                                   dict(MK_HELP_EAGER="0", MK_HELP_EVERY="1", MK_ROLES="0"),
                                   dict(MK_LAND_SPLIT="1", MK_TILE="224", MK_ITEM_KIB="64"),
                                   dict(MK_TILE_MAP="3"),
                                   dict(MK_TILE_MAP="3", MK_NO_SLABS="0", MK_LAND_SPLIT="0")])
def test_ag_gemm_schedule_knobs(mk, knobs):
    """Tile orders, slab landing, item sizes and helper counts change only the
    schedule, never the bits."""
    print(f"ag knobs {knobs}", flush=True)
    h = _handle_with_env(mk, **knobs)
    try:
        for shape in [(4, 2, 512, 520, 4096), (8, 5, 256, 776, 2048)]:
            W, rank, m_s, n, k = shape
            d = I.gen_ag(W, m_s, n, k, I.INTEGER, config=280 + W)
            c, ag = run_ag(h, d, rank=rank)
            check_full(d, c, ag, exact=True)
    finally:
        h.close()


@pytest.mark.parametrize("tile_map", [None, "0", "2"])
def test_ag_gemm_split_landing_tile_orders(mk, tile_map):
    """Tile grids that fill whole rounds of the grid take the split landing
    schedule (no dedicated land workgroups); with the default rounds order,
    the global order and an XCD-strided order every tile is computed once and
    the bits match the oracle (exact and ragged shard heights)."""
    print(f"ag split landing tile_map={tile_map}", flush=True)
    h = _handle_with_env(mk, **({} if tile_map is None else dict(MK_TILE_MAP=tile_map)))
    try:
        for shape in [(4, 1, 1024, 3584, 2048), (8, 3, 1000, 3584, 1024)]:
            W, rank, m_s, n, k = shape
            d = I.gen_ag(W, m_s, n, k, I.INTEGER, config=290 + W)
            c, ag = run_ag(h, d, rank=rank)
            (n_land, n_compute, _), grid = h.last_launch(mk.OP_AG_GEMM)
            assert n_land == 0 and n_compute == grid, (n_land, n_compute, grid)
            check_full(d, c, ag, exact=True)
    finally:
        h.close()
