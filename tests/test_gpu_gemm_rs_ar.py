"""GPU parity of GEMM+ReduceScatter and GEMM+AllReduce against the CPU oracle."""
import os

import numpy as np
import pytest
import torch

import oracle as O
from communication_gemm_persistent_amd import inputs as I
from tests.gpu_util import bits, dev_bf16, dev_f32, empty_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def handle(mk):
    h = mk.Handle(0, spin_timeout_ms=10000)
    yield h
    h.close()


# ---------------------------------------------------------------- ReduceScatter

def run_rs(h, d, rank, where="hbm", out_where="hbm"):
    W = len(d["peers"])
    m, k = d["a"].shape
    n = d["b"].shape[1]
    ms = m // W
    a = dev_bf16(d["a"])
    bt = dev_bf16(I.transpose_bits(d["b"]))
    peers = [None if p is None else dev_f32(p, where) for p in d["peers"]]
    c_own = empty_bf16((ms, n))
    outbox = [None if q == rank else empty_bf16((ms, n), out_where) for q in range(W)]
    h.gemm_rs(a, bt, peers, c_own, outbox, rank=rank)
    h.sync()
    return bits(c_own), [None if o is None else bits(o) for o in outbox]


def check_rs(d, rank, c_own, outbox, exact):
    ref = O.gemm_rs(d["a"], d["b"], d["peers"], rank=rank)
    cmp = O.assert_bits_equal if exact else O.assert_close_bf16
    cmp(c_own, ref["c_own"], "c_own")
    for q, o in enumerate(outbox):
        if q != rank:
            cmp(o, ref["outbox"][q], f"outbox[{q}]")


@pytest.mark.parametrize("shape", [(4, 0, 512, 256, 128), (3, 2, 450, 200, 72), (8, 5, 1024, 264, 96),
                                   (1, 0, 64, 8, 8), (2, 1, 2, 16, 520)])
@pytest.mark.parametrize("variant", [I.FLOAT, I.INTEGER])
def test_gemm_rs_shapes(handle, shape, variant):
    W, rank, m, n, k = shape
    print(f"gemm_rs W={W} rank={rank} m={m} n={n} k={k} variant={variant}", flush=True)
    d = I.gen_rs(W, m, n, k, rank=rank, variant=variant, config=300 + W)
    c_own, outbox = run_rs(handle, d, rank)
    check_rs(d, rank, c_own, outbox, exact=variant == I.INTEGER)


@pytest.mark.parametrize("where,out_where", [("host", "hbm"), ("hbm", "host"), ("host", "host")])
def test_gemm_rs_peers_in_host_memory(handle, where, out_where):
    d = I.gen_rs(4, 512, 256, 136, rank=1, variant=I.INTEGER, config=310)
    c_own, outbox = run_rs(handle, d, 1, where=where, out_where=out_where)
    check_rs(d, 1, c_own, outbox, exact=True)


def test_gemm_rs_w_rank_emulation_on_gpu(handle):
    """Run the GPU op as every rank, feeding each rank the others' outboxes as its
    peer partials: the concatenated own slices are bf16(sum_r A_r @ B_r)."""
    W, m, n, k = 4, 512, 256, 64
    A = [I.draw_bf16(1, 320, r, (m, k), "normal") for r in range(W)]
    B = [I.draw_bf16(1, 320, 10 + r, (k, n), "normal") for r in range(W)]
    zero = np.zeros((m // W, n), np.float32)
    outs = []
    for r in range(W):
        d = dict(a=A[r], b=B[r], peers=[None if q == r else zero for q in range(W)])
        outs.append(run_rs(handle, d, r)[1])
    slices = []
    for r in range(W):
        peers = [None if q == r else O.bf16_to_f64(outs[q][r]).astype(np.float32) for q in range(W)]
        slices.append(run_rs(handle, dict(a=A[r], b=B[r], peers=peers), r)[0])
    tot = sum(O.bf16_to_f64(A[r]).astype(np.int64) @ O.bf16_to_f64(B[r]).astype(np.int64)
              for r in range(W))
    assert np.abs(tot).max() <= 256          # every partial and sum is exact in bf16
    O.assert_bits_equal(np.concatenate(slices), O.f64_to_bf16(tot.astype(np.float64)),
                        "reduce-scatter slices vs the full sum")


@pytest.mark.parametrize("variant", [I.FLOAT, I.INTEGER])
def test_gemm_rs_w8_full_size(handle, variant):
    """Every element of c_own and of the 7 outboxes, each against its own
    whole-tensor rms."""
    name = "gemm_rs_w8_8192x8192x3584"
    print(f"{name} variant={variant}", flush=True)
    d = I.gen_workload(name, variant)
    c_own, outbox = run_rs(handle, d, 0)
    check_rs(d, 0, c_own, outbox, exact=variant == I.INTEGER)


# ---------------------------------------------------------------- AllReduce

def run_ar(h, d, rank, n_bcast, where="hbm", out_where="hbm"):
    W = len(d["peers"])
    m, k = d["a"].shape
    n = d["b"].shape[1]
    a = dev_bf16(d["a"])
    bt = dev_bf16(I.transpose_bits(d["b"]))
    peers = [None if p is None else dev_f32(p, where) for p in d["peers"]]
    c = empty_bf16((m, n))
    bc = [empty_bf16((m, n), out_where) for _ in range(n_bcast)]
    h.gemm_ar(a, bt, peers, c, bc, rank=rank)
    h.sync()
    return bits(c), [bits(b) for b in bc]


@pytest.mark.parametrize("shape", [(4, 0, 256, 512, 128, 3), (3, 1, 300, 200, 72, 2),
                                   (8, 7, 129, 264, 1024, 7), (1, 0, 8, 8, 8, 0), (2, 0, 520, 136, 40, 1)])
@pytest.mark.parametrize("variant", [I.FLOAT, I.INTEGER])
def test_gemm_ar_shapes(handle, shape, variant):
    W, rank, m, n, k, nb = shape
    print(f"gemm_ar W={W} rank={rank} m={m} n={n} k={k} n_bcast={nb} variant={variant}", flush=True)
    d = I.gen_ar(W, m, n, k, rank=rank, variant=variant, config=330 + W)
    c, bc = run_ar(handle, d, rank, nb)
    ref = O.gemm_ar(d["a"], d["b"], d["peers"], rank=rank, n_bcast=nb)
    if variant == I.INTEGER:
        O.assert_bits_equal(c, ref["c"], "c")
    else:
        O.assert_close_bf16(c, ref["c"], "c")
    for i, b in enumerate(bc):
        O.assert_bits_equal(b, c, f"bcast[{i}] vs c")


def test_gemm_ar_host_memory_peers_and_bcast(handle):
    d = I.gen_ar(4, 256, 256, 64, rank=2, variant=I.INTEGER, config=340)
    c, bc = run_ar(handle, d, 2, 3, where="host", out_where="host")
    O.assert_bits_equal(c, O.gemm_ar(d["a"], d["b"], d["peers"], rank=2)["c"], "c")
    for b in bc:
        O.assert_bits_equal(b, c, "bcast vs c")


def test_gemm_ar_equals_rs_then_gather(handle):
    """At small integer shapes AllReduce equals ReduceScatter followed by a gather."""
    W, m, n, k = 4, 256, 128, 64
    A = [I.draw_bf16(1, 345, r, (m, k), "normal") for r in range(W)]
    B = [I.draw_bf16(1, 345, 10 + r, (k, n), "normal") for r in range(W)]
    P = [O.bf16_to_f64(A[r]) @ O.bf16_to_f64(B[r]) for r in range(W)]
    for r in (0, 3):
        d_ar = dict(a=A[r], b=B[r], peers=[None if q == r else P[q].astype(np.float32)
                                           for q in range(W)])
        c, _ = run_ar(handle, d_ar, r, 0)
        slices = []
        for rr in range(W):
            ms = m // W
            d_rs = dict(a=A[rr], b=B[rr], peers=[None if q == rr else
                                                 P[q][rr * ms:(rr + 1) * ms].astype(np.float32)
                                                 for q in range(W)])
            slices.append(run_rs(handle, d_rs, rr)[0])
        O.assert_bits_equal(c, np.concatenate(slices), f"AR vs RS+gather (rank {r})")


@pytest.mark.parametrize("variant", [I.FLOAT, I.INTEGER])
def test_gemm_ar_w8_full_size(handle, variant):
    """Every element of c; every broadcast copy bit for bit."""
    name = "gemm_ar_w8_2048x8192x1024"
    print(f"{name} variant={variant}", flush=True)
    d = I.gen_workload(name, variant)
    c, bc = run_ar(handle, d, 0, 7)
    for i, b in enumerate(bc):
        O.assert_bits_equal(b, c, f"bcast[{i}] vs c")
    ref = O.gemm_ar(d["a"], d["b"], d["peers"], rank=0)["c"]
    if variant == I.INTEGER:
        O.assert_bits_equal(c, ref, "c (integer inputs)")
    else:
        O.assert_close_bf16(c, ref, "c")


@pytest.mark.parametrize("tile_map", ["1", "2", "3"])
def test_rs_ar_tile_orders(mk, tile_map):
    """The per-XCD tile orders hand out every tile exactly once (RS and AR at
    shapes with ragged tile grids)."""
    old = os.environ.get("MK_TILE_MAP")
    os.environ["MK_TILE_MAP"] = tile_map
    try:
        h = mk.Handle(0, spin_timeout_ms=10000)
    finally:
        if old is None:
            del os.environ["MK_TILE_MAP"]
        else:
            os.environ["MK_TILE_MAP"] = old
    try:
        for shape in [(8, 3, 2560, 776, 264), (3, 1, 1500, 520, 72)]:
            W, rank, m, n, k = shape
            print(f"rs tile_map={tile_map} {shape}", flush=True)
            d = I.gen_rs(W, m, n, k, rank=rank, variant=I.INTEGER, config=330 + W)
            c_own, outbox = run_rs(h, d, rank)
            check_rs(d, rank, c_own, outbox, exact=True)
            print(f"ar tile_map={tile_map} {shape}", flush=True)
            d = I.gen_ar(W, m, n, k, rank=rank, variant=I.INTEGER, config=340 + W)
            c, bc = run_ar(h, d, rank, 2)
            ref = O.gemm_ar(d["a"], d["b"], d["peers"], rank=rank, n_bcast=2)
            O.assert_bits_equal(c, ref["c"], "c")
            for i, b in enumerate(bc):
                O.assert_bits_equal(b, c, f"bcast[{i}] vs c")
    finally:
        h.close()


@pytest.mark.parametrize("tile", ["256", "128"])
def test_rs_ar_own_slice_pipelined_epilogue(mk, tile):
    """Slice heights that are tile multiples put every own-slice tile inside
    one slice, where the reduce epilogue loads the next row group's peer
    partials before storing the current one (7, 3 and 1 peers), with ragged
    N and K; the AllReduce takes the same epilogue for every tile."""
    old = os.environ.get("MK_TILE")
    os.environ["MK_TILE"] = tile
    try:
        h = mk.Handle(0, spin_timeout_ms=10000)
    finally:
        if old is None:
            del os.environ["MK_TILE"]
        else:
            os.environ["MK_TILE"] = old
    try:
        for shape in [(8, 3, 2048, 264, 72), (4, 1, 2048, 520, 200), (2, 1, 512, 136, 40)]:
            W, rank, m, n, k = shape
            print(f"rs/ar pipelined epilogue tile={tile} {shape}", flush=True)
            d = I.gen_rs(W, m, n, k, rank=rank, variant=I.INTEGER, config=360 + W)
            c_own, outbox = run_rs(h, d, rank)
            check_rs(d, rank, c_own, outbox, exact=True)
            d = I.gen_ar(W, m, n, k, rank=rank, variant=I.INTEGER, config=370 + W)
            c, bc = run_ar(h, d, rank, 3)
            ref = O.gemm_ar(d["a"], d["b"], d["peers"], rank=rank, n_bcast=3)
            O.assert_bits_equal(c, ref["c"], "c")
            for i, b in enumerate(bc):
                O.assert_bits_equal(b, c, f"bcast[{i}] vs c")
    finally:
        h.close()


# ---------------------------------------------------------------- reduce role

RED_SHAPES = [(8, 3, 2048, 520, 200), (4, 1, 1024, 264, 72), (3, 2, 1500, 776, 136), (2, 0, 512, 256, 64)]


@pytest.mark.parametrize("shape", RED_SHAPES)
@pytest.mark.parametrize("n_reduce", [1, 5, 64])
@pytest.mark.parametrize("static", [False, True])
def test_rs_reduce_role_integer_bit_exact(handle, mk, shape, n_reduce, static):
    """Reduce workgroups sum the peers' partials of the own slice into the
    workspace; the own tiles' epilogues add that sum.  Integer inputs: every
    output bit-exact, whatever the role split (slices of 1500 / 3 = 500 rows
    put own rows in tiles that straddle slices)."""
    W, rank, m, n, k = shape
    print(f"rs reduce role n_reduce={n_reduce} static={static} {shape}", flush=True)
    d = I.gen_rs(W, m, n, k, rank=rank, variant=I.INTEGER, config=380 + W)
    handle.set_roles(mk.OP_GEMM_RS, n_reduce=n_reduce)
    try:
        c_own, outbox = _run_rs_flags(handle, d, rank, mk.F_STATIC_ROLES if static else 0)
        (_, n_compute, nr), grid = handle.last_launch(mk.OP_GEMM_RS)
        assert nr == n_reduce and grid == n_reduce + n_compute
    finally:
        handle.set_roles(mk.OP_GEMM_RS)
    check_rs(d, rank, c_own, outbox, exact=True)


def _run_rs_flags(h, d, rank, flags):
    W = len(d["peers"])
    m, k = d["a"].shape
    n = d["b"].shape[1]
    ms = m // W
    a = dev_bf16(d["a"])
    bt = dev_bf16(I.transpose_bits(d["b"]))
    peers = [None if p is None else dev_f32(p) for p in d["peers"]]
    c_own = empty_bf16((ms, n))
    outbox = [None if q == rank else empty_bf16((ms, n)) for q in range(W)]
    h.gemm_rs(a, bt, peers, c_own, outbox, rank=rank, flags=flags)
    h.sync()
    return bits(c_own), [None if o is None else bits(o) for o in outbox]


def _run_ar_flags(h, d, rank, n_bcast, flags):
    m, k = d["a"].shape
    n = d["b"].shape[1]
    a = dev_bf16(d["a"])
    bt = dev_bf16(I.transpose_bits(d["b"]))
    peers = [None if p is None else dev_f32(p) for p in d["peers"]]
    c = empty_bf16((m, n))
    bc = [empty_bf16((m, n)) for _ in range(n_bcast)]
    h.gemm_ar(a, bt, peers, c, bc, rank=rank, flags=flags)
    h.sync()
    return bits(c), [bits(b) for b in bc]


@pytest.mark.parametrize("shape", RED_SHAPES)
@pytest.mark.parametrize("n_reduce", [1, 7, 300])
def test_ar_reduce_role_integer_bit_exact(handle, mk, shape, n_reduce):
    W, rank, m, n, k = shape
    print(f"ar reduce role n_reduce={n_reduce} {shape}", flush=True)
    d = I.gen_ar(W, m, n, k, rank=rank, variant=I.INTEGER, config=390 + W)
    handle.set_roles(mk.OP_GEMM_AR, n_reduce=n_reduce)
    try:
        c, bc = _run_ar_flags(handle, d, rank, 2, 0)
        assert handle.last_launch(mk.OP_GEMM_AR)[0][2] == n_reduce
    finally:
        handle.set_roles(mk.OP_GEMM_AR)
    O.assert_bits_equal(c, O.gemm_ar(d["a"], d["b"], d["peers"], rank=rank)["c"], "c")
    for i, b in enumerate(bc):
        O.assert_bits_equal(b, c, f"bcast[{i}] vs c")


def test_rs_reduce_role_full_size(handle, mk):
    """The full GEMM+ReduceScatter workload with 16 reduce workgroups: every
    element of c_own and of the outboxes within the float rule."""
    name = "gemm_rs_w8_8192x8192x3584"
    print(f"{name} reduce role", flush=True)
    d = I.gen_workload(name, I.FLOAT)
    handle.set_roles(mk.OP_GEMM_RS, n_reduce=16)
    try:
        c_own, outbox = _run_rs_flags(handle, d, 0, 0)
    finally:
        handle.set_roles(mk.OP_GEMM_RS)
    check_rs(d, 0, c_own, outbox, exact=False)


@pytest.mark.parametrize("shape", [(8, 3, 2048, 520, 200), (3, 2, 1500, 776, 136)])
def test_rs_ar_transfer_alone_moves_the_reduce_bytes(handle, mk, shape):
    """n_compute = 0: the reduce workgroups alone write bf16 of the peers' sum
    (the operation with A = 0) and zero outboxes; nothing is computed."""
    W, rank, m, n, k = shape
    print(f"rs/ar transfer alone {shape}", flush=True)
    for nr in (-1, 3):
        d = I.gen_rs(W, m, n, k, rank=rank, variant=I.INTEGER, config=395)
        handle.set_roles(mk.OP_GEMM_RS, n_compute=0, n_reduce=nr)
        try:
            c_own, outbox = _run_rs_flags(handle, d, rank, 0)
            (_, nc, got_nr), grid = handle.last_launch(mk.OP_GEMM_RS)
            assert nc == 0 and got_nr == grid and (nr < 0 or got_nr == nr)
        finally:
            handle.set_roles(mk.OP_GEMM_RS)
        ref = O.gemm_rs(np.zeros_like(d["a"]), d["b"], d["peers"], rank=rank)
        O.assert_bits_equal(c_own, ref["c_own"], "c_own = bf16(sum of peers)")
        for q in range(W):
            if q != rank:
                assert (outbox[q] == 0).all(), f"outbox[{q}] holds zeros"
        d = I.gen_ar(W, m, n, k, rank=rank, variant=I.INTEGER, config=396)
        handle.set_roles(mk.OP_GEMM_AR, n_compute=0, n_reduce=nr)
        try:
            c, bc = _run_ar_flags(handle, d, rank, 2, 0)
        finally:
            handle.set_roles(mk.OP_GEMM_AR)
        O.assert_bits_equal(c, O.gemm_ar(np.zeros_like(d["a"]), d["b"], d["peers"], rank=rank)["c"],
                            "c = bf16(sum of peers)")
        for b in bc:
            O.assert_bits_equal(b, c, "bcast vs c")


@pytest.mark.parametrize("variant", [I.FLOAT, I.INTEGER])
def test_rs_ar_compute_alone_leaves_out_the_peers(handle, mk, variant):
    """MK_F_NO_PEERS: the operation with every peer partial zero; the peer
    pointers are not read (None)."""
    W, rank, m, n, k = 4, 1, 1024, 264, 136
    d = I.gen_rs(W, m, n, k, rank=rank, variant=variant, config=397)
    zero = [None if p is None else np.zeros_like(p) for p in d["peers"]]
    ms = m // W
    a, bt = dev_bf16(d["a"]), dev_bf16(I.transpose_bits(d["b"]))
    c_own = empty_bf16((ms, n))
    outbox = [None if q == rank else empty_bf16((ms, n)) for q in range(W)]
    handle.gemm_rs(a, bt, [None] * W, c_own, outbox, rank=rank, flags=mk.F_NO_PEERS)
    handle.sync()
    d0 = dict(d, peers=zero)
    check_rs(d0, rank, bits(c_own), [None if o is None else bits(o) for o in outbox],
             exact=variant == I.INTEGER)
    da = I.gen_ar(W, m, n, k, rank=rank, variant=variant, config=398)
    c = empty_bf16((m, n))
    handle.gemm_ar(dev_bf16(da["a"]), dev_bf16(I.transpose_bits(da["b"])), [None] * W, c, [],
                   rank=rank, flags=mk.F_NO_PEERS)
    handle.sync()
    ref = O.gemm_ar(da["a"], da["b"], [None if p is None else np.zeros_like(p) for p in da["peers"]],
                    rank=rank)["c"]
    (O.assert_bits_equal if variant == I.INTEGER else O.assert_close_bf16)(bits(c), ref, "c")


def test_reduce_role_argument_checks(mk):
    """n_reduce only where a reduce role exists; a workspace too small for the
    reduce role is refused before launching (no call allocates)."""
    h = mk.Handle(0, spin_timeout_ms=10000, workspace_bytes=1 << 20)
    try:
        for op in (mk.OP_AG_GEMM, mk.OP_MOE, mk.OP_RING_ATTN):
            with pytest.raises(mk.MkError) as e:
                h.set_roles(op, n_reduce=2)
            assert e.value.status == mk.MK_ERR_INVALID
        d = I.gen_rs(8, 8192, 520, 64, rank=0, variant=I.INTEGER, config=399)  # own slice 1024 x 520 fp32 > 1 MiB
        h.set_roles(mk.OP_GEMM_RS, n_reduce=4)
        with pytest.raises(mk.MkError) as e:
            _run_rs_flags(h, d, 0, 0)
        assert e.value.status == mk.MK_ERR_INVALID and "workspace" in str(e.value)
        h.set_roles(mk.OP_GEMM_RS, n_reduce=4, n_compute=0)
        with pytest.raises(mk.MkError) as e:
            _run_rs_flags(h, d, 0, mk.F_NO_PEERS)
        assert e.value.status == mk.MK_ERR_INVALID
        h.set_roles(mk.OP_GEMM_RS)
        c_own, outbox = _run_rs_flags(h, d, 0, 0)      # without the reduce role: no workspace
        check_rs(d, 0, c_own, outbox, exact=True)
    finally:
        h.close()
