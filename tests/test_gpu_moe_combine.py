"""GPU parity of the fused MoE dispatch + grouped GEMM + combine against the
CPU oracle.

Dispatch outputs are checked as in the dispatch-only tests.  The returned rows
are pure data movement: ret[s] at every position the oracle's return map names
must hold the GPU's own y row bit for bit, and every other row of ret[s] must
be untouched.  The combined rows are compared with the oracle to the float
tolerance, and bit for bit on integer inputs with exact gates (all logits
equal, so every gate is 1/E).
"""
import numpy as np
import pytest
import torch

import oracle as O
from communication_gemm_persistent_amd import inputs as I
from tests.gpu_util import bits, dev_bf16, dev_f32, empty_bf16, np_i32

pytestmark = pytest.mark.gpu

NAN_BITS = 0x7FC0  # what empty_bf16 fills with


@pytest.fixture(scope="module")
def handle(mk):
    h = mk.Handle(0, spin_timeout_ms=10000)
    yield h
    h.close()


def run_combine(h, d, E, top_k, rank=0, where="hbm", flags=0):
    S = len(d["x"])
    T, H = d["x"][0].shape
    E_loc, _, N = d["w"].shape
    cap = S * T * min(top_k, E_loc)
    x = [dev_bf16(xx, "hbm" if s == rank else where) for s, xx in enumerate(d["x"])]
    lg = [dev_f32(l, "hbm" if s == rank else where) for s, l in enumerate(d["logits"])]
    wt = dev_bf16(I.transpose_bits(d["w"]))
    y = empty_bf16((cap, N))
    idx = torch.full((S * T, top_k), -7, dtype=torch.int32, device="cuda")
    gate = torch.zeros((S * T, top_k), dtype=torch.float32, device="cuda")
    slot_token = torch.full((cap,), -7, dtype=torch.int32, device="cuda")
    eoff = torch.full((E_loc + 1,), -7, dtype=torch.int32, device="cuda")
    coff = torch.full((E_loc, S + 1), -7, dtype=torch.int32, device="cuda")
    xs = empty_bf16((cap, H))
    y_peer = dev_bf16(np.ascontiguousarray(d["y_peer"]).reshape(T * top_k, N), where)
    ret = [None if s == rank else empty_bf16((T * top_k, N), where) for s in range(S)]
    out = empty_bf16((T, N))
    h.moe_dispatch_gemm_combine(x, lg, wt, E, top_k, y, idx, gate, slot_token, eoff, coff, xs,
                                y_peer, ret, out, rank=rank, flags=flags)
    h.sync()
    return dict(y=bits(y), idx=np_i32(idx), slot_token=np_i32(slot_token),
                expert_offsets=np_i32(eoff), chunk_offsets=np_i32(coff),
                ret=[None if r is None else bits(r) for r in ret], out=bits(out))


def check_routing(out, ref):
    O.assert_bits_equal(out["idx"], ref["idx"], "topk_idx")
    O.assert_bits_equal(out["expert_offsets"], ref["expert_offsets"], "expert_offsets")
    O.assert_bits_equal(out["chunk_offsets"], ref["chunk_offsets"], "chunk_offsets")
    n = int(ref["expert_offsets"][-1])
    O.assert_bits_equal(out["slot_token"][:n], ref["slot_token"], "slot_token")


def check_returns(out, pos, T, top_k, rank):
    """ret[s] holds the GPU's y row of every slot returning to s, bit for bit,
    at the oracle's return position; every other row is untouched."""
    per_src = T * top_k
    src = pos // per_src
    for s, r in enumerate(out["ret"]):
        if r is None:
            assert s == rank
            continue
        sel = np.nonzero(src == s)[0]
        rows = pos[sel] - s * per_src
        O.assert_bits_equal(r[rows], out["y"][sel], f"ret[{s}] (returned rows)")
        untouched = np.ones(per_src, dtype=bool)
        untouched[rows] = False
        assert (r[untouched] == NAN_BITS).all(), f"ret[{s}]: rows outside the return map written"


SMALL = [  # S, T, H, N, E, E_loc, top_k, rank (rank < S: source `rank` is this rank's tokens)
    (3, 300, 264, 136, 16, 4, 2, 1),
    (2, 256, 64, 64, 8, 8, 2, 0),
    (4, 100, 128, 264, 32, 2, 1, 3),
    (3, 513, 72, 80, 12, 3, 3, 2),
    (1, 40, 32, 16, 4, 1, 4, 0),
]


@pytest.mark.parametrize("cfg", SMALL)
@pytest.mark.parametrize("variant", [I.FLOAT, I.INTEGER])
def test_moe_combine_small(handle, cfg, variant):
    S, T, H, N, E, E_loc, top_k, rank = cfg
    print(f"moe combine S={S} T={T} H={H} N={N} E={E} E_loc={E_loc} top_k={top_k} "
          f"rank={rank} variant={variant}", flush=True)
    d = I.gen_moe(S, T, H, N, E, E_loc, variant, config=440 + S, top_k=top_k)
    out = run_combine(handle, d, E, top_k, rank=rank)
    ref = O.moe_combine(d["x"], d["logits"], d["w"], top_k, d["y_peer"], rank=rank)
    check_routing(out, ref)
    n = ref["n_slots"]
    O.assert_close_bf16(out["y"][:n], ref["y"], "y")
    check_returns(out, ref["return_pos"], T, top_k, rank)
    O.assert_close_bf16(out["out"], ref["out"], "out")


@pytest.mark.parametrize("rank", [0, 1])
def test_moe_combine_exact_gates_integer_bit_exact(handle, rank):
    """All logits equal: every token takes all E = 4 experts (lower id first)
    with gate exactly 1/4; integer rows keep every sum exact, so y, the
    returned rows and out match the oracle bit for bit."""
    S, T, H, N, E, E_loc, top_k = 2, 200, 64, 64, 4, 2, 4
    d = I.gen_moe(S, T, H, N, E, E_loc, I.INTEGER, config=450, top_k=top_k)
    for lg in d["logits"]:
        lg[:] = 0.0
    out = run_combine(handle, d, E, top_k, rank=rank)
    ref = O.moe_combine(d["x"], d["logits"], d["w"], top_k, d["y_peer"], rank=rank)
    check_routing(out, ref)
    n = ref["n_slots"]
    assert n == S * T * E_loc
    O.assert_bits_equal(out["y"][:n], ref["y"], "y (exact gates)")
    check_returns(out, ref["return_pos"], T, top_k, rank)
    for s in range(S):
        if s != rank:
            O.assert_bits_equal(out["ret"][s].reshape(T, top_k, N)[ref["ret_mask"][s]],
                                ref["ret"][s][ref["ret_mask"][s]], f"ret[{s}] vs oracle")
    O.assert_bits_equal(out["out"], ref["out"], "out (exact gates)")


def test_moe_combine_peers_in_host_memory(handle):
    """Peer tokens, logits, y_peer and the return buffers in pinned host memory."""
    S, T, H, N, E, E_loc, top_k = 3, 200, 64, 64, 16, 4, 2
    d = I.gen_moe(S, T, H, N, E, E_loc, I.FLOAT, config=460, top_k=top_k)
    out = run_combine(handle, d, E, top_k, rank=2, where="host")
    ref = O.moe_combine(d["x"], d["logits"], d["w"], top_k, d["y_peer"], rank=2)
    check_routing(out, ref)
    check_returns(out, ref["return_pos"], T, top_k, 2)
    O.assert_close_bf16(out["out"], ref["out"], "out")


def test_moe_combine_no_local_tokens(handle):
    """No token picks a local expert: no tiles, nothing returned, and out is
    the plain sum of the returned rows."""
    S, T, H, N, E, E_loc, top_k = 2, 64, 32, 32, 8, 2, 2
    d = I.gen_moe(S, T, H, N, E, E_loc, I.FLOAT, config=470, top_k=top_k)
    for lg in d["logits"]:
        lg[:, :E_loc] = -50.0
    out = run_combine(handle, d, E, top_k, rank=0)
    ref = O.moe_combine(d["x"], d["logits"], d["w"], top_k, d["y_peer"], rank=0)
    assert out["expert_offsets"].tolist() == [0] * (E_loc + 1)
    check_returns(out, ref["return_pos"], T, top_k, 0)
    O.assert_close_bf16(out["out"], ref["out"], "out")


def test_moe_combine_after_other_launches(handle):
    """Counters reset between launches: combine, dispatch only, combine again
    on a smaller problem; the last result is checked."""
    from tests.test_gpu_moe import run_moe
    big = I.gen_moe(3, 300, 128, 64, 16, 4, I.FLOAT, config=480)
    run_combine(handle, big, 16, 2, rank=0)
    run_moe(handle, big, 16, 2, rank=1)
    S, T, H, N, E, E_loc, top_k = 2, 130, 64, 72, 8, 2, 2
    d = I.gen_moe(S, T, H, N, E, E_loc, I.FLOAT, config=481, top_k=top_k)
    out = run_combine(handle, d, E, top_k, rank=1)
    ref = O.moe_combine(d["x"], d["logits"], d["w"], top_k, d["y_peer"], rank=1)
    check_routing(out, ref)
    check_returns(out, ref["return_pos"], T, top_k, 1)
    O.assert_close_bf16(out["out"], ref["out"], "out")


def test_moe_combine_rejects_no_gate(handle, mk):
    d = I.gen_moe(2, 32, 32, 32, 4, 2, I.FLOAT, config=490)
    with pytest.raises(mk.MkError) as e:
        run_combine(handle, d, 4, 2, rank=0, flags=mk.F_NO_GATE)
    assert "MK_F_NO_GATE" in str(e.value)


def test_moe_combine_rejects_rank_without_own_tokens(handle, mk):
    """The dispatch accepts rank >= n_src (rank only picks the local experts);
    the combine needs source `rank`'s tokens and refuses before launching."""
    d = I.gen_moe(2, 32, 32, 32, 8, 2, I.FLOAT, config=491)
    with pytest.raises(mk.MkError) as e:
        run_combine(handle, d, 8, 2, rank=2)
    assert "rank >= n_src" in str(e.value)


@pytest.mark.parametrize("variant", [I.FLOAT, I.INTEGER])
def test_moe_combine_full_size(handle, variant):
    """8 sources x 4096 tokens, H 4096, N 1536, 64 experts (8 local), top-2:
    every returned row against the GPU's y, and every row of y and of out
    against the oracle."""
    name = "moe_s8_t4096_h4096_n1536_e64"
    p = I.CONFIGS[name].params
    print(f"{name} combine variant={variant}", flush=True)
    d = I.gen_workload(name, variant)
    T, top_k, rank = p["T"], p["top_k"], p["rank"]
    out = run_combine(handle, d, p["E"], top_k, rank=rank)
    ref = O.moe_combine(d["x"], d["logits"], d["w"], top_k, d["y_peer"], rank=rank)
    check_routing(out, ref)
    check_returns(out, ref["return_pos"], T, top_k, rank)
    n = ref["n_slots"]
    O.assert_close_bf16(out["y"][:n], ref["y"], "y (every slot)")
    O.assert_close_bf16(out["out"], ref["out"], "out (every token)")
