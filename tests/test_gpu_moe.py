"""GPU parity of MoE dispatch + grouped GEMM against the CPU oracle.

Routing (top-k ids), the slot permutation (slot_token), expert and chunk
offsets and the landed rows are compared bit for bit; gates to 1e-5 relative
(fp32 softmax against the float64 oracle); expert outputs with the float
tolerance, and bit for bit when the gate is not applied on integer inputs.
"""
import numpy as np
import pytest
import torch

import oracle as O
from communication_gemm_persistent_amd import inputs as I
from tests.gpu_util import bits, dev_bf16, dev_f32, empty_bf16, np_i32

pytestmark = pytest.mark.gpu

@pytest.fixture(scope="module")
def handle(mk):
    h = mk.Handle(0, spin_timeout_ms=10000)
    yield h
    h.close()


def run_moe(h, d, E, top_k, rank=0, where="hbm", flags=0):
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
    h.moe_dispatch_gemm(x, lg, wt, E, top_k, y, idx, gate, slot_token, eoff, coff, xs,
                        rank=rank, flags=flags)
    h.sync()
    return dict(y=bits(y), idx=np_i32(idx), gate=np_i32(gate), slot_token=np_i32(slot_token),
                expert_offsets=np_i32(eoff), chunk_offsets=np_i32(coff), x_slots=bits(xs))


def check_moe(d, out, top_k, rank, variant, no_gate=False):
    """Every output against the oracle: routing, offsets, slot order and landed
    rows bit for bit; gates by the gate rule; y over all n_slots rows by the
    float rule, and bit for bit on integer inputs (ungated, or gated with the
    kernel's own fp32 gates, which are themselves checked by the gate rule)."""
    S, T = len(d["x"]), d["x"][0].shape[0]
    E_loc = d["w"].shape[0]
    ref = O.moe_dispatch_gemm(d["x"], d["logits"], d["w"], top_k=top_k, rank=rank,
                              apply_gate=not no_gate)
    n = ref["n_slots"]
    O.assert_bits_equal(out["idx"], ref["idx"], "topk_idx")
    O.assert_gates_close(out["gate"], ref["gate"], "topk_gate")
    O.assert_bits_equal(out["expert_offsets"], ref["expert_offsets"], "expert_offsets")
    O.assert_bits_equal(out["chunk_offsets"], ref["chunk_offsets"], "chunk_offsets")
    O.assert_bits_equal(out["slot_token"][:n], ref["slot_token"], "slot_token")
    O.assert_bits_equal(out["x_slots"][:n], ref["x_slots"], "x_slots")
    y = out["y"][:n]
    if variant == I.INTEGER:
        if no_gate:
            O.assert_bits_equal(y, ref["y"], "y (integer inputs, no gate)")
        else:
            pos = O.moe_return_positions(ref["slot_token"], ref["idx"], ref["expert_offsets"], T,
                                         top_k, E_loc, rank)
            g = np.asarray(out["gate"], dtype=np.float32).reshape(-1)[pos]
            O.assert_bits_equal(y, O.moe_y_given_gates(ref["x_slots"], d["w"],
                                                       ref["expert_offsets"], g),
                                "y (integer inputs, the kernel's fp32 gates)")
    O.assert_close_bf16(y, ref["y"], "y")
    return ref


SMALL = [  # S, T, H, N, E, E_loc, top_k, rank
    (3, 300, 264, 136, 16, 4, 2, 1),
    (2, 256, 64, 64, 8, 8, 2, 0),
    (4, 100, 128, 264, 32, 2, 1, 3),
    (2, 513, 72, 80, 12, 3, 3, 2),
    (1, 40, 32, 16, 4, 1, 4, 0),
]


@pytest.mark.parametrize("cfg", SMALL)
@pytest.mark.parametrize("variant", [I.FLOAT, I.INTEGER])
def test_moe_small(handle, cfg, variant):
    S, T, H, N, E, E_loc, top_k, rank = cfg
    print(f"moe S={S} T={T} H={H} N={N} E={E} E_loc={E_loc} top_k={top_k} rank={rank} "
          f"variant={variant}", flush=True)
    d = I.gen_moe(S, T, H, N, E, E_loc, variant, config=400 + S)
    out = run_moe(handle, d, E, top_k, rank=rank)
    check_moe(d, out, top_k, rank, variant)


@pytest.mark.parametrize("cfg", SMALL[:3])
def test_moe_no_gate_integer_bit_exact(handle, mk, cfg):
    S, T, H, N, E, E_loc, top_k, rank = cfg
    d = I.gen_moe(S, T, H, N, E, E_loc, I.INTEGER, config=410 + S)
    out = run_moe(handle, d, E, top_k, rank=rank, flags=mk.F_NO_GATE)
    check_moe(d, out, top_k, rank, I.INTEGER, no_gate=True)


def test_moe_ties_and_peers_in_host_memory(handle):
    S, T, H, N, E, E_loc, top_k = 3, 200, 64, 64, 16, 4, 2
    d = I.gen_moe(S, T, H, N, E, E_loc, I.FLOAT, config=420)
    for s in range(S):                      # forced ties at the top and among local experts
        lg = d["logits"][s]
        lg[::3, 1] = lg[::3, 2] = lg[::3].max(axis=1) + 1.0
        lg[1::5, :] = 0.5
    out = run_moe(handle, d, E, top_k, rank=0, where="host")
    check_moe(d, out, top_k, 0, I.FLOAT)


@pytest.mark.parametrize("top_k", [2, 3])
def test_moe_e64_routing_with_ties(handle, top_k):
    """E = 64 routes from vector loads of each token's logits (top-2 by a
    two-slot selection); forced ties keep the lower expert id first."""
    S, T, H, N, E, E_loc = 2, 300, 64, 64, 64, 8
    print(f"moe E=64 top_k={top_k} with ties", flush=True)
    d = I.gen_moe(S, T, H, N, E, E_loc, I.FLOAT, config=440 + top_k)
    for s in range(S):
        lg = d["logits"][s]
        lg[::3, 5] = lg[::3, 6] = lg[::3].max(axis=1) + 1.0   # tie at the top (local experts)
        lg[1::4, 40] = lg[1::4, 3] = lg[1::4].max(axis=1) + 2.0  # tie across the local boundary
        lg[2::7, :] = 0.25                                      # all equal
    out = run_moe(handle, d, E, top_k, rank=0)
    check_moe(d, out, top_k, 0, I.FLOAT)


@pytest.mark.parametrize("variant", [I.FLOAT, I.INTEGER])
def test_moe_e64_top2_pair_routing_with_ties(mk, monkeypatch, variant):
    """E = 64, top-2 on the 256-row kernel (MK_TILE=256 forces it at this
    size) routes each token with two lanes whose top-2 lists merge; forced
    ties at the top, across the two lanes' halves of the logits (experts 31
    and 32) and among all 64 experts keep the lower expert id first."""
    S, T, H, N, E, E_loc, top_k = 2, 700, 64, 64, 64, 8, 2
    print(f"moe pair routing with ties, variant={variant}", flush=True)
    d = I.gen_moe(S, T, H, N, E, E_loc, variant, config=445)
    for s in range(S):
        lg = d["logits"][s]
        top = lg.max(axis=1)
        lg[::3, 5] = lg[::3, 6] = top[::3] + 1.0      # tie at the top, one lane
        lg[1::4, 31] = lg[1::4, 32] = top[1::4] + 2.0  # tie across the lanes' halves
        lg[2::5, 40] = lg[2::5, 3] = top[2::5] + 1.5   # tie, higher id in the other lane
        lg[3::7, :] = 0.25                              # all equal
    monkeypatch.setenv("MK_TILE", "256")
    with mk.Handle(0, spin_timeout_ms=10000) as h:
        out = run_moe(h, d, E, top_k, rank=0)
    check_moe(d, out, top_k, 0, variant)


@pytest.mark.parametrize("roles,static", [((1, -1), False), ((1, 3), False), ((4, 60), False),
                                          ((4, 60), True), ((1, 3), True)])
def test_moe_role_splits_bit_identical(handle, mk, roles, static):
    """Every workgroup lands, then takes tiles (land workgroups too, unless
    the roles are static); every split of the roles gives the same bits."""
    S, T, H, N, E, E_loc, top_k = 4, 700, 128, 136, 64, 8, 2
    print(f"moe role split {roles} static {static}", flush=True)
    d = I.gen_moe(S, T, H, N, E, E_loc, I.INTEGER, config=450)
    ref = run_moe(handle, d, E, top_k, rank=1)
    check_moe(d, ref, top_k, 1, I.INTEGER)
    handle.set_roles(mk.OP_MOE, n_land=roles[0], n_compute=roles[1])
    try:
        out = run_moe(handle, d, E, top_k, rank=1, flags=mk.F_STATIC_ROLES if static else 0)
    finally:
        handle.set_roles(mk.OP_MOE)
    for key in ref:
        assert np.array_equal(out[key], ref[key]), f"{key} differs with roles {roles}"


def test_moe_no_local_tokens(handle):
    """Degenerate case: no token picks a local expert -> zero slots, no tiles."""
    S, T, H, N, E, E_loc, top_k = 2, 64, 32, 32, 8, 2, 1
    d = I.gen_moe(S, T, H, N, E, E_loc, I.FLOAT, config=430)
    for s in range(S):
        d["logits"][s][:, :E_loc] = -50.0
    out = run_moe(handle, d, E, top_k, rank=0)
    assert out["expert_offsets"].tolist() == [0] * (E_loc + 1)
    check_moe(d, out, top_k, 0, I.FLOAT)


@pytest.mark.parametrize("variant", [I.FLOAT, I.INTEGER])
def test_moe_full_size(handle, variant):
    """The full workload: every routed slot's output row."""
    name = "moe_s8_t4096_h4096_n1536_e64"
    p = I.CONFIGS[name].params
    print(f"{name} variant={variant}", flush=True)
    d = I.gen_workload(name, variant)
    out = run_moe(handle, d, p["E"], p["top_k"], rank=0)
    check_moe(d, out, p["top_k"], 0, variant)
