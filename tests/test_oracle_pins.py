"""Pins for the CPU oracle, independent of the oracle's own code paths.

Each test checks the oracle against something fixed outside it: exhaustive or
brute-force enumeration, exact rational arithmetic, special cases with a closed
form, invariants of the operations, or hand-worked examples (tests/golden).
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O
from communication_gemm_persistent_amd import inputs as I

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bits(vals):
    """Exact bf16 bit patterns of values that are representable in bf16."""
    f = np.asarray(vals, dtype=np.float32)
    u = f.view(np.uint32)
    assert np.all((u & 0xFFFF) == 0), "value not representable in bf16"
    return (u >> 16).astype(np.uint16)


def _load(name):
    with open(os.path.join(GOLDEN, name)) as fh:
        return json.load(fh)


# ---------------------------------------------------------------- bf16 rounding

ALL_BF16 = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)


def _finite_bf16_sorted():
    v = O.bf16_to_f64(ALL_BF16)
    fin = np.isfinite(v)
    vals, bits = v[fin], ALL_BF16[fin]
    # drop -0 (keeps +0 as the representative of zero)
    keep = ~((vals == 0) & (bits == 0x8000))
    vals, bits = vals[keep], bits[keep]
    o = np.argsort(vals, kind="stable")
    return vals[o], bits[o]


def _nearest_even_bruteforce(x):
    """Nearest finite bf16 by search over all patterns; ties to even mantissa."""
    vals, bits = _finite_bf16_sorted()
    out = np.empty(x.shape, dtype=np.uint16)
    i = np.searchsorted(vals, x)
    for n, xv in enumerate(x):
        lo = max(i[n] - 1, 0)
        hi = min(i[n], len(vals) - 1)
        cands = [(abs(vals[j] - xv), int(bits[j]) & 1, j) for j in {lo, hi}]
        cands.sort()
        if len(cands) == 2 and cands[0][0] == cands[1][0]:
            j = cands[0][2] if cands[0][1] == 0 else cands[1][2]
        else:
            j = cands[0][2]
        b = int(bits[j])
        if vals[j] == 0 and xv < 0:
            b = 0x8000                         # -0 for negative underflow
        out[n] = b
    return out


def test_bf16_hand_patterns():
    one = 1.0
    cases = [
        (one, 0x3F80),
        (one + 2.0 ** -8, 0x3F80),            # tie -> even (1.0)
        (one + 3 * 2.0 ** -8, 0x3F82),        # tie between 0x3F81 and 0x3F82 -> even
        (one + 2.0 ** -8 + 2.0 ** -30, 0x3F81),  # just above the tie
        (2.0 - 2.0 ** -9, 0x4000),            # carry into the exponent
        (0.0, 0x0000),
        (-0.0, 0x8000),
        (3.3895313892515355e38, 0x7F7F),      # largest finite bf16
        (-2.0, 0xC000),
        (2.0 ** -133, 0x0001),                # smallest subnormal
    ]
    for x, want in cases:
        got = int(O.f64_to_bf16(np.array([x]))[0])
        assert got == want, (x, hex(got), hex(want))
    assert np.isinf(O.bf16_to_f64(O.f64_to_bf16(np.array([3.4e38]))))[0]
    assert np.isnan(O.bf16_to_f64(O.f64_to_bf16(np.array([np.nan]))))[0]


def test_bf16_roundtrip_exhaustive():
    v = O.bf16_to_f64(ALL_BF16)
    ok = ~np.isnan(v)
    assert np.array_equal(O.f64_to_bf16(v[ok]), ALL_BF16[ok])
    assert np.array_equal(O.f32_to_bf16(v[ok].astype(np.float32)), ALL_BF16[ok])


def test_f64_to_bf16_matches_bruteforce_nearest():
    g = np.random.default_rng(7)
    x = np.concatenate([
        g.standard_normal(3000),
        g.standard_normal(500) * 1e-39,       # subnormal range
        g.uniform(-1, 1, 500) * 3.3e38,
        (1 + (g.integers(0, 256, 500) + 0.5) * 2.0 ** -7),  # exact ties
        g.integers(-40000, 40000, 500).astype(np.float64),
    ])
    assert np.array_equal(O.f64_to_bf16(x), _nearest_even_bruteforce(x))


def test_f32_to_bf16_matches_torch_library_conversion():
    g = np.random.default_rng(8)
    x = np.concatenate([g.standard_normal(20000).astype(np.float32),
                        g.integers(-(1 << 24), 1 << 24, 2000).astype(np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(O.f32_to_bf16(x), ref)


# ---------------------------------------------------------------- GEMM

def _exact_gemm(a_bits, b_bits):
    a = [[Fraction(float(v)) for v in row] for row in O.bf16_to_f64(a_bits)]
    b = [[Fraction(float(v)) for v in row] for row in O.bf16_to_f64(b_bits)]
    M, K, N = len(a), len(b), len(b[0])
    return [[sum((a[i][k] * b[k][j] for k in range(K)), Fraction(0)) for j in range(N)]
            for i in range(M)]


@pytest.mark.parametrize("shape", [(3, 5, 7), (1, 1, 1), (7, 1, 4), (4, 16, 2), (9, 33, 6), (5, 6, 6)])
def test_gemm_exact_bruteforce(shape):
    M, K, N = shape
    a = I.draw_bf16(0, 901, 0, (M, K), "normal", 1.0)
    b = I.draw_bf16(0, 901, 1, (K, N), "normal", 1.0)
    p = O.gemm(a, b)
    ex = _exact_gemm(a, b)
    absab = np.abs(O.bf16_to_f64(a)) @ np.abs(O.bf16_to_f64(b))
    gam = K * 2.0 ** -53 / (1 - K * 2.0 ** -53)
    c = O.f64_to_bf16(p)
    for i in range(M):
        for j in range(N):
            assert abs(Fraction(p[i, j]) - ex[i][j]) <= Fraction(gam * absab[i, j]) + Fraction(1, 1 << 1100)
            # the bf16 output is the correctly rounded exact value unless the
            # exact value sits within the float64 error band of a rounding tie
            want = int(_nearest_even_bruteforce(np.array([float(ex[i][j])]))[0])
            if int(c[i, j]) != want:
                lo = float(ex[i][j]) - gam * absab[i, j]
                hi = float(ex[i][j]) + gam * absab[i, j]
                assert O.f64_to_bf16(np.array([lo]))[0] != O.f64_to_bf16(np.array([hi]))[0]


def test_gemm_integer_exact():
    a = I.draw_bf16(1, 902, 0, (6, 40), "normal")
    b = I.draw_bf16(1, 902, 1, (40, 5), "normal")
    ai = O.bf16_to_f64(a).astype(np.int64)
    bi = O.bf16_to_f64(b).astype(np.int64)
    want = [[sum(int(ai[i, k]) * int(bi[k, j]) for k in range(40)) for j in range(5)]
            for i in range(6)]
    assert np.array_equal(O.gemm(a, b), np.array(want, dtype=np.float64))


def test_gemm_identity_and_unit_vectors():
    a = I.draw_bf16(0, 903, 0, (5, 8), "normal")
    eye = _bits(np.eye(8))
    assert np.array_equal(O.f64_to_bf16(O.gemm(a, eye)), a)
    b = I.draw_bf16(0, 903, 1, (8, 6), "normal")
    for i in range(8):
        e = np.zeros((1, 8))
        e[0, i] = 1.0
        assert np.array_equal(O.f64_to_bf16(O.gemm(_bits(e), b))[0], b[i])


def test_gemm_rejects_mismatched_shapes():
    with pytest.raises(ValueError):
        O.gemm(np.zeros((2, 3), np.uint16), np.zeros((4, 2), np.uint16))


# ---------------------------------------------------------------- AllGather + GEMM

def test_ag_gemm_golden_hand_example():
    g = _load("ag_gemm_w2_hand.json")
    shards = [_bits(s) for s in g["shards"]]
    out = O.ag_gemm(shards, _bits(g["b"]))
    assert np.array_equal(out["c"], _bits(g["c"]))


def test_ag_gemm_identity_pins_gather_order():
    shards = [I.draw_bf16(0, 904, q, (3, 16), "normal") for q in range(4)]
    out = O.ag_gemm(shards, _bits(np.eye(16)))
    assert np.array_equal(out["c"], np.concatenate(shards))
    assert np.array_equal(out["a_gathered"], np.concatenate(shards))


def test_ag_gemm_integer_small_config_exact():
    d = I.gen_workload("ag_gemm_w4_512x256x256", I.INTEGER)
    out = O.ag_gemm(d["shards"], d["b"])
    a = np.concatenate([O.bf16_to_f64(s) for s in d["shards"]]).astype(np.int64)
    b = O.bf16_to_f64(d["b"]).astype(np.int64)
    p = a @ b                                   # integer arithmetic
    assert np.abs(p).max() < 2 ** 24
    assert np.array_equal(out["c"], O.f64_to_bf16(p.astype(np.float64)))


def test_ag_gemm_rows_matches_full():
    d = I.gen_ag(3, 5, 7, 16, I.FLOAT, config=905)
    full = O.ag_gemm(d["shards"], d["b"])["c"]
    rows = np.array([0, 4, 5, 14])
    assert np.array_equal(O.ag_gemm_rows(d["shards"], d["b"], rows), full[rows])


# ---------------------------------------------------------------- GEMM + ReduceScatter

def test_gemm_rs_golden_hand_example():
    g = _load("gemm_rs_w2_hand.json")
    out = O.gemm_rs(_bits(g["a"]), _bits(g["b"]),
                    [None, np.array(g["peer_partial_slice0_from_rank1"], np.float32)], rank=0)
    assert np.array_equal(out["c_own"], _bits(g["c_own"]))
    assert np.array_equal(out["outbox"][1], _bits(g["outbox_to_rank1"]))


def test_gemm_rs_zero_a_is_pure_reduce():
    W, m, n, k = 4, 8, 6, 5
    d = I.gen_rs(W, m, n, k, rank=2, config=906)
    zero = np.zeros((m, k), np.uint16)
    out = O.gemm_rs(zero, d["b"], d["peers"], rank=2)
    s = sum(np.asarray(p, np.float64) for p in d["peers"] if p is not None)
    assert np.array_equal(out["c_own"], O.f64_to_bf16(s))
    for q in range(W):
        if q != 2:
            assert not out["outbox"][q].any()


def test_gemm_rs_zero_peers_slices_tile_product():
    W, m, n, k = 4, 12, 5, 7
    d = I.gen_rs(W, m, n, k, rank=1, config=907)
    peers = [None if p is None else np.zeros_like(p) for p in d["peers"]]
    out = O.gemm_rs(d["a"], d["b"], peers, rank=1)
    tiles = [out["c_own"] if q == 1 else out["outbox"][q] for q in range(W)]
    assert np.array_equal(np.concatenate(tiles), O.f64_to_bf16(O.gemm(d["a"], d["b"])))


def test_gemm_rs_w_rank_emulation_tiles_full_sum():
    """Run the op as every rank; each rank's peers are the others' outboxes.
    The concatenated own slices must equal bf16(sum_r A_r @ B_r) exactly."""
    W, m, n, k = 4, 8, 6, 10
    A = [I.draw_bf16(1, 908, r, (m, k), "normal") for r in range(W)]
    B = [I.draw_bf16(1, 908, 10 + r, (k, n), "normal") for r in range(W)]
    zero_peers = [np.zeros((m // W, n), np.float32)] * W
    outbox = [O.gemm_rs(A[r], B[r], [None if q == r else zero_peers[q] for q in range(W)],
                        rank=r)["outbox"] for r in range(W)]
    slices = []
    for r in range(W):
        peers = [None if q == r else O.bf16_to_f64(outbox[q][r]).astype(np.float32)
                 for q in range(W)]
        slices.append(O.gemm_rs(A[r], B[r], peers, rank=r)["c_own"])
    tot = sum(O.bf16_to_f64(A[r]).astype(np.int64) @ O.bf16_to_f64(B[r]).astype(np.int64)
              for r in range(W))
    assert np.abs(tot).max() <= 256
    assert np.array_equal(np.concatenate(slices), O.f64_to_bf16(tot.astype(np.float64)))


def test_gemm_rs_rows_matches_full():
    W, m, n, k = 4, 8, 5, 6
    d = I.gen_rs(W, m, n, k, rank=0, config=909)
    out = O.gemm_rs(d["a"], d["b"], d["peers"], rank=0)
    full = np.concatenate([out["c_own"]] + [out["outbox"][q] for q in range(1, W)])
    rows = np.array([0, 1, 3, 6, 7])
    assert np.array_equal(O.gemm_rs_rows(d["a"], d["b"], d["peers"], 0, rows), full[rows])


# ---------------------------------------------------------------- GEMM + AllReduce

def test_gemm_ar_golden_hand_example():
    g = _load("gemm_ar_w2_hand.json")
    out = O.gemm_ar(_bits(g["a"]), _bits(g["b"]),
                    [None, np.array(g["peer_partial_from_rank1"], np.float32)], rank=0, n_bcast=1)
    assert np.array_equal(out["c"], _bits(g["c"]))
    assert np.array_equal(out["bcast"][0], out["c"])


def test_gemm_ar_equals_rs_then_gather_integer():
    W, m, n, k = 4, 8, 6, 9
    A = [I.draw_bf16(1, 910, r, (m, k), "normal") for r in range(W)]
    B = [I.draw_bf16(1, 910, 10 + r, (k, n), "normal") for r in range(W)]
    P = [O.bf16_to_f64(A[r]).astype(np.int64) @ O.bf16_to_f64(B[r]).astype(np.int64)
         for r in range(W)]
    ar = [O.gemm_ar(A[r], B[r], [None if q == r else P[q].astype(np.float32)
                                 for q in range(W)], rank=r, n_bcast=2) for r in range(W)]
    rs_slices = []
    for r in range(W):
        peers = [None if q == r else P[q][r * m // W:(r + 1) * m // W].astype(np.float32)
                 for q in range(W)]
        rs_slices.append(O.gemm_rs(A[r], B[r], peers, rank=r)["c_own"])
    gathered = np.concatenate(rs_slices)
    for r in range(W):
        assert np.array_equal(ar[r]["c"], gathered)
        for bb in ar[r]["bcast"]:
            assert np.array_equal(bb, ar[r]["c"])


def test_gemm_ar_zero_a_is_pure_sum():
    d = I.gen_ar(3, 4, 5, 6, rank=0, config=911)
    out = O.gemm_ar(np.zeros((4, 6), np.uint16), d["b"], d["peers"], rank=0, n_bcast=1)
    s = np.asarray(d["peers"][1], np.float64) + np.asarray(d["peers"][2], np.float64)
    assert np.array_equal(out["c"], O.f64_to_bf16(s))


def test_gemm_ar_rows_matches_full():
    d = I.gen_ar(3, 6, 5, 4, rank=1, config=912)
    full = O.gemm_ar(d["a"], d["b"], d["peers"], rank=1)["c"]
    rows = np.array([0, 2, 5])
    assert np.array_equal(O.gemm_ar_rows(d["a"], d["b"], d["peers"], 1, rows), full[rows])


# ---------------------------------------------------------------- MoE

def test_moe_golden_hand_example():
    g = _load("moe_dispatch_hand.json")
    S, T, E, E_loc = g["S"], g["T"], g["E"], g["E_loc"]
    logits = np.array(g["logits"], np.float32).reshape(S * T, E)
    r = O.moe_route(logits, g["top_k"])
    assert np.array_equal(r["idx"], np.array(g["topk_idx"], np.int32))
    u = g["uniform_token"]
    assert np.array_equal(r["gate"][u["row"]], np.array(u["gates"]))
    d = O.moe_dispatch(r["idx"], r["gate"], S, T, E_loc, g["rank"])
    assert np.array_equal(d["slot_token"], np.array(g["slot_token"], np.int32))
    assert np.array_equal(d["expert_offsets"], np.array(g["expert_offsets"], np.int32))
    assert np.array_equal(d["chunk_offsets"], np.array(g["chunk_offsets"], np.int32))


def test_moe_routing_matches_bruteforce_sort():
    lg = I.draw_logits(0, 913, 0, (300, 64))
    lg[:20, 5] = lg[:20, 9] = lg[:20].max(axis=1) + 1.0     # forced top ties
    r = O.moe_route(lg, 2)
    for t in range(lg.shape[0]):
        want = sorted(range(64), key=lambda e: (-float(lg[t, e]), e))[:2]
        assert list(r["idx"][t]) == want
    assert np.all(r["idx"][:20] == np.array([5, 9]))


def test_moe_gates_are_softmax():
    """Gates: softmax over all experts, pinned by its two defining properties
    (probabilities sum to 1, p_i / p_j = exp(l_i - l_j)) and the uniform case."""
    lg = I.draw_logits(0, 914, 0, (200, 64))
    r = O.moe_route(lg, 2)
    p = r["prob"]
    assert np.allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-12)
    l64 = lg.astype(np.float64)
    for t in range(0, 200, 17):
        for i, j in [(0, 1), (3, 40), (int(r["idx"][t, 0]), int(r["idx"][t, 1]))]:
            assert math.isclose(p[t, i] / p[t, j], math.exp(l64[t, i] - l64[t, j]), rel_tol=1e-12)
    assert np.array_equal(r["gate"], np.take_along_axis(p, r["idx"].astype(np.int64), 1))
    ru = O.moe_route(np.zeros((3, 64), np.float32), 2)
    assert np.all(ru["gate"] == 1.0 / 64) and np.all(ru["idx"] == np.array([0, 1]))


def _small_moe(variant=I.FLOAT, S=3, T=50, H=24, N=16, E=8, E_loc=4, config=915):
    return I.gen_moe(S, T, H, N, E, E_loc, variant, config=config)


def test_moe_counts_and_offsets_bruteforce():
    S, T, E, E_loc, rank = 3, 50, 8, 4, 1
    d = _small_moe(S=S, T=T, E=E, E_loc=E_loc)
    lg = np.concatenate(d["logits"])
    r = O.moe_route(lg, 2)
    disp = O.moe_dispatch(r["idx"], r["gate"], S, T, E_loc, rank)
    for e in range(E_loc):
        for s in range(S):
            cnt = sum(1 for t in range(T) if rank * E_loc + e in r["idx"][s * T + t])
            assert disp["chunk_offsets"][e, s + 1] - disp["chunk_offsets"][e, s] == cnt
        assert disp["chunk_offsets"][e, 0] == disp["expert_offsets"][e]
        assert disp["chunk_offsets"][e, S] == disp["expert_offsets"][e + 1]
    n_local = int(np.isin(r["idx"], np.arange(rank * E_loc, (rank + 1) * E_loc)).sum())
    assert disp["expert_offsets"][-1] == n_local
    tok, cnt = np.unique(disp["slot_token"], return_counts=True)
    assert cnt.max() <= 2


def test_moe_dispatch_permutation_inverts():
    S, T = 3, 50
    d = _small_moe(S=S, T=T)
    out = O.moe_dispatch_gemm(d["x"], d["logits"], d["w"], top_k=2, rank=0)
    x_all = np.concatenate(d["x"])
    back = np.zeros_like(x_all)
    back[out["slot_token"]] = out["x_slots"]
    sel = np.unique(out["slot_token"])
    assert np.array_equal(back[sel], x_all[sel])
    e = O.slot_expert(out["expert_offsets"], out["n_slots"])
    for i in range(out["n_slots"]):
        t = out["slot_token"][i]
        assert e[i] in out["idx"][t] - 0            # rank 0: local id == global id
        assert out["slot_gate"][i] == out["gate"][t][list(out["idx"][t]).index(e[i])]
    # within an expert, slot tokens ascend (source-major, token-minor order)
    for k in range(len(out["expert_offsets"]) - 1):
        st = out["slot_token"][out["expert_offsets"][k]:out["expert_offsets"][k + 1]]
        assert np.all(np.diff(st) > 0)


def test_moe_identity_expert_weights_pin_gating():
    """With W_e = [I; 0] the expert GEMM selects the first N features, so
    y = bf16(gate * x[:, :N]) exactly for every slot."""
    S, T, H, N, E, E_loc = 2, 40, 24, 16, 8, 4
    d = _small_moe(S=S, T=T, H=H, N=N, E=E, E_loc=E_loc, config=916)
    w = np.zeros((E_loc, H, N), np.float32)
    for e in range(E_loc):
        w[e, :N, :N] = np.eye(N)
    wb = _bits(w)
    out = O.moe_dispatch_gemm(d["x"], d["logits"], wb, top_k=2)
    x_all = np.concatenate(d["x"])
    xs = O.bf16_to_f64(x_all[out["slot_token"]][:, :N])
    assert np.array_equal(out["y"], O.f64_to_bf16(xs * out["slot_gate"][:, None]))
    ung = O.moe_dispatch_gemm(d["x"], d["logits"], wb, top_k=2, apply_gate=False)
    assert np.array_equal(ung["y"], x_all[out["slot_token"]][:, :N])


def test_moe_slot_subset_matches_full():
    d = _small_moe(config=917)
    full = O.moe_dispatch_gemm(d["x"], d["logits"], d["w"], top_k=2)
    sl = np.array([0, 3, full["n_slots"] - 1])
    part = O.moe_dispatch_gemm(d["x"], d["logits"], d["w"], top_k=2, slots=sl)
    assert np.array_equal(part["y"], full["y"][sl])


# ---------------------------------------------------------------- inputs

def test_generator_is_deterministic_and_seed_keyed():
    a = I.draw_bf16(0, 1, 3, (64, 32), "normal")
    b = I.draw_bf16(0, 1, 3, (64, 32), "normal")
    c = I.draw_bf16(1, 1, 3, (64, 32), "normal")
    d = I.draw_bf16(0, 1, 4, (64, 32), "normal")
    assert np.array_equal(a, b) and not np.array_equal(a, c) and not np.array_equal(a, d)
    iv = O.bf16_to_f64(c)
    assert set(np.unique(iv)).issubset({-2.0, -1.0, 0.0, 1.0, 2.0})
    p = I.draw_f32(1, 1, 5, (100,))
    assert set(np.unique(p)).issubset(set(float(v) for v in range(-4, 5)))


def test_generator_distributions():
    x = O.bf16_to_f64(I.draw_bf16(0, 2, 0, (512, 512), "normal", 0.02))
    assert abs(x.std() - 0.02) < 0.001 and abs(x.mean()) < 0.001
    u = O.bf16_to_f64(I.draw_bf16(0, 2, 1, (512, 512), "uniform", 1.0))
    assert u.min() >= -1 and u.max() <= 1 and abs(u.std() - 1 / math.sqrt(3)) < 0.01


# ---------------------------------------------------------------- MoE combine

def _combine_hand():
    g = json.load(open(os.path.join(GOLDEN, "moe_combine_hand.json")))
    bf = lambda a: O.f64_to_bf16(np.asarray(a, dtype=np.float64))
    x = [bf(v) for v in g["x"]]
    logits = [np.asarray(v, dtype=np.float32) for v in g["logits"]]
    w = bf(g["w"])
    return g, O.moe_combine(x, logits, w, g["top_k"], bf(g["y_peer"]), rank=g["rank"])


def test_moe_combine_hand_worked():
    g, r = _combine_hand()
    np.testing.assert_array_equal(r["idx"], np.asarray(g["topk_idx"]))
    np.testing.assert_array_equal(r["slot_token"], np.asarray(g["slot_token"]))
    np.testing.assert_array_equal(O.bf16_to_f64(r["y"]), np.asarray(g["y"]))
    np.testing.assert_array_equal(r["return_pos"], np.asarray(g["return_pos"]))
    np.testing.assert_array_equal(r["ret_mask"][1], np.asarray(g["ret_mask_source1"]))
    np.testing.assert_array_equal(O.bf16_to_f64(r["ret"][1]), np.asarray(g["ret_source1"]))
    np.testing.assert_array_equal(O.bf16_to_f64(r["out"]), np.asarray(g["out"]))


def test_moe_combine_return_is_a_permutation_of_the_slots():
    """Every slot returns to exactly one (source, token, k) whose top-k entry
    is the slot's expert; no two slots share a position."""
    S, T, H, N, E, E_loc, k, rank = 3, 40, 16, 8, 6, 2, 2, 1
    rng = np.random.default_rng(7)
    x = [O.f64_to_bf16(rng.standard_normal((T, H))) for _ in range(S)]
    logits = [rng.standard_normal((T, E)).astype(np.float32) for _ in range(S)]
    w = O.f64_to_bf16(0.1 * rng.standard_normal((E_loc, H, N)))
    yp = O.f64_to_bf16(rng.standard_normal((T, k, N)))
    r = O.moe_combine(x, logits, w, k, yp, rank=rank)
    pos = r["return_pos"]
    assert len(set(pos.tolist())) == len(pos)
    flat_idx = r["idx"].reshape(-1)
    exp_of = O.slot_expert(r["expert_offsets"], len(pos))
    np.testing.assert_array_equal(flat_idx[pos], rank * E_loc + exp_of)
    np.testing.assert_array_equal(pos // k, r["slot_token"])
    # the mask marks exactly the (t, k) pairs of local experts
    local = (r["idx"] >= rank * E_loc) & (r["idx"] < (rank + 1) * E_loc)
    np.testing.assert_array_equal(r["ret_mask"].reshape(S * T, k), local)


def test_moe_combine_all_experts_remote_is_a_plain_sum():
    """No token picks a local expert: the combine sums the returned rows."""
    S, T, H, N, E, E_loc, k = 2, 8, 4, 4, 4, 2, 2
    rng = np.random.default_rng(3)
    logits = [rng.standard_normal((T, E)).astype(np.float32) for _ in range(S)]
    for l in logits:
        l[:, :E_loc] -= 1000.0  # experts 0..E_loc-1 (rank 0's) are never chosen
    x = [O.f64_to_bf16(rng.standard_normal((T, H))) for _ in range(S)]
    w = O.f64_to_bf16(rng.standard_normal((E_loc, H, N)))
    yp = O.f64_to_bf16(np.arange(T * k * N, dtype=np.float64).reshape(T, k, N) * 0.5 - 7.0)
    r = O.moe_combine(x, logits, w, k, yp, rank=0)
    assert r["n_slots"] == 0 and not r["ret_mask"].any()
    expect = (np.arange(T * k * N, dtype=np.float64).reshape(T, k, N) * 0.5 - 7.0).sum(axis=1)
    np.testing.assert_array_equal(O.bf16_to_f64(r["out"]), expect)


def test_moe_combine_top1_all_local_is_y_in_token_order():
    """top_k = 1 and every expert local: out[t] is y of t's slot, unchanged."""
    S, T, H, N, E = 1, 24, 8, 8, 3
    rng = np.random.default_rng(5)
    x = [O.f64_to_bf16(rng.standard_normal((T, H)))]
    logits = [rng.standard_normal((T, E)).astype(np.float32)]
    w = O.f64_to_bf16(rng.standard_normal((E, H, N)))
    r = O.moe_combine(x, logits, w, 1, np.zeros((T, 1, N), dtype=np.uint16), rank=0)
    inv = np.empty(T, dtype=np.int64)
    inv[r["slot_token"]] = np.arange(T)
    np.testing.assert_array_equal(r["out"], r["y"][inv])


def test_moe_combine_sampled_tokens_match_the_full_combine():
    """The sampled form (used at large sizes) gives the full form's rows for
    the sampled tokens and multiplies only the slots they use."""
    S, T, H, N, E, E_loc, k, rank = 3, 50, 16, 8, 8, 3, 3, 1
    rng = np.random.default_rng(11)
    x = [O.f64_to_bf16(rng.standard_normal((T, H))) for _ in range(S)]
    logits = [rng.standard_normal((T, E)).astype(np.float32) for _ in range(S)]
    w = O.f64_to_bf16(0.2 * rng.standard_normal((E_loc, H, N)))
    yp = O.f64_to_bf16(rng.standard_normal((T, k, N)))
    full = O.moe_combine(x, logits, w, k, yp, rank=rank)
    toks = np.array([0, 3, 17, 31, 49])
    part = O.moe_combine(x, logits, w, k, yp, rank=rank, tokens=toks)
    assert 0 < len(part["slots"]) < full["n_slots"]
    np.testing.assert_array_equal(part["out"], full["out"][toks])
    np.testing.assert_array_equal(part["y"], full["y"][part["slots"]])
    np.testing.assert_array_equal(part["return_pos"], full["return_pos"])
    used = np.isin(full["slot_token"], rank * T + toks)
    np.testing.assert_array_equal(part["slots"], np.nonzero(used)[0])


# ---------------------------------------------------------------- ring attention

def _bf(a):
    return O.f64_to_bf16(np.asarray(a, dtype=np.float64))


def _ring_hand():
    g = json.load(open(os.path.join(GOLDEN, "ring_attention_hand.json")))
    q = _bf(g["q"])
    ks = [_bf(k) for k in g["k_src"]]
    vs = [_bf(v) for v in g["v_src"]]
    return g, q, ks, vs


@pytest.mark.parametrize("rank", [0, 1])
def test_ring_attention_hand_worked(rank):
    g, q, ks, vs = _ring_hand()
    r = O.ring_attention(q, ks, vs, rank=rank, scale=g["scale"])
    np.testing.assert_allclose(r["o_f64"], np.asarray(g["o"]), rtol=1e-12, atol=1e-15)
    np.testing.assert_array_equal(r["o"], _bf(g["o"]))
    np.testing.assert_allclose(r["lse"], np.asarray(g["lse"]), rtol=1e-12)
    np.testing.assert_array_equal(r["order"], g[f"order_rank{rank}"])


def _ring_random(seed, W=3, B=2, H=2, S_q=5, S_kv=4, D=8):
    rng = np.random.default_rng(seed)
    q = _bf(rng.standard_normal((B, H, S_q, D)))
    ks = [_bf(rng.standard_normal((B, H, S_kv, D))) for _ in range(W)]
    vs = [_bf(rng.standard_normal((B, H, S_kv, D))) for _ in range(W)]
    return q, ks, vs


def test_ring_attention_zero_queries_average_the_values():
    """Q = 0: every score is 0, the weights are uniform over all W * S_kv keys,
    o is the mean of every value row and lse = log(W * S_kv)."""
    q, ks, vs = _ring_random(1)
    q = np.zeros_like(q)
    r = O.ring_attention(q, ks, vs, rank=2)
    allv = np.concatenate([O.bf16_to_f64(v) for v in vs], axis=2)      # [B, H, W*S_kv, D]
    mean = allv.mean(axis=2, keepdims=True)
    np.testing.assert_allclose(r["o_f64"], np.broadcast_to(mean, r["o_f64"].shape), atol=1e-14)
    np.testing.assert_allclose(r["lse"], np.log(3 * 4), rtol=1e-14)


def test_ring_attention_equal_values_pass_through():
    """Every value row equal to u: the output is u whatever the scores."""
    q, ks, vs = _ring_random(2)
    u = _bf(np.linspace(-2, 3, 8))
    vs = [np.broadcast_to(u, v.shape).copy() for v in vs]
    r = O.ring_attention(q, ks, vs, rank=0)
    np.testing.assert_array_equal(r["o"], np.broadcast_to(u, r["o"].shape))


def test_ring_attention_single_key_is_its_value():
    """One rank, one key: the softmax weight is 1, o = v and lse = scale q.k."""
    q, ks, vs = _ring_random(3, W=1, S_kv=1)
    r = O.ring_attention(q, ks, vs, rank=0, scale=0.75)
    np.testing.assert_array_equal(r["o"], np.broadcast_to(vs[0], r["o"].shape))
    qk = (O.bf16_to_f64(q) * O.bf16_to_f64(ks[0])).sum(axis=-1)
    np.testing.assert_allclose(r["lse"], 0.75 * qk, rtol=1e-13, atol=1e-13)


def test_ring_attention_order_and_head_split_invariance():
    """The ring order permutes (key, value) pairs only: every rank order gives
    the same result; heads and batches are independent problems."""
    q, ks, vs = _ring_random(4)
    base = O.ring_attention(q, ks, vs, rank=0)
    for rank in (1, 2):
        r = O.ring_attention(q, ks, vs, rank=rank)
        assert r["order"][0] == rank
        np.testing.assert_allclose(r["o_f64"], base["o_f64"], rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(r["lse"], base["lse"], rtol=1e-13)
    one = O.ring_attention(q[1:2, 1:2], [k[1:2, 1:2] for k in ks], [v[1:2, 1:2] for v in vs])
    np.testing.assert_allclose(one["o_f64"][0, 0], base["o_f64"][1, 1], rtol=1e-12, atol=1e-14)


def test_ring_attention_scale_acts_on_the_queries():
    """scale c on Q equals scale 1 on c Q (c a power of two keeps Q exact)."""
    q, ks, vs = _ring_random(5)
    a = O.ring_attention(q, ks, vs, rank=1, scale=0.25)
    q4 = _bf(O.bf16_to_f64(q) * 0.25)
    b = O.ring_attention(q4, ks, vs, rank=1, scale=1.0)
    np.testing.assert_allclose(a["o_f64"], b["o_f64"], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(a["lse"], b["lse"], rtol=1e-13)


def test_ring_attention_rows_subset_matches_full():
    q, ks, vs = _ring_random(6)
    full = O.ring_attention(q, ks, vs, rank=1)
    rows = np.array([0, 3, 4])
    part = O.ring_attention(q, ks, vs, rank=1, rows=rows)
    np.testing.assert_array_equal(part["o"], full["o"][:, :, rows])
    np.testing.assert_allclose(part["lse"], full["lse"][:, :, rows], rtol=1e-15)


def test_ring_attention_peaked_scores_select_one_value():
    """One key scores far above the rest (120 against 0): o is its value to
    within exp(-120) relative."""
    q, ks, vs = _ring_random(7, W=2, B=1, H=1, S_q=1, S_kv=3, D=4)
    q = _bf([[[[8.0, 0, 0, 0]]]])
    ks = [np.zeros_like(k) for k in ks]
    ks[1] = ks[1].copy()
    ks[1][0, 0, 2] = _bf([15.0, 0, 0, 0])
    r = O.ring_attention(q, ks, vs, rank=0, scale=1.0)
    np.testing.assert_allclose(r["o_f64"][0, 0, 0], O.bf16_to_f64(vs[1][0, 0, 2]), atol=1e-20)


# ---------------------------------------------------------------- gated output from given fp32 gates

def _round_even(x, frac_bits):
    """Exact round-to-nearest-even of a Fraction to a binary float with
    frac_bits fraction bits (normal range only)."""
    from fractions import Fraction
    if x == 0:
        return Fraction(0)
    sgn = -1 if x < 0 else 1
    a = abs(x)
    e = 0
    while a >= 2:
        a /= 2
        e += 1
    while a < 1:
        a *= 2
        e -= 1
    ulp = Fraction(2) ** (e - frac_bits)
    q = abs(x) / ulp
    fl = q.numerator // q.denominator
    rem = q - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sgn * fl * ulp


def _two_step(gate32, acc):
    """fp32(gate * acc), then bf16: the kernel's gate multiply and store."""
    from fractions import Fraction
    return float(_round_even(_round_even(Fraction(float(gate32)) * int(acc), 23), 7))


def test_moe_y_given_gates_bruteforce():
    """Integer expert products times fp32 gates: y equals, element by element,
    exact rational arithmetic rounded to fp32 and then to bf16."""
    g = np.random.default_rng(11)
    n_slots, H, N, E_loc = 12, 24, 8, 2
    x = O.f64_to_bf16(g.integers(-2, 3, (n_slots, H)).astype(np.float64))
    w = O.f64_to_bf16(g.integers(-2, 3, (E_loc, H, N)).astype(np.float64))
    eoff = np.array([0, 5, n_slots], dtype=np.int32)
    gates = g.uniform(0.01, 1.0, n_slots).astype(np.float32)
    y = O.moe_y_given_gates(x, w, eoff, gates)
    xf = O.bf16_to_f64(x)
    wf = O.bf16_to_f64(w)
    for slot in range(n_slots):
        e = 0 if slot < 5 else 1
        for j in range(N):
            acc = int(sum(int(xf[slot, h]) * int(wf[e, h, j]) for h in range(H)))
            want = _two_step(gates[slot], acc)
            assert O.bf16_to_f64(y[slot:slot + 1, j])[0] == want, (slot, j, acc)


def test_moe_y_given_gates_rounds_in_fp32_first():
    """Where rounding the exact product straight to bf16 differs from rounding
    it to fp32 first (a double rounding), the fp32-first result is taken.
    Cases: gate = fp32(m / acc) for a bf16 midpoint m, so that gate * acc lies
    within half an fp32 ulp of m, above it; fp32 rounding lands on m, which
    then ties to even, while a direct rounding goes up."""
    found = 0
    for m in (1.0 + 2.0 ** -8, 3.0 + 2.0 ** -7, 0.75 + 2.0 ** -9):
        for acc in range(3, 256, 2):
            gate = np.float32(m / acc)
            prod = float(gate) * acc
            if not prod > m:
                continue
            direct = O.bf16_to_f64(O.f64_to_bf16(np.array([prod])))[0]
            two = _two_step(gate, acc)
            assert two != direct
            x = O.f64_to_bf16(np.array([[float(acc)]]))      # a 1 x 1 x 1 product: acc itself
            w = O.f64_to_bf16(np.ones((1, 1, 1)))
            y = O.moe_y_given_gates(x, w, np.array([0, 1], np.int32), np.array([gate]))
            assert O.bf16_to_f64(y)[0, 0] == two
            found += 1
            break
    assert found == 3, "no double-rounding case found"


def test_moe_y_given_gates_unit_gates_give_the_product():
    g = np.random.default_rng(13)
    x = O.f64_to_bf16(g.integers(-2, 3, (9, 16)).astype(np.float64))
    w = O.f64_to_bf16(g.integers(-2, 3, (1, 16, 8)).astype(np.float64))
    y = O.moe_y_given_gates(x, w, np.array([0, 9], np.int32), np.ones(9, np.float32))
    O.assert_bits_equal(y, O.f64_to_bf16(O.gemm(x, w[0])), "unit gates")
