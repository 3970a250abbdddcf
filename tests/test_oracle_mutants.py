"""Planted mistakes in the oracle (on the CPU) must each be caught by a pin.

Each mutant replaces one oracle function with a plausible wrong version; the
listed pin tests must then fail.  This shows the pins constrain the oracle.
"""
import numpy as np
import pytest

import oracle as O
import oracle.mk_oracle as M
from tests import test_oracle_pins as P


def _truncating_bf16(x):
    x32 = np.asarray(x, np.float64).astype(np.float32)
    return (x32.view(np.uint32) >> 16).astype(np.uint16)


def _gemm_transposed_b(a_bits, b_bits):
    a = M.bf16_to_f64(a_bits)
    b = M.bf16_to_f64(b_bits)
    if a.shape[1] != b.shape[0]:
        raise ValueError("shape")
    if b.shape[0] == b.shape[1]:
        return a @ b.T
    return a @ b


def _gemm_drops_last_k(a_bits, b_bits):
    a = M.bf16_to_f64(a_bits)
    b = M.bf16_to_f64(b_bits)
    if a.shape[1] != b.shape[0]:
        raise ValueError("shape")
    return a[:, :-1] @ b[:-1] if a.shape[1] > 1 else a @ b


def _sum_skips_last_peer(own, peers, rank):
    acc = np.array(own, dtype=np.float64, copy=True)
    last = max(q for q in range(len(peers)) if q != rank)
    for q, p in enumerate(peers):
        if q == rank or q == last:
            continue
        acc = acc + np.asarray(p, dtype=np.float64)
    return acc


def _sum_subtracts(own, peers, rank):
    acc = np.array(own, dtype=np.float64, copy=True)
    for q, p in enumerate(peers):
        if q != rank:
            acc = acc - np.asarray(p, dtype=np.float64)
    return acc


_orig_route = M.moe_route


def _route_ties_to_higher_id(logits, top_k):
    lg = np.asarray(logits, np.float32)
    E = lg.shape[1]
    r = _orig_route(lg[:, ::-1], top_k)
    idx = (E - 1 - r["idx"]).astype(np.int32)
    prob = r["prob"][:, ::-1]
    return dict(idx=idx, gate=np.take_along_axis(prob, idx.astype(np.int64), 1), prob=prob)


def _route_renormalised(logits, top_k):
    r = _orig_route(logits, top_k)
    g = r["gate"] / r["gate"].sum(axis=1, keepdims=True)
    return dict(r, gate=g)


_orig_dispatch = M.moe_dispatch


def _dispatch_token_major(idx, gate, S, T, E_loc, rank=0):
    d = _orig_dispatch(idx, gate, S, T, E_loc, rank)
    o = np.argsort(d["slot_token"], kind="stable")
    return dict(d, slot_token=d["slot_token"][o], slot_gate=d["slot_gate"][o])


_orig_return_pos = M.moe_return_positions


def _return_pos_k_reversed(slot_token, idx, expert_offsets, T, top_k, E_loc, rank):
    pos = _orig_return_pos(slot_token, idx, expert_offsets, T, top_k, E_loc, rank)
    return (pos // top_k) * top_k + (top_k - 1 - pos % top_k)


def _combine_variant(regate=False, drop_peer=False, peer_everywhere=False):
    def combine(x, logits, w, top_k, y_peer, rank=0):
        r = dict(_orig_combine(x, logits, w, top_k, y_peer, rank))
        T, N = x[0].shape[0], w.shape[2]
        mask = r["ret_mask"][rank][:, :, None]
        yp = np.asarray(y_peer, dtype=np.uint16).reshape(T, top_k, N)
        if drop_peer:
            yp = np.zeros_like(yp)
        rows = M.bf16_to_f64(yp if peer_everywhere else np.where(mask, r["ret"][rank], yp))
        if regate:
            rows = rows * r["gate"][rank * T:(rank + 1) * T][:, :, None]
        r["out"] = M.f64_to_bf16(rows.sum(axis=1))
        return r
    combine.__name__ = ("_combine_regates" if regate else "_combine_drops_peer_rows" if drop_peer
                        else "_combine_peer_rows_everywhere")
    return combine


_orig_combine = M.moe_combine



def _ring_variant(kind):
    """ring_attention with one plausible mistake: 'noscale' ignores the scale,
    'qaxis' normalises over the queries, 'local' sees only the rank's own
    block, 'log2' reports lse in base 2, 'vorder' pairs keys in ring order
    with values in rank order."""
    def ring(q, k_src, v_src, rank=0, scale=None, rows=None):
        W = len(k_src)
        B, H, S_q, D = q.shape
        sc = 1.0 / np.sqrt(D) if scale is None else float(scale)
        if kind == "noscale":
            sc = 1.0
        order = M.ring_order(W, rank)
        korder = [rank] if kind == "local" else order
        vorder = list(range(W)) if kind == "vorder" else korder
        sel = np.arange(S_q) if rows is None else np.asarray(rows)
        o = np.zeros((B, H, len(sel), D))
        lse = np.zeros((B, H, len(sel)))
        for b in range(B):
            for h in range(H):
                k = np.concatenate([M.bf16_to_f64(np.asarray(k_src[r])[b, h]) for r in korder])
                v = np.concatenate([M.bf16_to_f64(np.asarray(v_src[r])[b, h]) for r in vorder])
                sq = (M.bf16_to_f64(np.asarray(q)[b, h][sel]) @ k.T) * sc
                ax = 0 if kind == "qaxis" else 1
                m = sq.max(axis=ax, keepdims=True)
                pr = np.exp(sq - m)
                den = pr.sum(axis=ax, keepdims=True)
                o[b, h] = (pr / den) @ v
                l = (m + np.log(den))
                l = l[:, 0] if ax == 1 else np.broadcast_to(l, sq.shape)[:, 0]
                lse[b, h] = l / np.log(2.0) if kind == "log2" else l
        return dict(o=M.f64_to_bf16(o), o_f64=o, lse=lse, order=np.array(order),
                    k_recv=np.stack(k_src), v_recv=np.stack(v_src))
    ring.__name__ = f"_ring_{kind}"
    return ring


def _y_given_gates_direct(x_slots, w, expert_offsets, gates_f32):
    n = int(expert_offsets[-1])
    y = np.zeros((n, w.shape[2]), dtype=np.uint16)
    for e in range(w.shape[0]):
        lo, hi = int(expert_offsets[e]), int(expert_offsets[e + 1])
        if hi > lo:
            acc = M.gemm(np.asarray(x_slots)[lo:hi], w[e])
            y[lo:hi] = M.f64_to_bf16(np.asarray(gates_f32, np.float64)[lo:hi, None] * acc)
    return y


MUTANTS = [
    ("moe_y_given_gates", _y_given_gates_direct, [P.test_moe_y_given_gates_rounds_in_fp32_first]),
    ("f64_to_bf16", _truncating_bf16, [P.test_bf16_hand_patterns]),
    ("gemm", _gemm_transposed_b, [lambda: P.test_gemm_exact_bruteforce((5, 6, 6))]),
    ("gemm", _gemm_drops_last_k, [lambda: P.test_gemm_exact_bruteforce((3, 5, 7))]),
    ("_sum_partials", _sum_skips_last_peer, [P.test_gemm_rs_w_rank_emulation_tiles_full_sum]),
    ("_sum_partials", _sum_subtracts, [P.test_gemm_ar_golden_hand_example]),
    ("moe_route", _route_ties_to_higher_id, [P.test_moe_golden_hand_example]),
    ("moe_route", _route_renormalised, [P.test_moe_gates_are_softmax]),
    ("moe_dispatch", _dispatch_token_major, [P.test_moe_golden_hand_example]),
    ("moe_return_positions", _return_pos_k_reversed,
     [P.test_moe_combine_hand_worked, P.test_moe_combine_return_is_a_permutation_of_the_slots]),
    ("moe_combine", _combine_variant(regate=True), [P.test_moe_combine_hand_worked]),
    ("moe_combine", _combine_variant(drop_peer=True),
     [P.test_moe_combine_hand_worked, P.test_moe_combine_all_experts_remote_is_a_plain_sum]),
    ("moe_combine", _combine_variant(peer_everywhere=True),
     [P.test_moe_combine_hand_worked, P.test_moe_combine_top1_all_local_is_y_in_token_order]),
    ("ring_attention", _ring_variant("noscale"), [lambda: P.test_ring_attention_hand_worked(0)]),
    ("ring_attention", _ring_variant("qaxis"), [lambda: P.test_ring_attention_hand_worked(0)]),
    ("ring_attention", _ring_variant("local"),
     [lambda: P.test_ring_attention_hand_worked(0), P.test_ring_attention_zero_queries_average_the_values]),
    ("ring_attention", _ring_variant("log2"), [P.test_ring_attention_single_key_is_its_value]),
    ("ring_attention", _ring_variant("vorder"), [lambda: P.test_ring_attention_hand_worked(1)]),
]


@pytest.mark.parametrize("name,mutant,pins", MUTANTS,
                         ids=[f"{m[0]}-{m[1].__name__}" for m in MUTANTS])
def test_planted_mistake_is_caught(monkeypatch, name, mutant, pins):
    monkeypatch.setattr(M, name, mutant)
    if hasattr(O, name):
        monkeypatch.setattr(O, name, mutant)
    for pin in pins:
        with pytest.raises((AssertionError, ValueError)):
            pin()


# ---------------------------------------------------------------- the comparison rules

import oracle.compare as C  # noqa: E402
from tests import test_compare_pins as CP  # noqa: E402

_orig_report = C.tolerance_report


def _report_variant(kind):
    """tolerance_report with one plausible mistake: 'nan' lets non-finite
    values through (d > bound is False for NaN), 'noabs' uses ref instead of
    |ref|, 'sample_rms' ignores the whole tensor's rms, 'strict' uses < for <=,
    'norel' drops the relative term."""
    def report(gpu_bits, ref_bits, rms=None, rel=C.REL_TOL, rms_tol=C.RMS_TOL):
        g = M.bf16_to_f64(np.asarray(gpu_bits, dtype=np.uint16))
        r = M.bf16_to_f64(np.asarray(ref_bits, dtype=np.uint16))
        if g.shape != r.shape:
            return dict(ok=False, worst=np.inf, n_bad=-1, rms=np.nan, n=r.size, why="shape")
        if rms is None or kind == "sample_rms":
            rms = float(np.sqrt(np.mean(r * r))) if r.size else 0.0
        relterm = 0.0 if kind == "norel" else rel * (r if kind == "noabs" else np.abs(r))
        bound = relterm + rms_tol * rms
        d = np.abs(g - r)
        with np.errstate(invalid="ignore"):
            if kind == "nan":
                bad = d > bound
            elif kind == "strict":
                bad = ~(d < bound)
            else:
                bad = ~(d <= bound)
        return dict(ok=not bad.any(), worst=0.0, n_bad=int(bad.sum()), rms=rms, n=r.size, why="")
    report.__name__ = f"_report_{kind}"
    return report


def _bits_equal_as_floats(gpu, ref, what=""):
    g = M.bf16_to_f64(np.asarray(gpu, np.uint16)) if np.asarray(gpu).dtype == np.uint16 else gpu
    r = M.bf16_to_f64(np.asarray(ref, np.uint16)) if np.asarray(ref).dtype == np.uint16 else ref
    if np.shape(g) != np.shape(r) or not np.array_equal(g, r):
        raise AssertionError(what)


def _gates_absolute(gpu, ref, what=""):
    if not (np.abs(np.asarray(gpu) - np.asarray(ref)) <= C.GATE_RTOL).all():
        raise AssertionError(what)


COMPARE_MUTANTS = [
    ("tolerance_report", _report_variant("nan"), [lambda: CP.test_non_finite_gpu_values_fail(0x7FC0)]),
    ("tolerance_report", _report_variant("noabs"), [CP.test_relative_term_inside_and_outside]),
    ("tolerance_report", _report_variant("sample_rms"), [CP.test_part_of_an_output_uses_the_whole_tensors_rms]),
    ("tolerance_report", _report_variant("strict"), [CP.test_rms_term_inside_boundary_and_outside]),
    ("tolerance_report", _report_variant("norel"), [CP.test_rms_term_inside_boundary_and_outside]),
    ("assert_bits_equal", _bits_equal_as_floats, [CP.test_bit_equality]),
    ("assert_gates_close", _gates_absolute, [CP.test_gate_rule]),
]


@pytest.mark.parametrize("name,mutant,pins", COMPARE_MUTANTS,
                         ids=[f"{m[0]}-{m[1].__name__}" for m in COMPARE_MUTANTS])
def test_planted_comparator_mistake_is_caught(monkeypatch, name, mutant, pins):
    monkeypatch.setattr(C, name, mutant)
    if hasattr(O, name):
        monkeypatch.setattr(O, name, mutant)
    for pin in pins:
        # a pin fails by an assertion, or by a pytest.raises that saw nothing
        with pytest.raises((AssertionError, ValueError, pytest.fail.Exception)):
            pin()
