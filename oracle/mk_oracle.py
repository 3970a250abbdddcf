"""CPU oracle for the fused communication + GEMM operations -- TEST INFRASTRUCTURE.

This module is the plain, slow, obviously correct definition that the GPU path
is checked against.  Only the tests, the smoke check and the benchmark's CPU
baseline may import it; the product path never does, and it shares no code
with the HIP library (only the seeded input generators are common).

Sources are cited by page and section:

* [P1] the German article on mKernel (chatgpz.de), the table "Die fuenf
  verschmolzenen Kerne" (the five fused kernels), one row per kernel.
* [P3] the Romanian article (world.tibi.club), section "Cum functioneaza? O
  privire sub capota" (reduce, broadcast and scatter fused in one kernel).

Numerics.  All arithmetic is float64.  A product of two bf16 values is exact in
float64 and a sum of K of them carries a relative error of at most about
K * 2**-53, far below the bf16 output rounding; results are rounded once to
bf16 with round-to-nearest-even.  The workloads accumulate in fp32 on the GPU;
for integer-valued inputs every partial sum is an integer below 2**24, so both
precisions are exact and the bf16 outputs must agree bit for bit.

Readings of points the pages leave open (each also listed in the design notes):

* r1  the local rank is 0 unless given; peers are the other ranks.
* r2  the gathered matrix concatenates the shards by rank (row block q = shard q).
* r3  every output is bf16, rounded once from the exact/float64 result (RNE).
* r4  the peer partials of GEMM+ReduceScatter cover only this rank's row slice.
* r5  the ReduceScatter outbox for peer q holds bf16 of this rank's unreduced
      partial rows of slice q.
* r6  GEMM+AllReduce writes the reduced result to the output and to every
      broadcast buffer, bit-identical.
* r7  "softmax top-2": softmax over all experts' logits; the two experts with
      the largest logits are chosen (ties -> lower expert id), in descending
      order; their softmax probabilities are the gates, not renormalised.
* r8  local experts are rank*E_loc ... rank*E_loc + E_loc - 1; slots are ordered
      by (local expert, source rank, token); there is no capacity limit and no
      token is dropped.
* r9  the expert output is y[slot] = bf16(gate * (x @ W_e)); an ungated variant
      (gate applied later, in the combine) gives bf16(x @ W_e).
* r10 (combine; the pages describe the dispatch only) each output row of this
      rank's experts returns to its source at (token, k), k being the
      expert's place in the token's top-k list; a source's combined row is
      the bf16 of the sum over k of its returned rows (gates already applied).
* r11 (ring attention; the pages give one sentence) the local queries attend
      to the keys and values of every rank's block: full (non-causal)
      softmax attention over their concatenation, scores scaled by a given
      factor (1/sqrt(D) by default); block s of the ring is the one that
      started on rank (rank - s) mod W; the order affects rounding only.
      Outputs: o = bf16(softmax(Q K^T scale) V) and the log of each row's
      softmax denominator, lse = max + log(sum exp(s - max)), unrounded.

Parity is pinned (tests marked "not gpu"): bf16 rounding by exhaustive and
brute-force nearest-value search; the GEMM by exact rational brute force on
tiny shapes and by identity / unit-vector special cases; the gather order by
B = I; ReduceScatter by a W-rank emulation whose slices must tile the full
sum; AllReduce by its equivalence to ReduceScatter followed by a gather; MoE
routing by a brute-force sort and the dispatch permutation by its inverse;
the MoE combine by its return permutation and exact-gate examples; ring
attention by closed forms (zero queries, equal values, one key), the
invariance of the result to the ring order and to splitting heads, the
scale acting as a factor on the queries; and hand-worked examples under
tests/golden.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence

import numpy as np

# --------------------------------------------------------------------------
# bf16 <-> float (own helpers; no library bf16 type is used here)
# --------------------------------------------------------------------------


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Decode bf16 bit patterns: a bf16 is the upper half of an fp32 (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def f32_to_bf16(x32: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 with round-to-nearest-even on the bit pattern.

    Adding 0x7FFF plus the lowest kept bit and truncating rounds to nearest
    with ties to even; NaNs stay quiet NaNs.
    """
    x32 = np.ascontiguousarray(x32, dtype=np.float32)
    u = x32.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)
    nan = np.isnan(x32)
    if nan.any():
        r = np.where(nan, ((u >> np.uint64(16)).astype(np.uint16) | np.uint16(0x0040)), r)
    return r.astype(np.uint16)


def f64_to_bf16(x: np.ndarray) -> np.ndarray:
    """float64 -> bf16, correctly rounded to nearest even.

    Two steps: round to fp32 with round-to-odd (truncate toward zero, then set
    the last bit if anything was discarded), then round that to bf16 to nearest
    even.  Because fp32 keeps more than two bits beyond bf16's precision, the
    pair gives the same result as one direct rounding (Boldo & Melquiond,
    "Emulation of FMA and correctly rounded sums: proved algorithms using
    rounding to odd", 2008).
    """
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore", invalid="ignore"):
        f = x.astype(np.float32)
        away = np.abs(f.astype(np.float64)) > np.abs(x)
        f = np.where(away, np.nextafter(f, np.float32(0.0)), f).astype(np.float32)
        inexact = (f.astype(np.float64) != x) & ~np.isnan(x)
    bits = f.view(np.uint32).copy()
    bits[inexact] |= np.uint32(1)
    return f32_to_bf16(bits.view(np.float32))


# --------------------------------------------------------------------------
# dense product (the GEMM inside every fused kernel)
# --------------------------------------------------------------------------


def gemm(a_bits: np.ndarray, b_bits: np.ndarray) -> np.ndarray:
    """P = A @ B for bf16 A [M,K] and B [K,N], computed in float64 (unrounded).

    [P1] every GEMM row of the five-kernel table computes C = A @ B.  The
    matrix product is numpy's float64 matmul used as a library step.
    """
    a = bf16_to_f64(a_bits)
    b = bf16_to_f64(b_bits)
    if a.ndim != 2 or b.ndim != 2 or a.shape[1] != b.shape[0]:
        raise ValueError(f"bad GEMM shapes {a.shape} @ {b.shape}")
    return a @ b


# --------------------------------------------------------------------------
# AllGather + GEMM
# --------------------------------------------------------------------------


def all_gather(shards: Sequence[np.ndarray]) -> np.ndarray:
    """Concatenate the ranks' shards by rank (reading r2): bit copy."""
    return np.concatenate([np.asarray(s, dtype=np.uint16) for s in shards], axis=0)


def ag_gemm(shards: Sequence[np.ndarray], b_bits: np.ndarray) -> Dict[str, np.ndarray]:
    """[P1] AllGather + GEMM: every rank holds one shard of A; the shards are
    gathered and the GEMM runs on the full A.  C = bf16(gather(A) @ B)."""
    a_full = all_gather(shards)
    return dict(c=f64_to_bf16(gemm(a_full, b_bits)), a_gathered=a_full)


def ag_gemm_rows(shards: Sequence[np.ndarray], b_bits: np.ndarray,
                 rows: np.ndarray) -> np.ndarray:
    """Rows `rows` of ag_gemm's C, computed one by one from the shards."""
    m_s = shards[0].shape[0]
    a_rows = np.stack([shards[int(r) // m_s][int(r) % m_s] for r in rows])
    return f64_to_bf16(gemm(a_rows, b_bits))


# --------------------------------------------------------------------------
# GEMM + ReduceScatter
# --------------------------------------------------------------------------


def _sum_partials(own: np.ndarray, peers: Sequence[Optional[np.ndarray]], rank: int) -> np.ndarray:
    """own + sum of the peer partials, own first then ascending peer rank."""
    acc = np.array(own, dtype=np.float64, copy=True)
    for q, p in enumerate(peers):
        if q == rank:
            continue
        acc = acc + np.asarray(p, dtype=np.float64)
    return acc


def gemm_rs(a_bits: np.ndarray, b_bits: np.ndarray, peers: Sequence[Optional[np.ndarray]],
            rank: int = 0) -> Dict[str, object]:
    """[P1] GEMM + ReduceScatter: C = A @ B, the output is reduced over ranks and
    each output slice goes to the rank that owns it.

    With W = len(peers) ranks and M rows, slice q is rows [q*M/W, (q+1)*M/W).
    This rank keeps c_own = bf16(P[slice rank] + sum of the peers' partials of
    that slice) (reading r4) and sends outbox[q] = bf16(P[slice q]) to every
    other rank q (reading r5).
    """
    world = len(peers)
    p = gemm(a_bits, b_bits)
    m = p.shape[0]
    if m % world:
        raise ValueError("M must be a multiple of the world size")
    ms = m // world
    own = p[rank * ms:(rank + 1) * ms]
    c_own = f64_to_bf16(_sum_partials(own, peers, rank))
    outbox: List[Optional[np.ndarray]] = []
    for q in range(world):
        outbox.append(None if q == rank else f64_to_bf16(p[q * ms:(q + 1) * ms]))
    return dict(c_own=c_own, outbox=outbox)


def gemm_rs_rows(a_bits: np.ndarray, b_bits: np.ndarray, peers: Sequence[Optional[np.ndarray]],
                 rank: int, rows: np.ndarray) -> np.ndarray:
    """Rows of the full [M, N] bf16 result layout: rows in slice `rank` give
    c_own rows, rows in another slice q give outbox[q] rows."""
    world = len(peers)
    m = a_bits.shape[0]
    ms = m // world
    p = gemm(np.asarray(a_bits)[np.asarray(rows)], b_bits)
    out = np.empty(p.shape, dtype=np.uint16)
    for i, r in enumerate(rows):
        q = int(r) // ms
        if q == rank:
            acc = _sum_partials(p[i], [None if pp is None else pp[int(r) - q * ms]
                                       for pp in peers], rank)
            out[i] = f64_to_bf16(acc)
        else:
            out[i] = f64_to_bf16(p[i])
    return out


# --------------------------------------------------------------------------
# GEMM + AllReduce
# --------------------------------------------------------------------------


def gemm_ar(a_bits: np.ndarray, b_bits: np.ndarray, peers: Sequence[Optional[np.ndarray]],
            rank: int = 0, n_bcast: int = 0) -> Dict[str, object]:
    """[P1] GEMM + AllReduce: C = A @ B with the partial outputs of all ranks
    summed; [P3] reduce and broadcast in one kernel.

    c = bf16(P + sum of the peers' full partials); every broadcast buffer holds
    a copy of c (reading r6).
    """
    p = gemm(a_bits, b_bits)
    c = f64_to_bf16(_sum_partials(p, peers, rank))
    return dict(c=c, bcast=[c.copy() for _ in range(n_bcast)])


def gemm_ar_rows(a_bits: np.ndarray, b_bits: np.ndarray, peers: Sequence[Optional[np.ndarray]],
                 rank: int, rows: np.ndarray) -> np.ndarray:
    rows = np.asarray(rows)
    p = gemm(np.asarray(a_bits)[rows], b_bits)
    sub = [None if pp is None else np.asarray(pp)[rows] for pp in peers]
    return f64_to_bf16(_sum_partials(p, sub, rank))


# --------------------------------------------------------------------------
# MoE dispatch + grouped GEMM
# --------------------------------------------------------------------------


def moe_route(logits: np.ndarray, top_k: int) -> Dict[str, np.ndarray]:
    """Top-k routing of tokens over experts (reading r7).

    logits: [n_tokens, E] fp32.  The experts are sorted by logit descending with
    the lower id first among equal logits (a stable sort of the negated
    logits), and the first top_k are taken.  The gates are the softmax over all
    E logits, evaluated in float64, at the chosen experts.
    """
    lg = np.asarray(logits, dtype=np.float32)
    order = np.argsort(-lg, axis=1, kind="stable")
    idx = order[:, :top_k].astype(np.int32)
    l64 = lg.astype(np.float64)
    mx = l64.max(axis=1, keepdims=True)
    ex = np.exp(l64 - mx)
    prob = ex / ex.sum(axis=1, keepdims=True)
    gate = np.take_along_axis(prob, idx.astype(np.int64), axis=1)
    return dict(idx=idx, gate=gate, prob=prob)


def moe_dispatch(idx: np.ndarray, gate: np.ndarray, S: int, T: int, E_loc: int,
                 rank: int = 0) -> Dict[str, np.ndarray]:
    """Assign the (token, expert) pairs routed to this rank's experts to slots.

    [P1] MoE dispatch: tokens are sent to the ranks that own their experts and
    land in per-expert slots.  Slots are ordered by (local expert, source rank,
    token) (reading r8).  Returns slot_token (= s*T + t), slot_gate,
    expert_offsets [E_loc+1] and chunk_offsets [E_loc, S+1], where
    chunk_offsets[e, s] is the first slot of source s's tokens for local expert
    e and chunk_offsets[e, S] = expert_offsets[e+1].
    """
    idx = np.asarray(idx)
    slot_token: List[int] = []
    slot_gate: List[float] = []
    expert_offsets = np.zeros(E_loc + 1, dtype=np.int32)
    chunk_offsets = np.zeros((E_loc, S + 1), dtype=np.int32)
    for e in range(E_loc):
        g = rank * E_loc + e
        expert_offsets[e] = len(slot_token)
        for s in range(S):
            chunk_offsets[e, s] = len(slot_token)
            sel = idx[s * T:(s + 1) * T]
            tok, j = np.nonzero(sel == g)          # ascending token order
            for t, jj in zip(tok.tolist(), j.tolist()):
                slot_token.append(s * T + t)
                slot_gate.append(float(gate[s * T + t, jj]))
        chunk_offsets[e, S] = len(slot_token)
    expert_offsets[E_loc] = len(slot_token)
    return dict(slot_token=np.array(slot_token, dtype=np.int32),
                slot_gate=np.array(slot_gate, dtype=np.float64),
                expert_offsets=expert_offsets, chunk_offsets=chunk_offsets)


def slot_expert(expert_offsets: np.ndarray, n_slots: int) -> np.ndarray:
    """Local expert id of every slot."""
    e = np.zeros(n_slots, dtype=np.int64)
    for i in range(len(expert_offsets) - 1):
        e[expert_offsets[i]:expert_offsets[i + 1]] = i
    return e


def moe_dispatch_gemm(x: Sequence[np.ndarray], logits: Sequence[np.ndarray], w: np.ndarray,
                      top_k: int, rank: int = 0, apply_gate: bool = True,
                      slots: Optional[np.ndarray] = None) -> Dict[str, np.ndarray]:
    """[P1] MoE dispatch + GEMM: route tokens to their experts, land them in
    per-expert slots and run each expert's GEMM on its slots.

    x: S arrays [T, H] bf16; logits: S arrays [T, E] fp32; w: [E_loc, H, N] bf16.
    y[slot] = bf16(gate * (x_s[t] @ W_e)) (reading r9).  If `slots` is given,
    y is computed only for those slot indices (rows of the result).
    """
    S = len(x)
    T = x[0].shape[0]
    E_loc = w.shape[0]
    route = moe_route(np.concatenate([np.asarray(l) for l in logits], axis=0), top_k)
    d = moe_dispatch(route["idx"], route["gate"], S, T, E_loc, rank)
    n_slots = int(d["expert_offsets"][-1])
    x_all = np.concatenate([np.asarray(xx, dtype=np.uint16) for xx in x], axis=0)
    x_slots = x_all[d["slot_token"]]
    sel = np.arange(n_slots) if slots is None else np.asarray(slots)
    exp_of = slot_expert(d["expert_offsets"], n_slots)
    y = np.zeros((len(sel), w.shape[2]), dtype=np.uint16)
    for e in range(E_loc):
        rows = np.nonzero(exp_of[sel] == e)[0]
        if rows.size == 0:
            continue
        p = gemm(x_slots[sel[rows]], w[e])
        if apply_gate:
            p = p * d["slot_gate"][sel[rows]][:, None]
        y[rows] = f64_to_bf16(p)
    out = dict(route, **d)
    out.update(x_slots=x_slots, y=y, n_slots=n_slots)
    return out


def moe_y_given_gates(x_slots: np.ndarray, w: np.ndarray, expert_offsets: np.ndarray,
                      gates_f32: np.ndarray) -> np.ndarray:
    """Expert outputs recomputed with given fp32 gates, for a bit-exact check
    of the gated output on integer-valued inputs (reading of the integer
    variant: the gate a kernel computed is taken as an input).

    y[slot] = bf16(fp32(gate[slot] * acc)), acc = x_slots[slot] @ W_e: the
    gate multiply is one fp32 multiply (rounded to nearest even in fp32), then
    the product is rounded to bf16.  With integer-valued bf16 inputs whose
    products sum below 2**24 in magnitude, acc is an exact integer in fp32 and
    in float64, so the float64 product of the fp32 gate and acc is exact and
    its fp32 rounding is the kernel's.  Returns [n_slots, N] bf16 bits.
    """
    n_slots = int(expert_offsets[-1])
    g = np.asarray(gates_f32, dtype=np.float32)[:n_slots].astype(np.float64)
    y = np.zeros((n_slots, w.shape[2]), dtype=np.uint16)
    for e in range(w.shape[0]):
        lo, hi = int(expert_offsets[e]), int(expert_offsets[e + 1])
        if hi <= lo:
            continue
        acc = gemm(np.asarray(x_slots)[lo:hi], w[e])
        if np.abs(acc).max(initial=0.0) >= 2.0 ** 24 or not np.array_equal(acc, np.round(acc)):
            raise ValueError("the accumulator is not an exact integer below 2**24")
        y[lo:hi] = f32_to_bf16((g[lo:hi, None] * acc).astype(np.float32))
    return y


# --------------------------------------------------------------------------
# MoE combine (completes the MoE layer after dispatch + grouped GEMM)
# --------------------------------------------------------------------------


def moe_return_positions(slot_token: np.ndarray, idx: np.ndarray, expert_offsets: np.ndarray,
                         T: int, top_k: int, E_loc: int, rank: int) -> np.ndarray:
    """For every slot of this rank, the position s*T*top_k + t*top_k + k its
    output row returns to: source s = slot_token // T, token t, and k the
    place of the slot's expert in the token's top-k list (reading r10)."""
    n = len(slot_token)
    exp_of = slot_expert(expert_offsets, n)
    pos = np.zeros(n, dtype=np.int64)
    for slot in range(n):
        st = int(slot_token[slot])
        g = rank * E_loc + int(exp_of[slot])
        ks = np.nonzero(np.asarray(idx[st]) == g)[0]
        assert ks.size == 1, "a slot's expert appears once in its token's top-k list"
        pos[slot] = st * top_k + int(ks[0])
    return pos


def moe_combine(x: Sequence[np.ndarray], logits: Sequence[np.ndarray], w: np.ndarray,
                top_k: int, y_peer: np.ndarray, rank: int = 0,
                tokens: Optional[np.ndarray] = None) -> Dict[str, np.ndarray]:
    """[P1] MoE layer of one rank: dispatch + grouped GEMM (moe_dispatch_gemm),
    then the combine of reading r10.

    Every output row y[slot] of this rank's experts returns to its source s at
    position (t, k), k being the slot's expert's place in token t's top-k list:
    ret[s] is [T, top_k, N] bf16 with ret_mask[s] [T, top_k] marking the rows
    this rank writes (its own experts' pairs).  For this rank's own tokens,
    out[t] = bf16(sum over k of v_k), v_k = y[slot] when expert k of token t is
    local and y_peer[t, k] (the row its owner returned) otherwise; the gate is
    already in the rows, the sum runs over k in float64 and rounds once.

    With `tokens` (a sample of this rank's token indices, for large sizes) only
    those tokens are combined: out is [len(tokens), N], y holds the rows of the
    slots they use (their indices in "slots"), and ret / ret_mask are not built.
    """
    S = len(x)
    T = x[0].shape[0]
    E_loc, N = w.shape[0], w.shape[2]
    assert 0 <= rank < S, "this rank's own tokens are source `rank`"
    if tokens is not None:
        return _moe_combine_sampled(x, logits, w, top_k, y_peer, rank, np.asarray(tokens))
    d = moe_dispatch_gemm(x, logits, w, top_k, rank)
    pos = moe_return_positions(d["slot_token"], d["idx"], d["expert_offsets"], T, top_k, E_loc, rank)
    ret = np.zeros((S, T, top_k, N), dtype=np.uint16)
    ret_mask = np.zeros((S, T, top_k), dtype=bool)
    flat = ret.reshape(S * T * top_k, N)
    flat[pos] = d["y"]
    ret_mask.reshape(-1)[pos] = True
    yp = np.asarray(y_peer, dtype=np.uint16).reshape(T, top_k, N)
    rows = np.where(ret_mask[rank][:, :, None], ret[rank], yp)
    out = f64_to_bf16(bf16_to_f64(rows).sum(axis=1))
    res = dict(d)
    res.update(ret=ret, ret_mask=ret_mask, out=out, return_pos=pos)
    return res


def _moe_combine_sampled(x, logits, w, top_k, y_peer, rank, tokens):
    """moe_combine restricted to some of this rank's tokens: the same steps,
    with the expert GEMM run only on the slots those tokens use."""
    T = x[0].shape[0]
    E_loc, N = w.shape[0], w.shape[2]
    d0 = moe_dispatch_gemm(x, logits, w, top_k, rank, slots=np.zeros(0, dtype=np.int64))
    pos = moe_return_positions(d0["slot_token"], d0["idx"], d0["expert_offsets"], T, top_k,
                               E_loc, rank)
    want = set(int(rank * T + t) for t in tokens)
    slots = np.array([i for i, st in enumerate(d0["slot_token"]) if int(st) in want],
                     dtype=np.int64)
    d = moe_dispatch_gemm(x, logits, w, top_k, rank, slots=slots)
    yp = np.asarray(y_peer, dtype=np.uint16).reshape(T, top_k, N)
    rows = yp[tokens].copy()                      # [n, top_k, N]
    where = {int(pos[sl]): i for i, sl in enumerate(slots)}
    for r, t in enumerate(tokens):
        for k in range(top_k):
            i = where.get(int((rank * T + t) * top_k + k))
            if i is not None:
                rows[r, k] = d["y"][i]
    out = f64_to_bf16(bf16_to_f64(rows).sum(axis=1))
    res = dict(d)
    res.update(out=out, return_pos=pos, slots=slots)
    return res


# --------------------------------------------------------------------------
# Ring attention
# --------------------------------------------------------------------------


def ring_order(world: int, rank: int) -> List[int]:
    """[P1] ring attention row: at step s a rank holds the KV block that
    started on rank (rank - s) mod W, the previous step's block having moved
    one rank along the ring (reading r11)."""
    return [(rank - s) % world for s in range(world)]


def ring_attention(q: np.ndarray, k_src: Sequence[np.ndarray], v_src: Sequence[np.ndarray],
                   rank: int = 0, scale: Optional[float] = None,
                   rows: Optional[np.ndarray] = None) -> Dict[str, np.ndarray]:
    """[P1] table "Die fuenf verschmolzenen Kerne", ring attention row:
    sequence-parallel attention of this rank's queries over every rank's
    keys and values, the blocks taken in ring order (reading r11).

    q: [B, H, S_q, D] bf16; k_src, v_src: W arrays [B, H, S_kv, D] bf16 (block
    of rank r).  scale defaults to 1/sqrt(D).  rows (optional) restricts the
    queries to those row indices (for sampled checks at large sizes).
    Returns o [B, H, R, D] bf16, o_f64 (unrounded), lse [B, H, R] float64, the
    ring order, and k_recv / v_recv [W, B, H, S_kv, D]: every block by source
    rank, as landed.
    """
    W = len(k_src)
    B, H, S_q, D = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    order = ring_order(W, rank)
    sel = np.arange(S_q) if rows is None else np.asarray(rows)
    o = np.zeros((B, H, len(sel), D))
    lse = np.zeros((B, H, len(sel)))
    for b in range(B):
        for h in range(H):
            k = np.concatenate([bf16_to_f64(np.asarray(k_src[r])[b, h]) for r in order], axis=0)
            v = np.concatenate([bf16_to_f64(np.asarray(v_src[r])[b, h]) for r in order], axis=0)
            qq = bf16_to_f64(np.asarray(q)[b, h][sel])
            s = (qq @ k.T) * float(scale)                 # [R, S_total]
            m = s.max(axis=1, keepdims=True)
            p = np.exp(s - m)
            den = p.sum(axis=1, keepdims=True)
            o[b, h] = (p @ v) / den
            lse[b, h] = (m + np.log(den))[:, 0]
    return dict(o=f64_to_bf16(o), o_f64=o, lse=lse, order=np.array(order),
                k_recv=np.stack([np.asarray(x, dtype=np.uint16) for x in k_src]),
                v_recv=np.stack([np.asarray(x, dtype=np.uint16) for x in v_src]))
