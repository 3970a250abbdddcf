"""Seeded synthetic inputs for the fused communication + GEMM operations.

This module is shared by the CPU oracle (``oracle/``) and the GPU path's tests and
benchmark.  It only draws random numbers and stores them in the dtypes the
operations consume; it performs none of the operations' arithmetic.

Every tensor is drawn from ``numpy.random.default_rng([variant, config, index])``
(PCG64) so that the oracle and the GPU see identical bytes:

* ``variant`` 0 = floating-point inputs, 1 = small-integer inputs (bf16 values in
  {-2..2}, fp32 partials in {-4..4}) for bit-exact checking.
* ``config`` names the workload (``CONFIGS`` below); ad-hoc test shapes use their
  own ids.
* ``index`` is the tensor's position in the draw order of its workload.

bf16 tensors are returned as ``uint16`` bit patterns, fp32 tensors as
``float32``.  Float draws are made in float64, narrowed to float32 by numpy and
to bfloat16 by torch's round-to-nearest-even conversion: this only defines the
inputs, so the double rounding is immaterial.  "N(0, s)" means standard
deviation s.

Matrix B of every GEMM is generated as the logical [K, N] matrix the workloads
describe.  The GPU entry points take B transposed ([N, K], K contiguous, the
layout of a linear layer's weight); callers transpose the bits, which is a pure
copy.

The five workloads are the data-parallel hot path of mKernel's fused kernels
(mKernel pages, page 1, "Die fuenf verschmolzenen Kerne" table): AllGather+GEMM,
GEMM+ReduceScatter, GEMM+AllReduce and MoE dispatch + grouped GEMM, each at one
GPU's share with peer ranks emulated by buffers.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import numpy as np
import torch

FLOAT = 0
INTEGER = 1


def _rng(variant: int, config: int, index: int) -> np.random.Generator:
    return np.random.default_rng([int(variant), int(config), int(index)])


def _to_bf16_bits(x: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def draw_bf16(variant: int, config: int, index: int, shape, dist: str,
              scale: float = 1.0) -> np.ndarray:
    """bf16 bit patterns of the given shape.

    dist: "normal" (N(0, scale)), "uniform" (U[-scale, scale]).  The integer
    variant ignores dist and draws uniformly from {-2, ..., 2}.
    """
    g = _rng(variant, config, index)
    if variant == INTEGER:
        x = g.integers(-2, 3, size=shape).astype(np.float64)
    elif dist == "normal":
        x = g.standard_normal(size=shape) * scale
    elif dist == "uniform":
        x = g.uniform(-scale, scale, size=shape)
    else:
        raise ValueError(f"unknown distribution {dist!r}")
    return _to_bf16_bits(x)


def draw_f32(variant: int, config: int, index: int, shape, scale: float = 1.0) -> np.ndarray:
    """fp32 values: N(0, scale), or integers in {-4..4} for the integer variant."""
    g = _rng(variant, config, index)
    if variant == INTEGER:
        return g.integers(-4, 5, size=shape).astype(np.float32)
    return (g.standard_normal(size=shape) * scale).astype(np.float32)


def draw_logits(variant: int, config: int, index: int, shape) -> np.ndarray:
    """Router logits, fp32 N(0, 1) in both variants (integer logits would tie)."""
    g = _rng(variant, config, index)
    return g.standard_normal(size=shape).astype(np.float32)


# --------------------------------------------------------------------------
# workload descriptions
# --------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    op: str
    config_id: int
    params: Dict[str, int]
    a_dist: str = "normal"
    a_scale: float = 1.0
    b_dist: str = "normal"
    b_scale: float = 0.02

    def flops(self, n_slots: Optional[int] = None) -> float:
        p = self.params
        if self.op == "ag_gemm":
            return 2.0 * p["world"] * p["m_s"] * p["n"] * p["k"]
        if self.op in ("gemm_rs", "gemm_ar"):
            return 2.0 * p["m"] * p["n"] * p["k"]
        if self.op == "moe":
            if n_slots is None:
                raise ValueError("MoE work depends on the routed slot count")
            return 2.0 * n_slots * p["H"] * p["N"]
        if self.op == "ring_attn":  # Q K^T and P V over every rank's keys
            return 4.0 * p["B"] * p["H"] * p["S_q"] * p["world"] * p["S_kv"] * p["D"]
        raise ValueError(self.op)


CONFIGS: Dict[str, Workload] = {
    # AllGather+GEMM, 4 emulated ranks: shards [128,256], B [256,256], U[-1,1].
    "ag_gemm_w4_512x256x256": Workload(
        "ag_gemm_w4_512x256x256", "ag_gemm", 0,
        dict(world=4, rank=0, m_s=128, n=256, k=256),
        a_dist="uniform", a_scale=1.0, b_dist="uniform", b_scale=1.0),
    # AllGather+GEMM, one rank of a TP MLP up-projection, 8 emulated ranks.
    "ag_gemm_w8_8192x3584x8192": Workload(
        "ag_gemm_w8_8192x3584x8192", "ag_gemm", 1,
        dict(world=8, rank=0, m_s=1024, n=3584, k=8192)),
    # GEMM+ReduceScatter, 8 emulated ranks, this rank owns rows 0..1023.
    "gemm_rs_w8_8192x8192x3584": Workload(
        "gemm_rs_w8_8192x8192x3584", "gemm_rs", 2,
        dict(world=8, rank=0, m=8192, n=8192, k=3584)),
    # GEMM+AllReduce, 8 emulated ranks, a K-shard of 1024 of 8192, 7 broadcast copies.
    "gemm_ar_w8_2048x8192x1024": Workload(
        "gemm_ar_w8_2048x8192x1024", "gemm_ar", 3,
        dict(world=8, rank=0, m=2048, n=8192, k=1024, n_bcast=7)),
    # MoE dispatch + grouped GEMM: 8 sources x 4096 tokens, 64 experts, top-2, 8 local.
    "moe_s8_t4096_h4096_n1536_e64": Workload(
        "moe_s8_t4096_h4096_n1536_e64", "moe", 4,
        dict(S=8, T=4096, H=4096, N=1536, E=64, E_loc=8, top_k=2, rank=0)),
    # Ring attention (the pages give no shape): a 32768-token sequence over 8
    # ranks, 4096 local queries and 4096 keys per block, 32 heads of 128.
    "ring_attn_w8_h32_s4096_d128": Workload(
        "ring_attn_w8_h32_s4096_d128", "ring_attn", 5,
        dict(world=8, rank=0, B=1, H=32, S_q=4096, S_kv=4096, D=128)),
}


# --------------------------------------------------------------------------
# generators: the tensor draw order below is part of the input definition
# --------------------------------------------------------------------------

def gen_ag(world: int, m_s: int, n: int, k: int, variant: int = FLOAT, config: int = 1,
           a_dist: str = "normal", a_scale: float = 1.0,
           b_dist: str = "normal", b_scale: float = 0.02) -> Dict[str, object]:
    """AllGather+GEMM inputs: tensors 0..W-1 are the shards [m_s, k], W is B [k, n]."""
    shards = [draw_bf16(variant, config, q, (m_s, k), a_dist, a_scale) for q in range(world)]
    b = draw_bf16(variant, config, world, (k, n), b_dist, b_scale)
    return dict(shards=shards, b=b)


def gen_rs(world: int, m: int, n: int, k: int, rank: int = 0, variant: int = FLOAT,
           config: int = 2, a_scale: float = 1.0, b_scale: float = 0.02) -> Dict[str, object]:
    """GEMM+ReduceScatter inputs: 0 = A [m,k], 1 = B [k,n], 2.. = the W-1 peer
    partials of this rank's slice, each [m/W, n] fp32, in ascending peer rank."""
    if m % world:
        raise ValueError("m must be a multiple of the world size")
    a = draw_bf16(variant, config, 0, (m, k), "normal", a_scale)
    b = draw_bf16(variant, config, 1, (k, n), "normal", b_scale)
    peers: List[Optional[np.ndarray]] = []
    idx = 2
    for q in range(world):
        if q == rank:
            peers.append(None)
        else:
            peers.append(draw_f32(variant, config, idx, (m // world, n)))
            idx += 1
    return dict(a=a, b=b, peers=peers)


def gen_ar(world: int, m: int, n: int, k: int, rank: int = 0, variant: int = FLOAT,
           config: int = 3, a_scale: float = 1.0, b_scale: float = 0.02) -> Dict[str, object]:
    """GEMM+AllReduce inputs: 0 = A [m,k], 1 = B [k,n], 2.. = the W-1 peer
    partials, each [m, n] fp32, in ascending peer rank."""
    a = draw_bf16(variant, config, 0, (m, k), "normal", a_scale)
    b = draw_bf16(variant, config, 1, (k, n), "normal", b_scale)
    peers: List[Optional[np.ndarray]] = []
    idx = 2
    for q in range(world):
        if q == rank:
            peers.append(None)
        else:
            peers.append(draw_f32(variant, config, idx, (m, n)))
            idx += 1
    return dict(a=a, b=b, peers=peers)


def gen_moe(S: int, T: int, H: int, N: int, E: int, E_loc: int, variant: int = FLOAT,
            config: int = 4, x_scale: float = 1.0, w_scale: float = 0.02, top_k: int = 2,
            y_scale: float = 0.05) -> Dict[str, object]:
    """MoE inputs: 0..S-1 = tokens x_s [T,H] bf16, S..2S-1 = logits_s [T,E] fp32,
    2S = expert weights W [E_loc, H, N] bf16 (logical [K, N] per expert),
    2S+1 = y_peer [T, top_k=2, N] bf16: the gated expert rows the peers return
    for this rank's tokens in the combine (standard deviation y_scale, about
    that of gate * x @ W at these scales)."""
    xs = [draw_bf16(variant, config, s, (T, H), "normal", x_scale) for s in range(S)]
    logits = [draw_logits(variant, config, S + s, (T, E)) for s in range(S)]
    w = draw_bf16(variant, config, 2 * S, (E_loc, H, N), "normal", w_scale)
    y_peer = draw_bf16(variant, config, 2 * S + 1, (T, top_k, N), "normal", y_scale)
    return dict(x=xs, logits=logits, w=w, y_peer=y_peer)


def gen_ring(W: int, B: int, H: int, S_q: int, S_kv: int, D: int, config: int = 5,
             scale: float = 1.0) -> Dict[str, object]:
    """Ring attention inputs: 0 = queries q [B,H,S_q,D] bf16, 1..W = keys of
    rank r (k_src[r]) [B,H,S_kv,D], W+1..2W = values of rank r; all N(0, scale).
    Only the float variant exists: softmax weights are never exact."""
    q = draw_bf16(FLOAT, config, 0, (B, H, S_q, D), "normal", scale)
    ks = [draw_bf16(FLOAT, config, 1 + r, (B, H, S_kv, D), "normal", scale) for r in range(W)]
    vs = [draw_bf16(FLOAT, config, 1 + W + r, (B, H, S_kv, D), "normal", scale) for r in range(W)]
    return dict(q=q, k=ks, v=vs)


def gen_workload(name: str, variant: int = FLOAT) -> Dict[str, object]:
    wl = CONFIGS[name]
    p = wl.params
    if wl.op == "ag_gemm":
        return gen_ag(p["world"], p["m_s"], p["n"], p["k"], variant, wl.config_id,
                      wl.a_dist, wl.a_scale, wl.b_dist, wl.b_scale)
    if wl.op == "gemm_rs":
        return gen_rs(p["world"], p["m"], p["n"], p["k"], p["rank"], variant, wl.config_id)
    if wl.op == "gemm_ar":
        return gen_ar(p["world"], p["m"], p["n"], p["k"], p["rank"], variant, wl.config_id)
    if wl.op == "moe":
        return gen_moe(p["S"], p["T"], p["H"], p["N"], p["E"], p["E_loc"], variant,
                       wl.config_id, top_k=p["top_k"])
    if wl.op == "ring_attn":
        return gen_ring(p["world"], p["B"], p["H"], p["S_q"], p["S_kv"], p["D"], wl.config_id)
    raise ValueError(wl.op)


def transpose_bits(b: np.ndarray) -> np.ndarray:
    """[..., K, N] -> [..., N, K] contiguous copy of bit patterns (no arithmetic)."""
    return np.ascontiguousarray(np.swapaxes(b, -1, -2))
