"""Comparison rules between GPU outputs and the oracle -- TEST INFRASTRUCTURE.

Float outputs (bf16): elementwise |gpu - ref| <= 1e-2*|ref| + 1e-2*rms(ref),
both sides decoded from bf16 to float64, where rms(ref) = sqrt(mean(ref^2))
is taken over the WHOLE reference output tensor.  A caller that compares a
part of an output passes the whole tensor's rms (rms_of(full_ref_bits));
otherwise the compared array is taken to be the whole output.  A NaN or an
infinity on the GPU side never passes; the oracle never produces either, so a
non-finite reference value is an error of the test itself.

Integer-valued inputs and all routing / permutation indices: bit equality
(the arrays' values, compared in their own integer type).

MoE gates (fp32): |gpu - ref| <= 1e-5 * ref.  Ring attention log-sum-exp
(fp32): |gpu - ref| <= 1e-3 + 1e-4 * |ref|.
"""
from __future__ import annotations

from typing import Dict, Optional

import numpy as np

from .mk_oracle import bf16_to_f64

REL_TOL = 1e-2
RMS_TOL = 1e-2
GATE_RTOL = 1e-5
LSE_ATOL = 1e-3
LSE_RTOL = 1e-4


def rms_of(ref_bits: np.ndarray) -> float:
    """Root-mean-square of a bf16 reference tensor (float64, whole array)."""
    r = bf16_to_f64(np.asarray(ref_bits, dtype=np.uint16))
    if r.size == 0:
        return 0.0
    if not np.isfinite(r).all():
        raise ValueError("the reference holds a non-finite value")
    return float(np.sqrt(np.mean(r * r)))


def tolerance_report(gpu_bits: np.ndarray, ref_bits: np.ndarray, rms: Optional[float] = None,
                     rel: float = REL_TOL, rms_tol: float = RMS_TOL) -> Dict[str, float]:
    """Check the float rule elementwise.  rms: the whole reference tensor's
    rms; None means ref_bits is the whole tensor."""
    g = bf16_to_f64(np.asarray(gpu_bits, dtype=np.uint16))
    r = bf16_to_f64(np.asarray(ref_bits, dtype=np.uint16))
    if g.shape != r.shape:
        return dict(ok=False, worst=float("inf"), n_bad=-1, rms=float("nan"), n=int(r.size),
                    why=f"shape mismatch {g.shape} vs {r.shape}")
    if not np.isfinite(r).all():
        raise ValueError("the reference holds a non-finite value")
    if rms is None:
        rms = rms_of(ref_bits)
    if r.size == 0:
        return dict(ok=True, worst=0.0, n_bad=0, rms=float(rms), n=0, why="")
    bound = rel * np.abs(r) + rms_tol * float(rms)
    with np.errstate(invalid="ignore"):
        d = np.abs(g - r)
        good = np.isfinite(g) & (d <= bound)
        ratio = np.where(bound > 0, d / np.maximum(bound, 1e-300), np.where(d > 0, np.inf, 0.0))
    ratio = np.where(np.isfinite(g), ratio, np.inf)
    n_bad = int((~good).sum())
    return dict(ok=n_bad == 0, worst=float(np.max(ratio)), n_bad=n_bad, rms=float(rms),
                n=int(r.size), why="")


def assert_close_bf16(gpu_bits: np.ndarray, ref_bits: np.ndarray, what: str = "",
                      rms: Optional[float] = None) -> None:
    rep = tolerance_report(gpu_bits, ref_bits, rms=rms)
    if rep["ok"]:
        return
    if rep["why"]:
        raise AssertionError(f"{what}: {rep['why']}")
    g = bf16_to_f64(np.asarray(gpu_bits, dtype=np.uint16))
    r = bf16_to_f64(np.asarray(ref_bits, dtype=np.uint16))
    with np.errstate(invalid="ignore"):
        good = np.isfinite(g) & (np.abs(g - r) <= REL_TOL * np.abs(r) + RMS_TOL * rep["rms"])
    bad = np.argwhere(~good)
    first = [tuple(int(v) for v in b) for b in bad[:5]]
    vals = [(g[tuple(b)], r[tuple(b)]) for b in bad[:5]]
    raise AssertionError(f"{what}: {rep['n_bad']} of {rep['n']} elements outside tolerance "
                         f"(rms {rep['rms']:.4g}); first at {first}: gpu/ref {vals}")


def assert_bits_equal(gpu: np.ndarray, ref: np.ndarray, what: str = "") -> None:
    """Bit equality of integer arrays (bf16 patterns, indices, offsets)."""
    g = np.asarray(gpu)
    r = np.asarray(ref)
    if g.shape != r.shape:
        raise AssertionError(f"{what}: shape {g.shape} != {r.shape}")
    if g.dtype.kind not in "iub" or r.dtype.kind not in "iub":
        raise AssertionError(f"{what}: bit equality compares integer arrays "
                             f"(got {g.dtype} and {r.dtype})")
    if g.dtype != r.dtype:
        r2 = r.astype(g.dtype)
        if not np.array_equal(r2.astype(r.dtype), r):
            raise AssertionError(f"{what}: reference values do not fit {g.dtype}")
        r = r2
    ne = np.argwhere(g != r)
    if ne.size:
        first = [tuple(int(v) for v in b) for b in ne[:5]]
        vals = [(g[tuple(b)], r[tuple(b)]) for b in ne[:5]]
        raise AssertionError(f"{what}: {len(ne)} of {g.size} elements differ; first at "
                             f"{first}: gpu/ref {vals}")


def assert_gates_close(gpu: np.ndarray, ref: np.ndarray, what: str = "topk_gate") -> None:
    """MoE gates: |gpu - ref| <= GATE_RTOL * ref elementwise (ref > 0)."""
    g = np.asarray(gpu, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    if g.shape != r.shape:
        raise AssertionError(f"{what}: shape {g.shape} != {r.shape}")
    with np.errstate(invalid="ignore"):
        bad = ~(np.abs(g - r) <= GATE_RTOL * np.abs(r))
    if bad.any():
        i = tuple(int(v) for v in np.argwhere(bad)[0])
        raise AssertionError(f"{what}: {int(bad.sum())} of {g.size} outside {GATE_RTOL} relative; "
                             f"first at {i}: gpu/ref {g[i]} {r[i]}")


def assert_lse_close(gpu: np.ndarray, ref: np.ndarray, what: str = "lse") -> None:
    """Log-sum-exp rows: |gpu - ref| <= LSE_ATOL + LSE_RTOL * |ref|."""
    g = np.asarray(gpu, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    if g.shape != r.shape:
        raise AssertionError(f"{what}: shape {g.shape} != {r.shape}")
    with np.errstate(invalid="ignore"):
        bad = ~(np.abs(g - r) <= LSE_ATOL + LSE_RTOL * np.abs(r))
    if bad.any():
        i = tuple(int(v) for v in np.argwhere(bad)[0])
        raise AssertionError(f"{what}: {int(bad.sum())} of {g.size} outside tolerance; "
                             f"first at {i}: gpu/ref {g[i]} {r[i]}")
