"""Comparison rules between GPU outputs and the oracle -- TEST INFRASTRUCTURE.

Float outputs: elementwise |gpu - ref| <= 1e-2*|ref| + 1e-2*rms(ref), with both
sides decoded from bf16 to float64 and rms taken over the compared elements.
Integer-valued inputs and all routing / permutation indices: bit equality.
"""
from __future__ import annotations

from typing import Dict

import numpy as np

from .mk_oracle import bf16_to_f64

REL_TOL = 1e-2
RMS_TOL = 1e-2


def tolerance_report(gpu_bits: np.ndarray, ref_bits: np.ndarray,
                     rel: float = REL_TOL, rms_tol: float = RMS_TOL) -> Dict[str, float]:
    g = bf16_to_f64(np.asarray(gpu_bits, dtype=np.uint16))
    r = bf16_to_f64(np.asarray(ref_bits, dtype=np.uint16))
    if g.shape != r.shape:
        raise ValueError(f"shape mismatch {g.shape} vs {r.shape}")
    if r.size == 0:
        return dict(ok=True, worst=0.0, n_bad=0, rms=0.0, n=0)
    rms = float(np.sqrt(np.mean(r * r)))
    bound = rel * np.abs(r) + rms_tol * rms
    d = np.abs(g - r)
    bad = ~(d <= bound)                       # NaN counts as bad
    worst = float(np.max(np.where(bound > 0, d / np.maximum(bound, 1e-300), d)))
    return dict(ok=not bool(bad.any()), worst=worst, n_bad=int(bad.sum()), rms=rms, n=int(r.size))


def assert_close_bf16(gpu_bits: np.ndarray, ref_bits: np.ndarray, what: str = "") -> None:
    rep = tolerance_report(gpu_bits, ref_bits)
    if not rep["ok"]:
        g = np.asarray(gpu_bits, dtype=np.uint16)
        r = np.asarray(ref_bits, dtype=np.uint16)
        gd, rd = bf16_to_f64(g), bf16_to_f64(r)
        rms = rep["rms"]
        bad = np.argwhere(~(np.abs(gd - rd) <= REL_TOL * np.abs(rd) + RMS_TOL * rms))
        first = [tuple(int(v) for v in b) for b in bad[:5]]
        vals = [(gd[tuple(b)], rd[tuple(b)]) for b in bad[:5]]
        raise AssertionError(f"{what}: {rep['n_bad']} of {rep['n']} elements outside "
                             f"tolerance; first at {first}: gpu/ref {vals}")


def assert_bits_equal(gpu: np.ndarray, ref: np.ndarray, what: str = "") -> None:
    g = np.asarray(gpu)
    r = np.asarray(ref)
    if g.shape != r.shape:
        raise AssertionError(f"{what}: shape {g.shape} != {r.shape}")
    if g.dtype != r.dtype:
        r = r.astype(g.dtype)
    ne = np.argwhere(g != r)
    if ne.size:
        first = [tuple(int(v) for v in b) for b in ne[:5]]
        vals = [(g[tuple(b)], r[tuple(b)]) for b in ne[:5]]
        raise AssertionError(f"{what}: {len(ne)} of {g.size} elements differ; first at "
                             f"{first}: gpu/ref {vals}")
