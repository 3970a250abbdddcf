"""Pins of the comparison rules (oracle/compare.py) -- CPU only.

The float rule is |gpu - ref| <= 1e-2 |ref| + 1e-2 rms(ref) with rms over the
whole reference tensor; these tests put values just inside and just outside
each term of the bound (on the bf16 grid, so the cases are exact), and check
that non-finite GPU values, shape mismatches and a part of an output compared
without the whole tensor's rms are handled as the rule says.  Bit equality,
the MoE gate rule and the log-sum-exp rule are pinned the same way.
"""
import numpy as np
import pytest

import oracle.compare as C
from oracle.mk_oracle import f64_to_bf16


def bf(*vals):
    """bf16 bits of values that bf16 represents exactly (checked)."""
    x = np.asarray(vals, dtype=np.float64)
    b = f64_to_bf16(x)
    back = (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert np.array_equal(back, x, equal_nan=True), "test value not on the bf16 grid"
    return b


def passes(gpu, ref, rms=None):
    try:
        C.assert_close_bf16(gpu, ref, "pin", rms=rms)
        return True
    except AssertionError:
        return False


def test_relative_term_inside_and_outside():
    # rms supplied as 0: the bound is 1e-2 |ref| alone; at |ref| = 128 it is
    # 1.28 and the bf16 grid there has spacing 1
    assert passes(bf(129.0), bf(128.0), rms=0.0)
    assert not passes(bf(130.0), bf(128.0), rms=0.0)
    # the bound uses |ref|: the same for a negative reference
    assert passes(bf(-129.0), bf(-128.0), rms=0.0)
    assert not passes(bf(-130.0), bf(-128.0), rms=0.0)
    assert not passes(bf(-126.0), bf(-128.0), rms=0.0)


def test_rms_term_inside_boundary_and_outside():
    # ref = one 1000 and 99 zeros: rms = sqrt(1000^2 / 100) = 100, so a zero
    # element may be off by 1e-2 * 100 = 1.0 (inclusive)
    ref = bf(*([1000.0] + [0.0] * 99))
    assert C.rms_of(ref) == pytest.approx(100.0, rel=0, abs=1e-12)
    for v, ok in [(0.99609375, True), (1.0, True), (1.0078125, False), (-1.0078125, False)]:
        gpu = ref.copy()
        gpu[57] = bf(v)[0]
        assert passes(gpu, ref) is ok, v
    # at the 1000 element the bound is 10 + 1 = 11; the grid spacing is 4
    for v, ok in [(1008.0, True), (992.0, True), (1012.0, False), (988.0, False)]:
        gpu = ref.copy()
        gpu[0] = bf(v)[0]
        assert passes(gpu, ref) is ok, v


def test_part_of_an_output_uses_the_whole_tensors_rms():
    full = bf(*([1000.0] + [0.0] * 99))
    part_ref = full[10:20]                       # zeros only: its own rms is 0
    part_gpu = part_ref.copy()
    part_gpu[3] = bf(0.5)[0]
    assert passes(part_gpu, part_ref, rms=C.rms_of(full))  # 0.5 <= 1e-2 * 100
    assert not passes(part_gpu, part_ref)                  # taken as the whole tensor: bound 0


@pytest.mark.parametrize("bad_bits", [0x7FC0, 0x7F80, 0xFF80])  # NaN, +inf, -inf
def test_non_finite_gpu_values_fail(bad_bits):
    ref = bf(1.0, 2.0, 3.0)
    gpu = ref.copy()
    gpu[1] = bad_bits
    assert not passes(gpu, ref)
    rep = C.tolerance_report(gpu, ref)
    assert not rep["ok"] and rep["n_bad"] == 1


def test_non_finite_reference_is_an_error():
    ref = bf(1.0, 2.0, 3.0)
    ref[2] = 0x7FC0
    with pytest.raises(ValueError):
        C.tolerance_report(bf(1.0, 2.0, 3.0), ref)


def test_shape_mismatch_fails_and_empty_passes():
    assert not passes(bf(1.0, 2.0), bf(1.0, 2.0, 3.0))
    assert not passes(bf(1.0, 2.0).reshape(2, 1), bf(1.0, 2.0))
    assert passes(np.zeros((0, 4), np.uint16), np.zeros((0, 4), np.uint16))


def test_identical_outputs_pass_at_every_scale():
    g = np.random.default_rng(5)
    x = f64_to_bf16(g.normal(0, 1e-3, 1000) * 10.0 ** g.integers(-20, 20, 1000))
    assert passes(x, x)


def test_bit_equality():
    a = np.array([0x3F80, 0x0000, 0x1234], dtype=np.uint16)
    C.assert_bits_equal(a, a.copy(), "same")
    b = a.copy()
    b[2] ^= 1                                     # one bit of one element
    with pytest.raises(AssertionError):
        C.assert_bits_equal(b, a, "one bit")
    z = a.copy()
    z[1] = 0x8000                                  # -0.0 against +0.0: different bits
    with pytest.raises(AssertionError):
        C.assert_bits_equal(z, a, "signed zero")
    with pytest.raises(AssertionError):
        C.assert_bits_equal(a[:2], a, "shape")
    with pytest.raises(AssertionError):
        C.assert_bits_equal(np.zeros(3), np.zeros(3), "float arrays are not bit patterns")
    C.assert_bits_equal(np.array([1, -2, 3], np.int32), np.array([1, -2, 3], np.int64), "widths")
    with pytest.raises(AssertionError):
        C.assert_bits_equal(np.array([1], np.int32), np.array([1 << 40], np.int64), "overflow")


def test_gate_rule():
    ref = np.array([0.5, 0.25], dtype=np.float64)
    C.assert_gates_close(np.array([0.5 + 4e-6, 0.25 - 2e-6]), ref)
    with pytest.raises(AssertionError):
        C.assert_gates_close(np.array([0.5 + 6e-6, 0.25]), ref)
    with pytest.raises(AssertionError):
        C.assert_gates_close(np.array([0.5, 0.25 + 3e-6]), ref)
    with pytest.raises(AssertionError):
        C.assert_gates_close(np.array([np.nan, 0.25]), ref)


def test_lse_rule():
    ref = np.array([10.0, -2.0])
    C.assert_lse_close(np.array([10.0019, -2.0011]), ref)   # bounds 2e-3 and 1.2e-3
    with pytest.raises(AssertionError):
        C.assert_lse_close(np.array([10.0021, -2.0]), ref)
    with pytest.raises(AssertionError):
        C.assert_lse_close(np.array([10.0, -2.0013]), ref)
    with pytest.raises(AssertionError):
        C.assert_lse_close(np.array([np.inf, -2.0]), ref)
