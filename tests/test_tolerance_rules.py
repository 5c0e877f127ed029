"""CPU checks of the comparison rules the GPU parity tests apply
(tests/harness.py): the bf16 and fp32 output bounds and the scope of the
gradient floor, which may stand in for a tensor's own RMS only when the
oracle tensor vanishes identically."""
import numpy as np
import pytest

from harness import check, check_grad


def test_floor_ignored_for_nonzero_tensor():
    ref = np.full(100, 1e-3)
    got = ref + 5e-5          # 5 % of the tensor's own RMS: outside 0.02 RMS + half-ulp
    with pytest.raises(AssertionError):
        check_grad("bf16", got, ref, "nonzero", floor=1.0)


def test_floor_applies_to_identically_zero_tensor():
    ref = np.zeros(100)
    got = np.full(100, 3e-7)  # cancellation residue of O(1) terms
    check_grad("bf16", got, ref, "vanishing", floor=1.0)
    check_grad("f32", got, ref, "vanishing", floor=1.0)
    with pytest.raises(AssertionError):
        check_grad("f32", got, ref, "no floor", floor=0.0)


def test_floor_threshold_is_relative():
    ref = np.full(10, 1e-7)   # RMS 1e-7 <= 1e-6 * floor(1): treated as vanishing
    check_grad("f32", ref + 5e-5, ref, "tiny", floor=1.0)
    ref = np.full(10, 1e-5)   # RMS 1e-5 > 1e-6: held to its own RMS
    with pytest.raises(AssertionError):
        check_grad("f32", ref + 5e-5, ref, "small", floor=1.0)


def test_bf16_output_bound():
    rng = np.random.default_rng(0)
    ref = rng.standard_normal(1000)
    rms = np.sqrt(np.mean(ref ** 2))
    got = ref + 0.019 * rms
    check("bf16", got, ref)
    with pytest.raises(AssertionError):
        check("bf16", ref + 0.03 * rms + 2.0 ** -8 * np.abs(ref), ref)


def test_fp32_output_bound():
    ref = np.linspace(-3, 3, 50)
    check("f32", ref + 0.9e-4, ref)
    with pytest.raises(AssertionError):
        check("f32", ref + 1.1e-4, ref)
