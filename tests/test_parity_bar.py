"""The parity bars themselves (CPU only): what each accepts and what it rejects."""
import numpy as np
import pytest

import parity


def rows(seed=0, n=64):
    return np.random.default_rng(seed).standard_normal((n, 512)) * 0.05


def test_bf16_bar_rejects_a_scaled_output():
    ref = rows()
    with pytest.raises(AssertionError, match="relative L2"):
        parity.assert_close(ref * 1.03, ref, parity.BF16, "3% too large")


def test_bf16_bar_rejects_one_wrong_element():
    ref = rows(1)
    got = ref.copy()
    got[7, 100] += 0.2 * np.sqrt((ref[7] ** 2).mean())   # a fifth of the row's rms on one element
    with pytest.raises(AssertionError, match="elements outside"):
        parity.assert_close(got, ref, parity.BF16, "one element")


def test_bf16_bar_accepts_bf16_sized_rounding():
    ref = rows(2)
    noise = np.random.default_rng(3).standard_normal(ref.shape) * 3e-3   # 0.3 % of each row's rms
    rms = np.sqrt((ref ** 2).mean(-1, keepdims=True))
    parity.assert_close(ref + noise * rms, ref, parity.BF16, "rounding-sized noise")


def test_f32_bar_and_arithmetic_choice():
    ref = rows(4)
    parity.assert_close(ref + 5e-5, ref, parity.F32, "within")
    with pytest.raises(AssertionError):
        parity.assert_close(ref + 2e-4, ref, parity.F32, "outside")
    assert parity.arithmetic(1, 2) == parity.BF16
    for kv, path in ((0, 2), (1, 1), (1, 3), (2, 2), (0, 1)):
        assert parity.arithmetic(kv, path) == parity.F32
    with pytest.raises(ValueError):
        parity.assert_close(ref, ref, 1, "an unnamed bf16 cache")
