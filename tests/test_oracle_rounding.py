"""Pins of the oracle's storage rounding against torch's CPU casts (an independent implementation)."""
import numpy as np
import pytest
import torch

from oracle import rne_bf16, rne_f32


def _torch_bf16(x32: np.ndarray) -> np.ndarray:
    return torch.from_numpy(x32).to(torch.bfloat16).to(torch.float64).numpy()


def test_bf16_matches_torch_on_random_floats():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(200000) * np.exp2(rng.integers(-40, 40, 200000))).astype(np.float32)
    np.testing.assert_array_equal(rne_bf16(x.astype(np.float64)), _torch_bf16(x))


def test_bf16_ties_round_to_even():
    rng = np.random.default_rng(1)
    hi = rng.integers(0, 0x7F00, 5000).astype(np.uint32)
    u = (hi << 16) | 0x8000            # exactly half way between two bf16 neighbours
    x = u.view(np.float32)
    got = rne_bf16(x.astype(np.float64))
    np.testing.assert_array_equal(got, _torch_bf16(x))
    even = ((hi & 1) == 0)
    down = (hi << 16).view(np.float32).astype(np.float64)
    assert np.all(got[even] == down[even])
    assert np.all(got[~even] != down[~even])


def test_bf16_subnormals_signs_zero():
    vals = np.array([0.0, -0.0, 1e-40, -1e-40, 2.0 ** -133, 2.0 ** -134, 3 * 2.0 ** -134, 2.0 ** -126,
                     -(2.0 ** -127), 1.0, -1.0, 3.0e38], dtype=np.float32)
    got = rne_bf16(vals.astype(np.float64))
    np.testing.assert_array_equal(got, _torch_bf16(vals))
    assert np.signbit(got[1]) and not np.signbit(got[0])


def test_bf16_direct_from_f64_is_single_rounding():
    # a float64 value just above a bf16 tie must round up even when float32 would round it to the tie
    tie = 1.0 + 2.0 ** -8                # halfway between bf16 1.0 and 1.0 + 2**-7
    x = np.array([tie + 2.0 ** -40])
    assert rne_bf16(x)[0] == 1.0 + 2.0 ** -7
    assert rne_bf16(np.array([tie]))[0] == 1.0


@pytest.mark.parametrize("seed", [0, 1])
def test_f32_matches_torch(seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(100000) * np.exp2(rng.integers(-60, 60, 100000))
    ref = torch.from_numpy(x).to(torch.float32).to(torch.float64).numpy()
    np.testing.assert_array_equal(rne_f32(x), ref)
