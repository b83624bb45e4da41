"""The bf16-storage parity gate accepts exactly the rounding it allows for."""
import numpy as np
import pytest
import torch

from util import GRAD_L2_BF16, TOL_BF16, U_BF16, check_bf16_stored, check_grad


def _round_bf16(a: np.ndarray) -> np.ndarray:
    """Round to nearest even bf16, as uint16 bit patterns (via torch's CPU cast)."""
    return torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16).view(torch.int16) \
        .numpy().view(np.uint16)


def test_rounded_reference_passes_with_zero_excess():
    rng = np.random.default_rng(3)
    ref = (rng.standard_normal(4096) * np.exp(rng.standard_normal(4096) * 2)).astype(np.float32)
    assert check_bf16_stored(_round_bf16(ref), ref, "rounded") == 0.0


def test_error_beyond_rounding_fails():
    rng = np.random.default_rng(4)
    ref = rng.standard_normal(4096)
    got = ref.copy()
    got[17] += 3 * TOL_BF16 * np.sqrt(np.mean(ref * ref))
    with pytest.raises(AssertionError):
        check_bf16_stored(_round_bf16(got), ref, "planted")


def test_gradient_gate_passes_rounding_flips():
    # against the storage-point chain: one-ulp flips at an element's own
    # storage point and at one of its inputs (up to 2 ulps = 4 U_BF16 of its
    # magnitude), on a third of the elements, the largest ones included
    rng = np.random.default_rng(5)
    ref = rng.standard_normal(200_000)
    ref[:10] = 12.0 * np.sign(ref[:10])
    flips = rng.integers(-2, 3, size=ref.size) * (rng.uniform(size=ref.size) < 0.33)
    flips[:10] = 2
    got = ref * (1 + 2 * U_BF16 * flips)
    check_grad(got, ref, "bf16", "two-ulp flips")


def test_gradient_gate_catches_a_wrong_tile_a_scale_error_and_a_three_ulp_error():
    rng = np.random.default_rng(6)
    ref = rng.standard_normal((256, 512))
    bad = ref.copy()
    bad[128:160, 256:288] *= 1.3   # one 32 x 32 block off by 30 %
    with pytest.raises(AssertionError):
        check_grad(bad, ref, "bf16", "wrong tile")
    with pytest.raises(AssertionError):
        check_grad(ref * (1 + 1.5 * GRAD_L2_BF16), ref, "bf16", "scaled")
    # one element at 10 RMS three ulps off: one ulp beyond the flip room is
    # 0.078 of the RMS, above the 2e-2 bar
    big = ref.copy()
    big[3, 7] = 10.0 * np.sqrt(np.mean(ref * ref))
    off = big.copy()
    off[3, 7] *= 1 + 3 * 2 * U_BF16
    with pytest.raises(AssertionError):
        check_grad(off, big, "bf16", "three ulps")
    off[3, 7] = big[3, 7] * (1 + 2 * 2 * U_BF16)
    check_grad(off, big, "bf16", "two ulps")
    assert TOL_BF16 == 2e-2
