"""The bf16-storage parity gate accepts exactly the rounding it allows for."""
import numpy as np
import pytest
import torch

from util import TOL_BF16, check_bf16_stored


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
