"""The element-wise bars of the GPU parity tests (``tests/_parity.py``), checked
on the CPU with planted deviations: a rounding cascade confined to a few rows
passes, the same size of deviation spread over every row does not."""
import numpy as np
import pytest
import torch

from ._parity import check_elements


def _ref(shape=(2, 40, 2, 64), seed=0):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=g).bfloat16()


def _bump(x, mask, ulps):
    """Move the bf16 values under ``mask`` ``ulps`` steps away from zero."""
    bits = x.view(torch.int16).clone()
    bits[mask] += ulps
    return bits.view(torch.bfloat16)


def _f64(x):
    return x.double().numpy()


def test_identical_passes():
    r = _ref()
    assert check_elements("dz", _f64(r), _f64(r), bf16=True) == 1.0


@pytest.mark.parametrize("nrows", [1, 4])
def test_cascade_in_few_rows_passes(nrows):
    # three-ulp deviations over whole token rows (every value of the row), as a
    # rotated value rounded to the other neighbour leaves them
    r = _ref()
    mask = torch.zeros(r.shape, dtype=torch.bool)
    for i in range(nrows):
        mask[0, 5 + 7 * i, i % 2, :] = True
    a = _bump(r, mask, 3)
    assert check_elements("dz", _f64(a), _f64(r), bf16=True) < 0.999


def test_cascade_in_five_rows_fails():
    r = _ref()
    mask = torch.zeros(r.shape, dtype=torch.bool)
    for i in range(5):
        mask[1, 3 + 5 * i, 0, :] = True
    a = _bump(r, mask, 3)
    with pytest.raises(AssertionError, match="within 1 bf16 ulp"):
        check_elements("dz", _f64(a), _f64(r), bf16=True)


def test_small_error_in_every_row_fails():
    # two ulps in one column of every row: inside the per-element bound, so only
    # the ulp count can catch it (a dropped small term, a wrong column)
    r = _ref()
    mask = torch.zeros(r.shape, dtype=torch.bool)
    mask[..., 17] = True
    a = _bump(r, mask, 2)
    dev = np.abs(_f64(a) - _f64(r))
    rms = float(np.sqrt(np.mean(_f64(r) ** 2)))
    assert (dev <= 2.0 ** -5 * np.abs(_f64(r)) + 2.0 ** -3 * rms).all()
    with pytest.raises(AssertionError, match="within 1 bf16 ulp"):
        check_elements("dz", _f64(a), _f64(r), bf16=True)


def test_up_to_32_scattered_elements_pass():
    r = _ref()
    mask = torch.zeros(r.numel(), dtype=torch.bool)
    mask[torch.randperm(r.numel(), generator=torch.Generator().manual_seed(1))[:32]] = True
    a = _bump(r, mask.view(r.shape), 2)
    check_elements("dz", _f64(a), _f64(r), bf16=True)
