"""The bound used for gradients stored in bf16 (CPU): half a bf16 unit in the
last place, the most that round-to-nearest-even can move an fp32 value."""
import numpy as np
import torch

from tests.test_parity_gpu import bf16_half_ulp, bf16_stored_excess


def test_half_ulp_values():
    # 8 significant bits: the unit at [1, 2) is 2^-7, at [4, 8) 2^-5
    assert bf16_half_ulp(1.0) == 2.0 ** -8
    assert bf16_half_ulp(1.999) == 2.0 ** -8
    assert bf16_half_ulp(2.0) == 2.0 ** -7
    assert bf16_half_ulp(-4.41) == 2.0 ** -6
    assert bf16_half_ulp(0.0) == 0.0
    assert bf16_half_ulp(3e-3) == 2.0 ** -17  # 3e-3 lies in [2^-9, 2^-8)


def test_half_ulp_bounds_rne_and_is_attained():
    gen = torch.Generator().manual_seed(7)
    x = torch.randn(200000, generator=gen) * 3.0
    r = x.to(torch.bfloat16).double()
    err = (r - x.double()).abs().numpy()
    hu = bf16_half_ulp(x.double().abs().numpy())
    assert np.all(err <= hu)
    assert np.max(err / hu) > 0.99  # tight: some value rounds by almost half a unit


def test_stored_excess_subtracts_only_the_rounding():
    ref = np.array([4.4, -1.0, 0.25])
    exact = torch.tensor(ref, dtype=torch.float32).to(torch.bfloat16)
    assert bf16_stored_excess(exact, ref, 2e-2) <= 0.0
    off = torch.tensor(ref + 0.05, dtype=torch.float32).to(torch.bfloat16)
    assert bf16_stored_excess(off, ref, 2e-2) > 2e-2
