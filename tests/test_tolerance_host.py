"""The rounding allowance of the GPU comparisons (tests/_gpu.py) on the CPU:
half a unit in the last place of bfloat16 / float16, against torch's own
rounding of the same values."""
import numpy as np
import torch

from _gpu import half_ulp


def test_half_ulp_matches_the_rounding_of_torch():
    rng = np.random.default_rng(0)
    # float32 values, rounded once to the 16-bit type (as the kernels round
    # their float32 results; float64 -> 16 bit in torch rounds twice)
    x32 = np.concatenate([rng.standard_normal(20000) * 4, rng.standard_normal(2000) * 1e-3,
                          [0.0, 1.0, 2.0, 4.0, -4.0, 3.99, 1e-5]]).astype(np.float32)
    x = x32.astype(np.float64)
    for dtype in (torch.bfloat16, torch.float16):
        r = torch.from_numpy(x32).to(dtype).double().numpy()
        err = np.abs(r - x)
        h = half_ulp(x, dtype)
        assert np.all(err <= h * (1 + 1e-12)), dtype
        # and it is tight: some value is rounded by (almost) the full half ulp
        big = np.abs(x) > 1
        assert np.max(err[big] / h[big]) > 0.99


def test_half_ulp_known_values():
    assert half_ulp(np.array([4.0]), torch.bfloat16)[0] == 2.0 ** -6
    assert half_ulp(np.array([3.9]), torch.bfloat16)[0] == 2.0 ** -7
    assert half_ulp(np.array([1.0]), torch.float16)[0] == 2.0 ** -11
