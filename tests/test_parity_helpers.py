"""CPU checks of the parity gate's helpers: the bf16 rounding it compares against."""
import numpy as np
import torch

from _gpu_helpers import bf16_half_ulp, rne_bf16


def test_rne_bf16_matches_torch_rounding():
    g = np.random.default_rng(0)
    x = np.concatenate([g.standard_normal(100000).astype(np.float32) * 10.0 ** g.integers(-8, 8, 100000),
                        np.float32([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3.4e38, -3.4e38, 1e-40])])
    x = x.astype(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    np.testing.assert_array_equal(rne_bf16(x).view(np.uint32), want.view(np.uint32))


def test_half_ulp_bounds_the_rounding():
    g = np.random.default_rng(1)
    x = (g.standard_normal(100000) * 5).astype(np.float32)
    err = np.abs(rne_bf16(x).astype(np.float64) - x.astype(np.float64))
    assert (err <= bf16_half_ulp(x) * (1 + 1e-6)).all()
