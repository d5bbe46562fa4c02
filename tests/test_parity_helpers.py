"""CPU checks of the parity gate's helpers: the bf16 rounding, the rounding
floor, and that the gate is applied to the raw error against the fp32 oracle."""
import numpy as np
import pytest
import torch

from _gpu_helpers import (MAX_ABS, MEAN_ABS, check_parity, check_parity_floor_case,
                          floor_breaks_gate, one_token_per_block, rne_bf16, rounding_floor)


def test_rne_bf16_matches_torch_rounding():
    g = np.random.default_rng(0)
    x = np.concatenate([g.standard_normal(100000).astype(np.float32) * 10.0 ** g.integers(-8, 8, 100000),
                        np.float32([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3.4e38, -3.4e38, 1e-40])])
    x = x.astype(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    np.testing.assert_array_equal(rne_bf16(x).view(np.uint32), want.view(np.uint32))


def test_rounding_floor_is_half_an_ulp_at_most():
    # bf16 keeps 8 significant bits: rounding x moves it by at most 2^-9 |x|
    g = np.random.default_rng(1)
    x = (g.standard_normal(100000) * 5).astype(np.float32)
    fmax, fmean = rounding_floor(x)
    assert fmax <= float(np.abs(x).max()) * 2.0 ** -8
    assert 0 < fmean < fmax
    # values exactly representable in bf16 have no floor
    assert rounding_floor(rne_bf16(x)) == (0.0, 0.0)


def test_floor_detects_only_rounding_breaches():
    # |o| ~ N(0, 1): rounding alone stays far below both bounds
    x = np.random.default_rng(2).standard_normal(4096).astype(np.float32)
    assert not floor_breaks_gate(x * 0.1)
    # |o| around 3.5: the mean rounding error passes 1e-3 (a single-key row of
    # dequantised E4M3 values is such a case)
    big = (3.0 + np.random.default_rng(3).random(4096)).astype(np.float32)
    assert floor_breaks_gate(big)


def test_gate_is_raw_for_both_output_dtypes():
    ref = np.random.default_rng(4).standard_normal((64, 512)).astype(np.float32) * 0.05
    good = torch.from_numpy(ref.copy())
    check_parity(good, ref, "exact fp32")
    check_parity(good.to(torch.bfloat16), ref, "rounded bf16")
    for dtype in (torch.float32, torch.bfloat16):
        bad = good.clone()
        bad[3, 7] += 2 * MAX_ABS          # one element past the max-abs bound
        with pytest.raises(AssertionError, match="max-abs"):
            check_parity(bad.to(dtype), ref, "one bad element")
        bad = good + 2 * MEAN_ABS        # every element a little off: mean-abs
        with pytest.raises(AssertionError, match="mean-abs"):
            check_parity(bad.to(dtype), ref, "uniform offset")


def test_floor_case_requires_the_rounded_fp32_output():
    ref = (3.0 + np.random.default_rng(5).random((8, 512))).astype(np.float32)
    f32 = torch.from_numpy(ref.copy())
    check_parity_floor_case(f32.to(torch.bfloat16), f32, ref, "floor case")
    off = f32.to(torch.bfloat16).clone()
    off.view(torch.int16)[0, 0] += 1     # one ulp away from rne(fp32)
    with pytest.raises(AssertionError, match="differs"):
        check_parity_floor_case(off, f32, ref, "floor case, wrong rounding")
    with pytest.raises(AssertionError, match="not a floor case"):
        small = ref * 0.01
        t = torch.from_numpy(small)
        check_parity_floor_case(t.to(torch.bfloat16), t, small, "no floor breach")


def test_one_token_per_block_covers_every_block():
    for q_len, block in ((8192, 16), (4096, 8), (37, 16), (1, 8)):
        t = one_token_per_block(q_len, block, seed=3)
        assert t[0] == 0 and t[-1] == q_len - 1
        assert set(x // block for x in t) == set(range((q_len + block - 1) // block))
        assert all(0 <= x < q_len for x in t)
