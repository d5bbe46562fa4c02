"""Pins for the paged KV append oracle and its E4M3 encoder."""
import numpy as np
import torch

import oracle
from oracle import kv_append


def test_encoder_matches_torch_inside_the_range():
    g = np.random.default_rng(0)
    x = np.concatenate([g.standard_normal(200000) * 10.0 ** g.uniform(-4, 2.6, 200000),
                        g.uniform(-448, 448, 10000)]).astype(np.float32)
    x = np.clip(x, -448, 448).astype(np.float32)
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = kv_append.e4m3_encode(x, 1.0)
    assert np.array_equal(got, want)


def test_every_finite_code_round_trips():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = oracle.e4m3_to_f32(codes)
    got = kv_append.e4m3_encode(vals, 1.0)
    # +0 and -0 keep their own codes
    assert np.array_equal(got, codes)


def test_midpoints_round_to_the_even_code_and_range_saturates():
    pos = np.arange(1, 0x7F, dtype=np.uint8)
    v = oracle.e4m3_to_f32(pos).astype(np.float64)
    mid = ((v[:-1] + v[1:]) / 2).astype(np.float32)
    ok = mid.astype(np.float64) == (v[:-1] + v[1:]) / 2   # exactly representable midpoints
    got = kv_append.e4m3_encode(mid[ok], 1.0)
    lo, hi = pos[:-1][ok], pos[1:][ok]
    assert np.array_equal(got, np.where(lo % 2 == 0, lo, hi))
    assert np.array_equal(kv_append.e4m3_encode(np.float32([500.0, -1e9, 448.0]), 1.0),
                          np.uint8([0x7E, 0xFE, 0x7E]))


def test_scale_divides_before_rounding():
    x = np.float32([1.0, 3.0, -7.0, 0.3])
    assert np.array_equal(kv_append.e4m3_encode(x, 0.5), kv_append.e4m3_encode(x * 2, 1.0))


def test_append_scatters_like_a_per_element_loop():
    g = np.random.default_rng(1)
    pages, hkv, ps, d = 6, 2, 4, 8
    kp = g.integers(0, 65535, (pages, hkv, ps, d), dtype=np.uint16)
    vp = kp.copy()
    table = np.array([[3, 1, 5], [0, 4, 2]], dtype=np.int32)
    cu = np.array([0, 3, 8], dtype=np.int32)
    qs = np.array([2, 9], dtype=np.int32)   # seq 0 rows at 2..4, seq 1 at 9..13 (12, 13 past the table)
    kn = torch.randn(8, hkv, d).to(torch.bfloat16)
    vn = torch.randn(8, hkv, d).to(torch.bfloat16)
    k2, v2 = kv_append.append(kp, vp, kn, vn, table, cu, qs, "bf16")
    want = kp.copy()
    bits = kn.view(torch.int16).numpy().view(np.uint16)
    for b in range(2):
        for i in range(cu[b + 1] - cu[b]):
            p = qs[b] + i
            if p // ps >= table.shape[1]:
                continue
            for h in range(hkv):
                for e in range(d):
                    want[table[b, p // ps], h, p % ps, e] = bits[cu[b] + i, h, e]
    assert np.array_equal(k2, want)
