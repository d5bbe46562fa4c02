"""Pins for the oracle's sliding window and ring cache (the local layers).

A row at position pos sees keys max(0, pos - W + 1) <= j <= pos (its own and
the W - 1 before it; A custom attention kernel for Gemma 4 on the RTX PRO
6000, "The deployment": the local layers attend to the last 1,024 tokens),
and a ring cache of C slots holds key j at slot j % C, reading only the live
band (Flash-Decoding for MQA in CUDA, "One KV head breaks the textbook").
The oracle is checked against:

- the float64 brute force, which de-pages through the ring on its own and
  marks keys the ring no longer holds as NaN (so a band that reaches one
  poisons the result);
- closed forms: W = 1 gives the row's own value exactly; q = 0 gives the mean
  of the band's values;
- invariants: a window covering every key equals no window (bitwise); a
  wrapped ring equals the same keys in an unbounded paged layout (bitwise).
"""
import numpy as np
import pytest
import torch

import attn_workloads as W
import oracle
from oracle import brute

SHAPES = [
    # seqs (q_len, q_start, kv_len), hq, hkv, page_size, head_dim, window, ring_pages
    ([(5, 0, 5)], 2, 1, 64, 256, 3, 0),
    ([(20, 30, 50), (7, 0, 7)], 4, 2, 16, 256, 8, 0),
    ([(9, 100, 109), (3, 5, 8)], 8, 1, 4, 64, 16, 0),
    ([(12, 52, 64), (20, 20, 40)], 4, 4, 16, 256, 10, 2),      # ring of 32 slots, wrapped
    ([(6, 90, 96), (1, 200, 201)], 8, 2, 4, 64, 7, 3),         # ring of 12 slots, wraps many times
    ([(16, 184, 200)], 2, 1, 64, 256, 64, 2),                  # 64-key pages, ring of 128 slots
]


def _case(seqs, hq, hkv, page, d, window, ring, seed=19, **kw):
    return W.build_case("win", seqs=seqs, hq=hq, hkv=hkv, seed=seed, out_dtype="fp32",
                        page_size=page, head_dim=d, window=window, ring_pages=ring, **kw)


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8_e4m3"])
def test_window_and_ring_match_float64_brute_force(shape, kv_dtype):
    case = _case(*shape, kv_dtype=kv_dtype)
    got = oracle.attend_all(case, threads=2)
    ref = brute.attention(case)
    assert np.isfinite(ref).all(), "the fixture's bands must be resident"
    np.testing.assert_allclose(got, ref, rtol=1e-5, atol=2e-5)


def test_brute_force_flags_a_band_the_ring_no_longer_holds():
    # ring of 8 slots, window 12: rows see keys the ring overwrote
    case = _case([(4, 60, 64)], 2, 1, 4, 64, 12, 2)
    assert np.isnan(brute.attention(case)).any()


def _logical_values(case, b, positions):
    """float64 V rows of sequence b at the given positions, read through the
    page table slot by slot (third, independent de-paging)."""
    P = int(case.v_pool.shape[2])
    C = case.ring_pages * P
    rows = []
    for j in positions:
        c = j % C if C else j
        page = int(case.page_table[b, c // P])
        rows.append(case.v_pool[page, :, c % P, :].float().double().numpy())
    return np.stack(rows)   # [n, Hkv, D]


def test_window_one_returns_the_rows_own_value():
    case = _case([(10, 70, 80), (3, 0, 3)], 4, 2, 16, 256, 1, 2)
    got = oracle.attend_all(case, threads=2)
    lc = case.launches[0]
    row = 0
    for b, (ql, st) in enumerate(zip(lc.q_lens, lc.q_starts)):
        V = _logical_values(case, b, range(st, st + ql))
        for i in range(ql):
            for h in range(4):
                assert np.array_equal(got[row + i, h], V[i, h // 2].astype(np.float32))
        row += ql


def test_q_zero_gives_the_mean_of_the_band():
    Wn = 9
    case = _case([(15, 40, 55), (6, 0, 6)], 4, 2, 16, 256, Wn, 3, q_zero=True)
    got = oracle.attend_all(case, threads=2)
    lc = case.launches[0]
    row = 0
    for b, (ql, st) in enumerate(zip(lc.q_lens, lc.q_starts)):
        for i in range(ql):
            pos = st + i
            band = range(max(0, pos - Wn + 1), pos + 1)
            V = _logical_values(case, b, band)
            for h in range(4):
                np.testing.assert_allclose(got[row + i, h], V[:, h // 2].mean(axis=0),
                                           rtol=0, atol=2e-6)
        row += ql


def test_window_covering_every_key_equals_no_window():
    seqs = [(30, 20, 50), (8, 0, 8)]
    a = oracle.attend_all(_case(seqs, 4, 2, 16, 256, 50, 0), threads=2)
    b = oracle.attend_all(_case(seqs, 4, 2, 16, 256, 0, 0), threads=2)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8_e4m3"])
def test_wrapped_ring_equals_the_unbounded_layout(kv_dtype):
    # same seed, so the same logical keys; only their placement differs
    seqs = [(24, 176, 200), (5, 90, 95)]
    ring = _case(seqs, 8, 2, 16, 256, 32, 4, kv_dtype=kv_dtype)      # 64 slots
    flat = _case(seqs, 8, 2, 16, 256, 32, 0, kv_dtype=kv_dtype)
    assert ring.k_pool.shape[0] != flat.k_pool.shape[0]
    assert np.array_equal(oracle.attend_all(ring, threads=2), oracle.attend_all(flat, threads=2))
