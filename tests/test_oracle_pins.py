"""Pins for the CPU oracle: it is checked against things other than itself.

- float64 brute force on tiny inputs (independent de-paging, dense scores);
- a library special case: torch's CPU scaled_dot_product_attention over the
  de-paged tensors with an explicit bottom-right causal mask;
- closed forms: q = 0 gives the mean of the attended values; V = 1 gives
  exactly 1 at every length (the long-split accumulation trap of vLLM
  flash-attention PR 199, first review comment); a single visible key gives
  that key's value; one late key ahead by Delta has a closed-form output
  (same PR, review finding F1); per-KV-head constant values give the group's
  constant (consecutive GQA grouping); positions as values give the mean
  position, which pins the causal alignment;
- invariants: key translation, convex hull, page placement (bitwise),
  in-page row permutation of fully visible pages;
- format decoders: all 256 E4M3 codes and random bf16 patterns against torch;
- the Flash-Decoding merge over random splits equals the unsplit row.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import attn_workloads as W
import oracle
from oracle import brute

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "printed_values.json")))

SHAPES = [
    # seqs (q_len, q_start, kv_len), hq, hkv, page_size
    ([(1, 0, 1)], 2, 1, 64),
    ([(3, 5, 8), (70, 0, 70), (5, 130, 200)], 4, 2, 64),
    ([(17, 40, 57), (33, 0, 100)], 8, 1, 16),
    ([(9, 3, 12), (1, 63, 64), (2, 64, 66)], 16, 1, 4),
    ([(6, 10, 16), (4, 0, 9)], 16, 8, 1),
    ([(64, 64, 200)], 8, 8, 64),
]


def _case(seqs, hq, hkv, page_size, seed=11, **kw):
    return W.build_case("pin", seqs=seqs, hq=hq, hkv=hkv, seed=seed, out_dtype="fp32",
                        page_size=page_size, **kw)


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8_e4m3"])
def test_matches_float64_brute_force(shape, kv_dtype):
    seqs, hq, hkv, ps = shape
    c = _case(seqs, hq, hkv, ps, kv_dtype=kv_dtype)
    got = oracle.attend_all(c)
    ref = brute.attention(c)
    assert np.isfinite(got).all()
    np.testing.assert_allclose(got, ref, rtol=1e-5, atol=2e-5)


@pytest.mark.parametrize("shape", SHAPES[1:4])
def test_matches_torch_sdpa_with_explicit_mask(shape):
    seqs, hq, hkv, ps = shape
    c = _case(seqs, hq, hkv, ps, seed=5)
    got = oracle.attend_all(c)
    lc = c.launches[0]
    g = hq // hkv
    dense = brute.depage(c)
    row0 = 0
    for b, (ql, st, L) in enumerate(seqs):
        K = torch.from_numpy(dense[b][0]).float().permute(1, 0, 2).repeat_interleave(g, 0)
        V = torch.from_numpy(dense[b][1]).float().permute(1, 0, 2).repeat_interleave(g, 0)
        Q = lc.q[row0:row0 + ql].float().permute(1, 0, 2)
        mask = torch.arange(L)[None, :] <= (st + torch.arange(ql))[:, None]
        ref = F.scaled_dot_product_attention(Q, K, V, attn_mask=mask, scale=c.softmax_scale)
        np.testing.assert_allclose(got[row0:row0 + ql], ref.permute(1, 0, 2).numpy(),
                                   rtol=1e-5, atol=2e-5)
        row0 += ql


def test_q_zero_gives_mean_of_attended_values():
    seqs = [(20, 30, 70), (5, 0, 5), (40, 100, 300)]
    c = _case(seqs, 4, 2, 64, q_zero=True)
    got = oracle.attend_all(c)
    dense = brute.depage(c)
    row0 = 0
    for b, (ql, st, L) in enumerate(seqs):
        V = dense[b][1]
        for i in range(ql):
            n = min(st + i + 1, L)
            for h in range(4):
                np.testing.assert_allclose(got[row0 + i, h], V[:n, h // 2].mean(axis=0),
                                           rtol=0, atol=2e-6)
        row0 += ql


@pytest.mark.parametrize("keys", GOLDEN["q0_v1_output"]["keys"])
def test_v_one_gives_exactly_one_at_long_lengths(keys):
    # one decode row over `keys` keys, random q: the output must be 1.0 exactly
    c = _case([(1, keys - 1, keys)], 2, 1, 64, v_one=True, extra_pages=1)
    got = oracle.attend_rows(c, [0, 1])
    assert np.all(got == GOLDEN["q0_v1_output"]["value"])


def test_v_one_exact_on_chunked_rows():
    c = _case([(64, 64, 200), (7, 0, 7)], 8, 2, 64, v_one=True)
    assert np.all(oracle.attend_all(c) == 1.0)


def test_single_visible_key_returns_its_value():
    c = _case([(3, 0, 3)], 4, 1, 64)
    got = oracle.attend_all(c)
    v0 = brute.depage(c)[0][1][0, 0]
    for h in range(4):
        assert np.array_equal(got[0, h], v0.astype(np.float32))


def _spike_case(n, delta, seed=3):
    """q = a e_0, keys zero in dim 0 except the last visible key: logits 0 and Delta."""
    c = _case([(1, n - 1, n)], 1, 1, 64, seed=seed, extra_pages=1)
    a = 16.0
    coef = delta / (c.softmax_scale * a)
    # choose the key coefficient as a bf16 value and recompute the exact Delta
    coef_b = float(torch.tensor(coef).to(torch.bfloat16))
    lc = c.launches[0]
    lc.q.zero_()
    lc.q[0, 0, 0] = a
    c.k_pool[:, :, :, 0] = 0
    late = n - 1
    page = int(c.page_table[0, late // 64])
    c.k_pool[page, 0, late % 64, 0] = coef_b
    d_exact = float(np.float32(np.float32(c.softmax_scale) * np.float32(a * coef_b)))
    return c, d_exact


@pytest.mark.parametrize("delta", GOLDEN["late_key_spike"]["deltas"])
@pytest.mark.parametrize("n", [4096, GOLDEN["late_key_spike"]["keys"]])
def test_late_key_spike_closed_form(n, delta):
    c, d = _spike_case(n, delta)
    j = torch.arange(n)
    V = c.v_pool[c.page_table[0, j // 64].long(), 0, j % 64].double().numpy()
    w_late = math.exp(d)
    expect = (V[:-1].sum(axis=0) + w_late * V[-1]) / (n - 1 + w_late)
    got = oracle.attend_rows(c, [0])[0]
    # fp32 sequential sums over n equal small weights drift by up to ~n*eps/4
    tol = 1e-5 if n <= 4096 else 2e-4
    np.testing.assert_allclose(got, expect, rtol=tol, atol=tol * np.abs(expect).max())


def test_key_translation_invariance():
    seqs = [(10, 20, 40), (30, 0, 90)]
    c = _case(seqs, 4, 2, 16, seed=9)
    gen = torch.Generator().manual_seed(2)
    grid = lambda shape, lim: (torch.randn(shape, generator=gen) * 8).round().clamp(-8 * lim, 8 * lim) / 8
    nan = c.k_pool.isnan()
    base = grid(c.k_pool.shape, 4)
    shift = grid((1, c.num_kv_heads, 1, W.HEAD_DIM), 2)
    c.k_pool.copy_(base.to(torch.bfloat16)).masked_fill_(nan, float("nan"))
    out1 = oracle.attend_all(c)
    c.k_pool.copy_((base + shift).to(torch.bfloat16)).masked_fill_(nan, float("nan"))
    assert torch.equal(c.k_pool[~nan].float(), (base + shift).expand_as(nan)[~nan])  # exact in bf16
    out2 = oracle.attend_all(c)
    np.testing.assert_allclose(out1, out2, rtol=1e-5, atol=2e-5)


def test_output_inside_convex_hull_of_attended_values():
    seqs = [(25, 40, 70), (12, 0, 12)]
    c = _case(seqs, 4, 1, 64, row_scale=(0.5, 2.0))
    got = oracle.attend_all(c)
    dense = brute.depage(c)
    row0 = 0
    for b, (ql, st, L) in enumerate(seqs):
        V = dense[b][1][:, 0, :]
        for i in range(ql):
            n = st + i + 1
            lo, hi = V[:n].min(axis=0), V[:n].max(axis=0)
            slack = 1e-6 * np.maximum(1, np.abs(V[:n]).max())
            assert np.all(got[row0 + i] >= lo - slack) and np.all(got[row0 + i] <= hi + slack)
        row0 += ql


def test_page_placement_is_bitwise_irrelevant():
    seqs = [(9, 100, 150), (40, 0, 40)]
    a = _case(seqs, 4, 2, 16, page_seed=1)
    b = _case(seqs, 4, 2, 16, page_seed=2)
    assert not torch.equal(a.page_table, b.page_table)
    assert np.array_equal(oracle.attend_all(a), oracle.attend_all(b))


def test_in_page_row_permutation_of_visible_pages():
    # decode rows see every key, so permuting K and V rows together inside
    # pages only reorders the fp32 sums
    seqs = [(1, 199, 200), (1, 63, 64), (1, 130, 131)]
    c = _case(seqs, 4, 2, 64, seed=4)
    before = oracle.attend_all(c)
    gen = torch.Generator().manual_seed(7)
    for b, (_, _, L) in enumerate(seqs):
        for pi in range(math.ceil(L / 64)):
            valid = min(64, L - 64 * pi)
            perm = torch.randperm(valid, generator=gen)
            page = int(c.page_table[b, pi])
            for pool in (c.k_pool, c.v_pool):
                pool[page, :, :valid] = pool[page, :, perm].clone()
    after = oracle.attend_all(c)
    np.testing.assert_allclose(before, after, rtol=1e-6, atol=1e-6)


def test_query_heads_map_to_consecutive_kv_heads():
    c = _case([(5, 3, 8), (2, 0, 20)], 16, 4, 16, v_one=True)
    for kvh in range(4):
        c.v_pool[:, kvh] *= (kvh + 1)
    got = oracle.attend_all(c)
    for h in range(16):
        np.testing.assert_allclose(got[:, h], h // 4 + 1, rtol=1e-6, atol=0)


def test_positions_as_values_pin_the_causal_alignment():
    # q = 0 and V[j] = j in dim 0: each row returns the mean visible position
    seqs = [(16, 48, 100), (7, 0, 7), (3, 200, 203)]
    c = _case(seqs, 2, 1, 64, q_zero=True)
    for b, (_, _, L) in enumerate(seqs):
        for j in range(L):
            c.v_pool[int(c.page_table[b, j // 64]), 0, j % 64, 0] = float(j)
    got = oracle.attend_all(c)
    row0 = 0
    for ql, st, L in seqs:
        for i in range(ql):
            n = st + i + 1
            assert got[row0 + i, 0, 0] == pytest.approx((n - 1) / 2, rel=1e-6)
        row0 += ql


def test_e4m3_decoder_matches_torch_for_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    got = oracle.e4m3_to_f32(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan) and set(np.nonzero(nan)[0]) == {0x7F, 0xFF}
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_bf16_widening_matches_torch():
    bits = np.random.default_rng(0).integers(0, 1 << 16, 100000, dtype=np.uint64).astype(np.uint16)
    got = oracle.bf16_to_f32(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_split_merge_equals_unsplit():
    seqs = [(1, 999, 1000), (1, 4095, 4096)]
    c = _case(seqs, 4, 2, 64, seed=8)
    rng = np.random.default_rng(3)
    row0 = 0
    for b, (_, _, L) in enumerate(seqs):
        for h in (0, 3):
            cuts = np.sort(rng.integers(1, L, 6))
            bounds = [0, *cuts.tolist(), L, L + 128]          # last split is empty
            parts = [oracle.partial(c, row0, h, k0, k1) for k0, k1 in zip(bounds[:-1], bounds[1:])]
            O = np.stack([p[0] for p in parts])
            m = np.array([p[1] for p in parts], dtype=np.float32)
            l = np.array([p[2] for p in parts], dtype=np.float32)
            assert m[-1] == -np.inf and l[-1] == 0 and not O[-1].any()
            merged = oracle.merge(O, m, l)
            whole = oracle.attend_rows(c, [row0 * 4 + h])[0]
            np.testing.assert_allclose(merged, whole, rtol=1e-6, atol=1e-6)
            assert np.array_equal(oracle.merge(O[:-1], m[:-1], l[:-1]), merged)
        row0 += 1


def test_masked_range_is_an_empty_partial():
    c = _case([(4, 10, 100)], 2, 1, 64)
    O, m, l = oracle.partial(c, 0, 0, 11, 100)   # row 0 sees keys 0..10 only
    assert m == -np.inf and l == 0.0 and not O.any()
