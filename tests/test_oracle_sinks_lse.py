"""Pins for the oracle's log-sum-exp output and attention sinks.

A sink is one more softmax term per query head with a logit and no value row
(vLLM flash-attention PR 199, second review, finding F4: a row with no visible
key reports the sink logit as its log-sum-exp).  The oracle is checked against
an independent float64 brute force (which appends the sink as an extra score
column), against closed forms (q = 0: n equal scores plus the sink; a single
visible key: the lse is that key's score), and the split-K merge with a sink
against the unsplit row.
"""
import math

import numpy as np
import pytest

import attn_workloads as W
import oracle
from oracle import brute

SHAPES = [
    ([(1, 0, 1)], 2, 1, 64),
    ([(3, 5, 8), (70, 0, 70), (5, 130, 200)], 4, 2, 64),
    ([(17, 40, 57), (33, 0, 100)], 8, 1, 16),
    ([(6, 10, 16), (4, 0, 9)], 16, 8, 1),
]


def _case(seqs, hq, hkv, page_size, seed=13, **kw):
    return W.build_case("pin", seqs=seqs, hq=hq, hkv=hkv, seed=seed, out_dtype="fp32",
                        page_size=page_size, **kw)


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8_e4m3"])
@pytest.mark.parametrize("with_sink", [False, True])
def test_lse_and_sinks_match_float64_brute_force(shape, kv_dtype, with_sink):
    seqs, hq, hkv, ps = shape
    c = _case(seqs, hq, hkv, ps, kv_dtype=kv_dtype)
    sinks = np.random.default_rng(3).uniform(-4, 6, hq).astype(np.float32) if with_sink else None
    got, lse = oracle.attend_all_lse(c, sinks=sinks)
    ref, ref_lse = brute.attention_lse(c, sinks=sinks)
    np.testing.assert_allclose(got, ref, rtol=1e-5, atol=2e-5)
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-5, atol=2e-5)


def test_sink_with_equal_scores_closed_form():
    # q = 0: every visible score is 0, so with sink s the weights are 1 per key
    # and e^s for the sink: o = n / (n + e^s) * mean(V), lse = log(n + e^s).
    seqs = [(20, 30, 70), (5, 0, 5)]
    hq, hkv = 4, 2
    c = _case(seqs, hq, hkv, 64, q_zero=True)
    sinks = np.float32([-3.0, 0.0, 1.5, 7.0])
    got, lse = oracle.attend_all_lse(c, sinks=sinks)
    dense = brute.depage(c)
    row0 = 0
    for b, (ql, st, L) in enumerate(seqs):
        V = dense[b][1]
        for i in range(ql):
            n = min(st + i + 1, L)
            for h in range(hq):
                es = math.exp(float(sinks[h]))
                np.testing.assert_allclose(got[row0 + i, h],
                                           n / (n + es) * V[:n, h // (hq // hkv)].mean(axis=0),
                                           rtol=2e-6, atol=2e-6)
                assert abs(lse[row0 + i, h] - math.log(n + es)) <= 2e-6 * max(1.0, math.log(n + es))
        row0 += ql


def test_lse_of_a_single_visible_key_is_its_score():
    c = _case([(3, 0, 3)], 4, 1, 64)
    _, lse = oracle.attend_all_lse(c)
    dense = brute.depage(c)
    q = c.launches[0].q[:3].float().double().numpy()
    K = dense[0][0]
    for h in range(4):
        s = float(np.float32(c.softmax_scale)) * float(q[0, h] @ K[0, 0])
        assert abs(lse[0, h] - s) <= 1e-5 * max(1.0, abs(s))


def test_merge_with_sink_equals_unsplit_row():
    c = _case([(1, 299, 300)], 2, 1, 64)
    sink = 1.25
    want, want_lse = oracle.attend_rows_lse(c, [1], sinks=[0.0, sink])
    cuts = [0, 37, 64, 128, 190, 300]
    parts = [oracle.partial(c, 0, 1, a, b) for a, b in zip(cuts[:-1], cuts[1:])]
    O = np.stack([p[0] for p in parts])
    m = np.array([p[1] for p in parts], dtype=np.float32)
    l = np.array([p[2] for p in parts], dtype=np.float32)
    got, lse = oracle.merge_lse(O, m, l, sink=sink)
    np.testing.assert_allclose(got, want[0], rtol=1e-5, atol=2e-6)
    assert abs(lse - want_lse[0]) <= 1e-5


def test_no_visible_key_reports_the_sink_or_minus_infinity():
    O = np.zeros((3, 512), np.float32)
    m = np.full(3, -np.inf, np.float32)
    l = np.zeros(3, np.float32)
    out, lse = oracle.merge_lse(O, m, l, sink=2.5)
    assert np.all(out == 0) and lse == np.float32(2.5)
    out, lse = oracle.merge_lse(O, m, l)
    assert np.all(out == 0) and lse == -np.inf


def test_sink_far_above_the_scores_drives_the_output_to_zero_not_nan():
    c = _case([(4, 0, 4)], 2, 1, 64)
    got, lse = oracle.attend_all_lse(c, sinks=np.float32([80.0, 80.0]))
    assert np.isfinite(got).all() and np.abs(got).max() < 1e-30
    np.testing.assert_allclose(lse, 80.0, rtol=0, atol=1e-5)
