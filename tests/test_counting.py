"""The work counts behind the reported rates, pinned to figures the pages print."""
import json
import os

import pytest

import attn_workloads as W

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "printed_values.json")))


def test_causal_flop_convention_reproduces_printed_total():
    g = GOLDEN["causal_flops_20k_prompt"]
    n = g["prompt_tokens"]
    per_layer = W.prefill_flops([n], [0], [n], g["q_heads"], g["head_dim"])
    total = per_layer * g["layers"]
    assert total / 1e12 == pytest.approx(g["printed_tflop"], rel=0.005)


def test_kv_bytes_per_token_reproduce_printed_total():
    g = GOLDEN["kv_bytes_per_token_32k"]
    per_layer = W.decode_kv_bytes([g["context"]], g["kv_heads"], g["head_dim"], g["bytes_per_elem"])
    assert per_layer * g["layers"] / 1e6 == pytest.approx(g["printed_mb"], rel=0.002)


def test_causal_pairs_against_brute_count():
    for seqs in ([(5, 0, 5)], [(3, 7, 10), (4, 0, 9)], [(8, 2, 6)], [(1, 0, 1)]):
        brute = 0
        for ql, st, L in seqs:
            brute += sum(min(st + i + 1, L) for i in range(ql))
        assert W.causal_pairs(*zip(*seqs)) == brute


def test_measured_workload_sizes():
    assert W.prefill_flops([256], [0], [256], 8) == 263168 * 2048
    assert W.prefill_flops([8192], [8192], [16384], 32) == 6597338202112
    total = sum(W.prefill_flops([4096], [4096 * c], [4096 * (c + 1)], 16) for c in range(8))
    assert total == 17592722915328
