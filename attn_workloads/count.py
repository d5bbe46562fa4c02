"""Algorithmic work of one call: the numerators of the reported rates.

Prefill counts 4 * head_dim FLOP per unmasked (query, key) pair and head: one
multiply-add per element for Q.K^T and one for P.V, nothing for masked pairs,
padding or the softmax.  That is the convention behind the 131 TFLOP the
Gemma-4 RTX PRO 6000 page gives for a 19,985-token prompt ("What it changed
end to end"), which tests/test_counting.py reproduces.  Decode counts the K
and V bytes of the live band [0, kv_len) of every sequence and KV head, read
once (Flash-Decoding for MQA in CUDA, "The starting point": cost must follow
the live length, not the allocation).  A sliding window of W keys caps both:
a row at pos sees min(pos + 1, kv_len) - max(0, pos - W + 1) keys, and decode
reads the band [max(0, kv_len - W), kv_len).
"""
from __future__ import annotations

from typing import Sequence


def causal_pairs(q_lens: Sequence[int], q_starts: Sequence[int], kv_lens: Sequence[int]) -> int:
    """Sum over query rows of min(pos + 1, kv_len): visible (query, key) pairs per head."""
    total = 0
    for ql, st, L in zip(q_lens, q_starts, kv_lens):
        a = max(0, min(ql, L - st))          # rows whose causal limit is below kv_len
        total += a * st + a * (a + 1) // 2 + (ql - a) * L
    return total


def window_pairs(q_lens: Sequence[int], q_starts: Sequence[int], kv_lens: Sequence[int],
                 window: int) -> int:
    """Visible (query, key) pairs per head with a sliding window (0: none)."""
    if window <= 0:
        return causal_pairs(q_lens, q_starts, kv_lens)
    total = 0
    for ql, st, L in zip(q_lens, q_starts, kv_lens):
        for pos in range(st, st + ql):
            total += max(0, min(pos + 1, L) - max(0, pos - window + 1))
    return total


def prefill_flops(q_lens, q_starts, kv_lens, num_q_heads: int, head_dim: int = 512,
                  window: int = 0) -> int:
    return 4 * head_dim * num_q_heads * window_pairs(q_lens, q_starts, kv_lens, window)


def decode_kv_bytes(kv_lens: Sequence[int], num_kv_heads: int, head_dim: int = 512,
                    bytes_per_elem: int = 2, window: int = 0) -> int:
    """K plus V bytes of every sequence's live band, each KV head read once."""
    keys = sum(min(L, window) if window > 0 else L for L in kv_lens)
    return keys * num_kv_heads * head_dim * bytes_per_elem * 2
