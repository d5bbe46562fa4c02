"""Seeded synthetic workloads shared by the tests, the bench and the oracle checks.

No attention arithmetic lives here (see gen.py's header).
"""
from .gen import (HEAD_DIM, PAGE_SIZE, BF16_NAN_BITS, E4M3_NAN_BYTE, E4M3_MAX, Launch,
                  PagedCase, build_case, decode_lengths, quantize_e4m3)
from .count import causal_pairs, decode_kv_bytes, prefill_flops, window_pairs
from .cases import (WORKLOADS, chunk_prefill_2k, chunk_prefill_8k_at_8k,
                    chunk_prefill_8k_at_8k_late_keys, decode_b64, decode_late_keys, decode_mtp_b64,
                    long_mqa_32k, prefix_prefill_512_at_32k, swa_decode_hd256_b64,
                    swa_prefill_hd256_8k_at_8k, tiny_prefill_mqa)

__all__ = ["HEAD_DIM", "PAGE_SIZE", "BF16_NAN_BITS", "E4M3_NAN_BYTE", "E4M3_MAX", "Launch",
           "PagedCase", "build_case", "decode_lengths", "quantize_e4m3", "WORKLOADS",
           "chunk_prefill_2k", "chunk_prefill_8k_at_8k", "chunk_prefill_8k_at_8k_late_keys",
           "decode_b64", "decode_late_keys", "decode_mtp_b64", "long_mqa_32k",
           "prefix_prefill_512_at_32k", "swa_decode_hd256_b64", "swa_prefill_hd256_8k_at_8k",
           "tiny_prefill_mqa", "causal_pairs", "decode_kv_bytes", "prefill_flops", "window_pairs"]
