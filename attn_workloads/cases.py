"""The measured workloads and the small parity fixtures, by name.

Shapes follow the pages' workloads: Gemma-4 global layers at head_dim 512,
32 query heads over 4 KV heads for the 31B model (pegainfer issue 1051,
"Description"; A custom attention kernel for Gemma 4 on the RTX PRO 6000,
"The kernel in three steps") and one KV head for the 12B model (Flash-Decoding
for MQA in CUDA, "One KV head breaks the textbook"), 64-token pages and 8 query
heads over 4 KV heads for decode (vLLM flash-attention PR 199, "Performance").
No public dataset is involved: every tensor is a seeded synthetic draw.
"""
from __future__ import annotations

from typing import Callable, Dict

import torch

from .gen import PagedCase, build_case, decode_lengths


def tiny_prefill_mqa(device="cpu", seed=1) -> PagedCase:
    """256 query rows causal over the same 256 keys, 8 q heads over 1 KV head, fp32 out."""
    return build_case("tiny_prefill_mqa_256", seqs=[(256, 0, 256)], hq=8, hkv=1,
                      seed=seed, out_dtype="fp32", device=device)


def _fp8_suffix(kv_dtype: str) -> str:
    return "" if kv_dtype == "bf16" else "_fp8"


def chunk_prefill_2k(device="cpu", seed=2, kv_dtype="bf16") -> PagedCase:
    """2048 rows causal over 2048 keys, 32 q heads over 4 KV heads, bf16 out."""
    return build_case("chunk_prefill_2048" + _fp8_suffix(kv_dtype), seqs=[(2048, 0, 2048)],
                      hq=32, hkv=4, seed=seed, out_dtype="bf16", device=device,
                      kv_dtype=kv_dtype)


def chunk_prefill_8k_at_8k(device="cpu", seed=3, kv_dtype="bf16") -> PagedCase:
    """One 8192-row chunk at positions 8192..16383 over 16384 keys, 32/4 heads, bf16 out.

    Hostile padding: 64 NaN q rows past the chunk, three spare NaN pages, a
    NaN page behind the table's padding column.
    """
    return build_case("chunk_prefill_8192_at_8192" + _fp8_suffix(kv_dtype),
                      seqs=[(8192, 8192, 16384)], hq=32, hkv=4, seed=seed, out_dtype="bf16",
                      device=device, q_pad_rows=64, extra_pages=3, table_pad=2,
                      kv_dtype=kv_dtype)


def long_mqa_32k(device="cpu", seed=4, q_zero=False, v_one=False, kv_dtype="bf16") -> PagedCase:
    """A 32768-token prompt as eight 4096-row causal chunks against the growing cache.

    16 q heads over 1 KV head; every (row, head) of Q, K and V carries its own
    factor U[0.5, 2]; fp32 out.  The whole 32768-key cache is resident from
    the start, so keys past a chunk's kv_len are finite data that must stay
    unread.  The q=0, V=1 variant must give exactly 1 everywhere.
    """
    chunks = [[(4096, 4096 * c, 4096 * (c + 1))] for c in range(8)]
    name = "long_mqa_32k_8x4096" + ("_q0_v1" if (q_zero or v_one) else "") + _fp8_suffix(kv_dtype)
    return build_case(name, seqs=None, chunks=chunks, hq=16, hkv=1, seed=seed,
                      out_dtype="fp32", device=device, row_scale=(0.5, 2.0),
                      q_zero=q_zero, v_one=v_one, kv_dtype=kv_dtype)


def chunk_prefill_8k_at_8k_late_keys(device="cpu", seed=3, kv_dtype="bf16") -> PagedCase:
    """The 8192-row chunk at 8192..16383 with late dominant keys.

    Every query row gets 1.5 u added (u = a fixed +-1 vector over the head
    dims, re-rounded to bf16), and three keys of every KV head are set to
    beta u with beta = 1.125, 2.25 and 4.5 at positions 4000, 8191 and 12288:
    about 38, 76 and 152 nats (scale 1/sqrt(512)) above a typical score, so
    each lies more than 32 log2 units above what the row saw before it --
    first above the row's first 32 keys (the softmax reference starts
    there), then above the previous late key.  Rows at 12288 and later see
    all three.  In an FP8-E4M3 pool the late keys are the E4M3 codes of
    beta u / k_scale.
    """
    case = chunk_prefill_8k_at_8k(device=device, seed=seed, kv_dtype=kv_dtype)
    case.name = "chunk_prefill_8192_at_8192_late_keys" + _fp8_suffix(kv_dtype)
    lc = case.launches[0]
    u = torch.where(torch.arange(case.head_dim, device=device) % 3 == 0, -1.0, 1.0)
    lc.q[:lc.total_q] = (lc.q[:lc.total_q].float() + 1.5 * u).to(torch.bfloat16)
    for j, beta in ((4000, 1.125), (8191, 2.25), (12288, 4.5)):
        page = int(case.page_table[0, j // 64])
        row = beta * u
        if kv_dtype == "bf16":
            case.k_pool[page, :, j % 64, :] = row.to(torch.bfloat16)
        else:
            code = (row / case.k_scale).to(torch.float8_e4m3fn).view(torch.uint8)
            case.k_pool[page, :, j % 64, :] = code
    return case


def prefix_prefill_512_at_32k(device="cpu", seed=6, kv_dtype="bf16") -> PagedCase:
    """A short chunk over a long prefix: 512 rows at positions 32256..32767 over
    32768 keys, 32 q heads over 4 KV heads, bf16 out.

    The single-pass launch has 32 row blocks x 4 KV heads = 128 workgroups,
    each walking all 512 key tiles; the split-K entry point spreads the key
    range over the compute units.  Hostile padding as in the 8192-row chunk.
    """
    return build_case("prefix_prefill_512_at_32k" + _fp8_suffix(kv_dtype),
                      seqs=[(512, 32256, 32768)], hq=32, hkv=4, seed=seed, out_dtype="bf16",
                      device=device, q_pad_rows=16, extra_pages=3, table_pad=2,
                      kv_dtype=kv_dtype)


def swa_prefill_hd256_8k_at_8k(device="cpu", seed=7) -> PagedCase:
    """A sliding-window (local) layer: one 8192-row chunk at positions
    8192..16383, window 1024, head_dim 256, 32 q heads over 4 KV heads, bf16
    out, in a ring cache of 144 pages (9216 slots = chunk + window) that has
    wrapped: the 16384 keys were written through it, so only the last 9216
    are resident and the table holds 144 entries."""
    return build_case("swa_prefill_hd256_8192_at_8192_w1024", seqs=[(8192, 8192, 16384)],
                      hq=32, hkv=4, seed=seed, out_dtype="bf16", device=device,
                      q_pad_rows=16, extra_pages=3, table_pad=2, head_dim=256, window=1024,
                      ring_pages=144)


def swa_decode_hd256_b64(device="cpu", seed=8, batch=64, lo=4096, hi=28672) -> PagedCase:
    """Single-token decode of a sliding-window layer: batch 64, window 1024,
    head_dim 256, 32 q heads over 4 KV heads, lengths U{4096..28672}, each
    sequence in a ring of 16 pages (1024 slots = the window)."""
    lens = decode_lengths(batch, lo, hi, seed)
    return build_case(f"swa_decode_hd256_b{batch}_w1024", seqs=[(1, L - 1, L) for L in lens],
                      hq=32, hkv=4, seed=seed, out_dtype="bf16", device=device, head_dim=256,
                      window=1024, ring_pages=16)


def decode_b64(device="cpu", seed=5, kv_dtype="bf16", batch=64, lo=4096, hi=28672) -> PagedCase:
    """Batch-64 single-token decode, 8 q heads over 4 KV heads, lengths U{4096..28672}.

    The FP8 variant stores the same bf16 values as E4M3 bytes with per-tensor
    k_scale and v_scale.
    """
    lens = decode_lengths(batch, lo, hi, seed)
    seqs = [(1, L - 1, L) for L in lens]
    name = f"decode_b{batch}_splitk" + ("_fp8" if kv_dtype != "bf16" else "")
    return build_case(name, seqs=seqs, hq=8, hkv=4, seed=seed, out_dtype="bf16",
                      device=device, kv_dtype=kv_dtype)


def decode_mtp_b64(device="cpu", seed=9, kv_dtype="bf16", batch=64, q_len=5, lo=4096,
                   hi=28672) -> PagedCase:
    """Batch-64 multi-token decode at the 31B model's global-layer shape: the
    current token plus a 4-token draft (q_len 5) per sequence, 32 q heads over
    4 KV heads (g = 8, so 40 (token, head) columns per KV head), lengths
    U{4096..28672} (Gemma-4 deployment with a 4-token draft: A custom
    attention kernel for Gemma 4 on the RTX PRO 6000, "The deployment").
    """
    lens = decode_lengths(batch, lo, hi, seed)
    seqs = [(q_len, L - q_len, L) for L in lens]
    name = f"decode_mtp_b{batch}_q{q_len}_g8" + ("_fp8" if kv_dtype != "bf16" else "")
    return build_case(name, seqs=seqs, hq=32, hkv=4, seed=seed, out_dtype="bf16",
                      device=device, kv_dtype=kv_dtype)


def decode_late_keys(device="cpu", seed=29, kv_dtype="bf16", q_len=1) -> PagedCase:
    """Decode of q_len tokens per sequence (kv_len 700, 1500, 3000; 32 q heads
    over 4 KV heads, fp32 out) with late dominant keys, for the split
    kernels' reference moves.

    As in the 8192-row chunk with late keys: every query row gets 1.5 u
    added (u = a fixed +-1 vector over the head dims), and some keys of every
    KV head are set to beta u.  beta = 0.375 puts a key about 18.6 log2 units
    above a typical score (scores are about N(0, 2.7) log2 units, a tile's
    maximum about 6.5): 12 above what its split saw before it, more than the
    decode kernels' margins (8 and 10).  Sequences 0 and 1 have one such key,
    at positions 100 and 1400 (inside a 256- or 1024-key split, after its
    first tile): it dominates the output while the keys before it still
    weigh about 2^-12 each, so O and l must be rescaled when the reference
    moves, not restarted.  Sequence 2 climbs: beta = 0.375, 0.625, 1 and 2
    at positions 100, 420, 2800 and 2900 (about 18.6, 31, 50 and 99 log2
    units).  In an FP8-E4M3 pool the keys are the E4M3 codes of beta u /
    k_scale (within the E4M3 range at these betas).
    """
    lens = (700, 1500, 3000)
    plant = (((100, 0.375),), ((1400, 0.375),),
             ((100, 0.375), (420, 0.625), (2800, 1.0), (2900, 2.0)))
    case = build_case(f"decode_late_keys_q{q_len}" + _fp8_suffix(kv_dtype),
                      seqs=[(q_len, L - q_len, L) for L in lens], hq=32, hkv=4, seed=seed,
                      out_dtype="fp32", device=device, kv_dtype=kv_dtype, extra_pages=2,
                      table_pad=2)
    lc = case.launches[0]
    u = torch.where(torch.arange(case.head_dim, device=device) % 3 == 0, -1.0, 1.0)
    lc.q[:lc.total_q] = (lc.q[:lc.total_q].float() + 1.5 * u).to(torch.bfloat16)
    for b in range(len(lens)):
        for j, beta in plant[b]:
            page = int(case.page_table[b, j // 64])
            row = beta * u
            if kv_dtype == "bf16":
                case.k_pool[page, :, j % 64, :] = row.to(torch.bfloat16)
            else:
                code = (row / case.k_scale).to(torch.float8_e4m3fn).view(torch.uint8)
                case.k_pool[page, :, j % 64, :] = code
    return case


WORKLOADS: Dict[str, Callable[..., PagedCase]] = {
    "tiny_prefill_mqa_256": tiny_prefill_mqa,
    "chunk_prefill_2048": chunk_prefill_2k,
    "chunk_prefill_8192_at_8192": chunk_prefill_8k_at_8k,
    "chunk_prefill_8192_at_8192_late_keys": chunk_prefill_8k_at_8k_late_keys,
    "long_mqa_32k_8x4096": long_mqa_32k,
    "prefix_prefill_512_at_32k": prefix_prefill_512_at_32k,
    "decode_b64_splitk": decode_b64,
    "decode_mtp_b64_q5_g8": decode_mtp_b64,
    "swa_prefill_hd256_8192_at_8192_w1024": swa_prefill_hd256_8k_at_8k,
    "swa_decode_hd256_b64_w1024": swa_decode_hd256_b64,
}
