"""Seeded synthetic inputs for paged head-dim-512 attention.

This module holds no attention arithmetic.  It only draws random numbers,
rounds them to the storage formats (bf16, OCP FP8-E4M3), places the keys and
values into a page pool through a shuffled page table and plants hostile
padding.  Both the CPU oracle and the HIP library consume what it builds, so
it is the one piece of code the two sides share.

Storage conventions (the boundary's, stated in the C header):
  q           bf16 [rows, Hq, 512]; rows of sequence b are
              cu_seqlens_q[b] .. cu_seqlens_q[b+1]; rows past total_q are padding
  k/v pools   [num_pages, Hkv, 64, 512], bf16 or e4m3 bytes; one (page, kv head)
              is one contiguous 64-key tile (the pool is paged at the key-tile
              size, as the pegainfer issue 1051 "Proposed Plan" asks)
  page_table  int32 [batch, max_pages]; logical key j of sequence b lives in
              page page_table[b][j // 64], slot j % 64; in a ring cache of
              C = ring_pages * 64 slots (sliding-window layers) key j lives at
              cache slot j % C instead, i.e. page page_table[b][(j % C) // 64],
              and only the last C keys are held
Hostile padding (pegainfer issue 1051, "Acceptance Criteria"; Flash-Decoding
for MQA in CUDA, "The test that catches what parity misses"): unused page
slots, spare pages and q padding rows hold NaN; table entries past a
sequence's last page point at an all-NaN page.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Sequence, Tuple

import torch

HEAD_DIM = 512
PAGE_SIZE = 64
BF16_NAN_BITS = 0x7FC0
E4M3_NAN_BYTE = 0x7F
E4M3_MAX = 448.0


@dataclasses.dataclass
class Launch:
    """One call's query side: which q rows, where they sit, what they see."""

    q: torch.Tensor            # bf16 [total_q + pad, Hq, D]
    total_q: int
    q_lens: List[int]
    q_starts: List[int]        # absolute position of each sequence's first query row
    kv_lens: List[int]         # keys visible to each sequence (cache incl. this chunk)
    cu_seqlens_q: torch.Tensor  # int32 [B+1]
    q_start: torch.Tensor      # int32 [B]
    kv_len: torch.Tensor       # int32 [B]

    @property
    def batch(self) -> int:
        return len(self.q_lens)

    @property
    def max_q_len(self) -> int:
        return max(self.q_lens)

    @property
    def max_kv_len(self) -> int:
        return max(self.kv_lens)

    def causal_pairs(self) -> int:
        """Visible (query, key) pairs of one head over the whole call."""
        from .count import causal_pairs
        return causal_pairs(self.q_lens, self.q_starts, self.kv_lens)


@dataclasses.dataclass
class PagedCase:
    name: str
    num_q_heads: int
    num_kv_heads: int
    softmax_scale: float
    kv_dtype: str               # "bf16" or "fp8_e4m3"
    k_scale: float              # per-tensor dequant scales (1.0 for bf16)
    v_scale: float
    k_pool: torch.Tensor        # bf16 or uint8 [num_pages, Hkv, 64, D]
    v_pool: torch.Tensor
    page_table: torch.Tensor    # int32 [B, max_pages]
    out_dtype: str              # "bf16" or "fp32"
    launches: List[Launch]
    nan_page: int               # id of an all-NaN page that padding entries point at
    window: int = 0             # sliding window in keys (0: none)
    ring_pages: int = 0         # ring cache pages per sequence (0: unbounded cache)

    @property
    def head_dim(self) -> int:
        return int(self.k_pool.shape[-1])

    @property
    def num_pages(self) -> int:
        return int(self.k_pool.shape[0])

    @property
    def max_pages_per_seq(self) -> int:
        return int(self.page_table.shape[1])

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    def kv_bytes_per_key_head(self) -> int:
        """Bytes of K plus V per (key, kv head)."""
        return 2 * self.head_dim * (1 if self.kv_dtype == "fp8_e4m3" else 2)

    def to(self, device) -> "PagedCase":
        """Copy of the case with every tensor on `device` (same bytes)."""
        mv = lambda t: t.to(device)
        launches = [dataclasses.replace(l, q=mv(l.q), cu_seqlens_q=mv(l.cu_seqlens_q),
                                        q_start=mv(l.q_start), kv_len=mv(l.kv_len))
                    for l in self.launches]
        return dataclasses.replace(self, k_pool=mv(self.k_pool), v_pool=mv(self.v_pool),
                                   page_table=mv(self.page_table), launches=launches)


def _nan_bf16(shape, device) -> torch.Tensor:
    return torch.full(shape, BF16_NAN_BITS, dtype=torch.int16, device=device).view(torch.bfloat16)


def _normal(shape, gen, device) -> torch.Tensor:
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32)


def quantize_e4m3(x: torch.Tensor, scale: float) -> torch.Tensor:
    """Round x / scale to OCP E4M3FN (RNE, saturated to +-448); returns raw bytes."""
    y = (x.float() / scale).clamp_(-E4M3_MAX, E4M3_MAX)
    return y.to(torch.float8_e4m3fn).view(torch.uint8)


def build_case(name: str, *, seqs: Sequence[Tuple[int, int, int]], hq: int, hkv: int,
               seed: int, out_dtype: str, device="cpu",
               chunks: Optional[Sequence[Sequence[Tuple[int, int, int]]]] = None,
               row_scale: Optional[Tuple[float, float]] = None,
               q_zero: bool = False, v_one: bool = False, kv_dtype: str = "bf16",
               extra_pages: int = 3, q_pad_rows: int = 0, table_pad: int = 1,
               page_size: int = PAGE_SIZE,
               shuffle_pages: bool = True, kv_len_total: Optional[Sequence[int]] = None,
               softmax_scale: Optional[float] = None,
               page_seed: Optional[int] = None, head_dim: int = HEAD_DIM,
               window: int = 0, ring_pages: int = 0) -> PagedCase:
    """Build one paged workload.

    seqs: per sequence (q_len, q_start, kv_len) of the (single) launch.  When
    `chunks` is given instead, it lists several launches over one shared cache:
    chunks[c] = per-sequence (q_len, q_start, kv_len); query rows of all chunks
    are drawn once as one prompt, and the cache holds kv_len_total[b] keys.

    Draw order: the device generator (seed) draws Q, then K_b and V_b for each
    sequence b in logical key order; with `row_scale`, each draw is followed
    by its per-row factors U[lo, hi] (one per (row, head)), applied in fp32
    before rounding.  The CPU generator (page_seed, default seed) draws the page
    permutation.
    Storage rounding is round-to-nearest-even.

    head_dim sets D (512 for the global layers, 256 for sliding-window ones).
    window is recorded in the case for the consumers.  ring_pages > 0 stores
    each sequence in a ring of C = ring_pages * page_size slots: key j of the
    resident band [max(0, L - C), L) at slot j % C, other slots NaN.
    """
    D, P = head_dim, page_size
    assert hq % hkv == 0
    if chunks is None:
        chunks = [list(seqs)]
    B = len(chunks[0])
    if kv_len_total is None:
        kv_len_total = [max(ch[b][2] for ch in chunks) for b in range(B)]
    # all query rows of all chunks of a sequence form one prompt: rows are
    # indexed by absolute position relative to the first chunk's start
    q_rows_per_seq = []
    for b in range(B):
        first = min(ch[b][1] for ch in chunks)
        last = max(ch[b][1] + ch[b][0] for ch in chunks)
        q_rows_per_seq.append((first, last - first))
    total_prompt_rows = sum(n for _, n in q_rows_per_seq)

    dgen = torch.Generator(device=device).manual_seed(seed)
    cgen = torch.Generator().manual_seed(seed if page_seed is None else page_seed)

    # --- Q, then K and V sequence by sequence (logical order) -------------
    def draw(shape):
        x = _normal(shape, dgen, device)
        if row_scale is not None:
            lo, hi = row_scale
            x.mul_(torch.empty(shape[:-1] + (1,), device=device).uniform_(lo, hi, generator=dgen))
        return x

    qf = draw((total_prompt_rows, hq, D))
    if q_zero:
        qf.zero_()
    q_prompt = qf.to(torch.bfloat16)
    del qf
    kb, vb = [], []
    for b in range(B):
        kb.append(draw((kv_len_total[b], hkv, D)).to(torch.bfloat16))
        v = draw((kv_len_total[b], hkv, D))
        if v_one:
            v.fill_(1.0)
        vb.append(v.to(torch.bfloat16))
        del v

    # --- FP8 per-tensor scales over the valid keys -------------------------
    if kv_dtype == "fp8_e4m3":
        k_amax = max(float(t.float().abs().max()) for t in kb)
        v_amax = max(float(t.float().abs().max()) for t in vb)
        k_scale = (k_amax / E4M3_MAX) if k_amax > 0 else 1.0
        v_scale = (v_amax / E4M3_MAX) if v_amax > 0 else 1.0
        # the scales are stored as fp32 by the boundary
        k_scale = float(torch.tensor(k_scale, dtype=torch.float32))
        v_scale = float(torch.tensor(v_scale, dtype=torch.float32))
    elif kv_dtype == "bf16":
        k_scale = v_scale = 1.0
    else:
        raise ValueError(kv_dtype)

    # --- pages -------------------------------------------------------------
    if ring_pages:
        n_pages = [ring_pages] * B
    else:
        n_pages = [math.ceil(L / P) for L in kv_len_total]
    n_logical = sum(n_pages)
    num_pages = n_logical + max(1, extra_pages)
    if shuffle_pages:
        perm = torch.randperm(num_pages, generator=cgen)
    else:
        perm = torch.arange(num_pages)
    nan_page = int(perm[n_logical])
    max_pages = max(n_pages) + table_pad
    table = torch.full((B, max_pages), nan_page, dtype=torch.int32)
    pool_shape = (num_pages, hkv, P, D)
    if kv_dtype == "bf16":
        k_pool = _nan_bf16(pool_shape, device)
        v_pool = _nan_bf16(pool_shape, device)
    else:
        k_pool = torch.full(pool_shape, E4M3_NAN_BYTE, dtype=torch.uint8, device=device)
        v_pool = torch.full(pool_shape, E4M3_NAN_BYTE, dtype=torch.uint8, device=device)
    base = 0
    for b in range(B):
        ids = perm[base:base + n_pages[b]]
        table[b, :n_pages[b]] = ids.to(torch.int32)
        idx = ids.to(device)
        for src, pool, scale in ((kb[b], k_pool, k_scale), (vb[b], v_pool, v_scale)):
            L = src.shape[0]
            if kv_dtype == "bf16":
                padded = _nan_bf16((n_pages[b] * P, hkv, D), device)
                stored = src
            else:
                padded = torch.full((n_pages[b] * P, hkv, D), E4M3_NAN_BYTE, dtype=torch.uint8, device=device)
                stored = quantize_e4m3(src, scale)
            if ring_pages:
                C = ring_pages * P
                j = torch.arange(max(0, L - C), L, device=device)
                padded[j % C] = stored[j]
            else:
                padded[:L] = stored
            pool[idx] = padded.view(n_pages[b], P, hkv, D).permute(0, 2, 1, 3)
        base += n_pages[b]
    del kb, vb

    # --- launches ----------------------------------------------------------
    launches = []
    for ch in chunks:
        q_lens = [c[0] for c in ch]
        q_starts = [c[1] for c in ch]
        kv_lens = [c[2] for c in ch]
        for b in range(B):
            assert 1 <= q_lens[b] and q_starts[b] + q_lens[b] <= kv_lens[b] <= kv_len_total[b]
        total_q = sum(q_lens)
        q = _nan_bf16((total_q + q_pad_rows, hq, D), device)
        row = 0
        prompt_base = 0
        for b in range(B):
            first, nrows = q_rows_per_seq[b]
            off = q_starts[b] - first
            q[row:row + q_lens[b]] = q_prompt[prompt_base + off: prompt_base + off + q_lens[b]]
            row += q_lens[b]
            prompt_base += nrows
        cu = [0]
        for ql in q_lens:
            cu.append(cu[-1] + ql)
        launches.append(Launch(
            q=q, total_q=total_q, q_lens=q_lens, q_starts=q_starts, kv_lens=kv_lens,
            cu_seqlens_q=torch.tensor(cu, dtype=torch.int32, device=device),
            q_start=torch.tensor(q_starts, dtype=torch.int32, device=device),
            kv_len=torch.tensor(kv_lens, dtype=torch.int32, device=device)))
    del q_prompt
    scale = softmax_scale if softmax_scale is not None else 1.0 / math.sqrt(D)
    return PagedCase(name=name, num_q_heads=hq, num_kv_heads=hkv, softmax_scale=scale,
                     kv_dtype=kv_dtype, k_scale=k_scale, v_scale=v_scale,
                     k_pool=k_pool, v_pool=v_pool, page_table=table.to(device),
                     out_dtype=out_dtype, launches=launches, nan_page=nan_page,
                     window=window, ring_pages=ring_pages)


def decode_lengths(batch: int, lo: int, hi: int, seed: int) -> List[int]:
    """Per-sequence KV lengths drawn uniformly from [lo, hi] on the CPU generator."""
    g = torch.Generator().manual_seed(seed * 7919 + 17)
    return [int(x) for x in torch.randint(lo, hi + 1, (batch,), generator=g)]
