"""Shared helpers of the GPU parity tests: run the library, compare with the oracle."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import attn_workloads as W

# Parity gate for floating-point outputs: max-abs and mean-abs error against
# the fp32 oracle.
MAX_ABS = 1e-2
MEAN_ABS = 1e-3
SENTINEL_F32 = 0x7F8DEAD1   # a NaN payload never produced by arithmetic
SENTINEL_BF16 = 0x7F8D


def library():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import attention_hd512_gqa_amd as A
    A.lib()   # raises when the HIP library is missing: no fallback exists
    return A


def out_tensor(rows: int, hq: int, dtype: str, pad_rows: int = 0,
               head_dim: int = W.HEAD_DIM) -> torch.Tensor:
    if dtype == "fp32":
        t = torch.empty((rows + pad_rows, hq, head_dim), dtype=torch.float32, device="cuda")
        t.view(torch.int32).fill_(SENTINEL_F32)
    else:
        t = torch.empty((rows + pad_rows, hq, head_dim), dtype=torch.bfloat16, device="cuda")
        t.view(torch.int16).fill_(SENTINEL_BF16)
    return t


def sentinel_intact(t: torch.Tensor) -> bool:
    if t.dtype == torch.float32:
        return bool((t.view(torch.int32) == SENTINEL_F32).all())
    return bool((t.view(torch.int16) == SENTINEL_BF16).all())


def run_prefill(A, case, li: int = 0, out_dtype: str = None, pad_rows: int = 0,
                fp8_mma: bool = False):
    lc = case.launches[li]
    out = out_tensor(lc.total_q, case.num_q_heads, out_dtype or case.out_dtype, pad_rows)
    A.prefill(lc.q, case.k_pool, case.v_pool, case.page_table, lc.cu_seqlens_q, lc.q_start,
              lc.kv_len, out, total_q=lc.total_q, max_q_len=lc.max_q_len,
              softmax_scale=case.softmax_scale, kv_dtype=case.kv_dtype,
              k_scale=case.k_scale, v_scale=case.v_scale, fp8_mma=fp8_mma)
    torch.cuda.synchronize()
    return out


def run_decode(A, case, out_dtype: str = None, keys_per_split: int = 0, poison_ws: bool = True):
    lc = case.launches[0]
    B = lc.batch
    out = out_tensor(B, case.num_q_heads, out_dtype or case.out_dtype)
    nbytes = A.decode_workspace_size(B, case.num_q_heads, case.num_kv_heads, lc.max_kv_len,
                                     keys_per_split)
    ws = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda")
    if poison_ws:
        ws.fill_(float("nan"))   # an unwritten partial that is read shows up as NaN
    A.decode(lc.q[:B], case.k_pool, case.v_pool, case.page_table, lc.kv_len, out, ws,
             max_kv_len=lc.max_kv_len, softmax_scale=case.softmax_scale,
             kv_dtype=case.kv_dtype, k_scale=case.k_scale, v_scale=case.v_scale,
             keys_per_split=keys_per_split)
    torch.cuda.synchronize()
    return out


def bf16_half_ulp(x: np.ndarray) -> np.ndarray:
    """Half a bf16 unit in the last place at |x| (the rounding of a bf16 output)."""
    ax = np.maximum(np.abs(x), np.float32(2.0 ** -126))
    e = np.floor(np.log2(ax))
    return np.float32(2.0) ** (e - 8)


def errors(got: torch.Tensor, ref: np.ndarray):
    g = got.float().cpu().numpy()
    assert np.isfinite(g).all(), "non-finite output"
    d = np.abs(g.astype(np.float64) - ref.astype(np.float64))
    return d, g


def rne_bf16(x: np.ndarray) -> np.ndarray:
    """x (finite fp32) rounded to nearest even bf16, returned as fp32."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return r.astype(np.uint32).view(np.float32)


def check_parity(got: torch.Tensor, ref: np.ndarray, what: str):
    """The gate: max-abs <= 1e-2 and mean-abs <= 1e-3 against the fp32 oracle.

    A bf16 output is the fp32 result rounded to nearest even (the defined
    epilogue), so for it the reference is the oracle's value rounded the same
    way: the per-element error beyond that rounding (half an ulp of bf16 at
    the reference value) is held to the max-abs bound, and the mean-abs bound
    applies to the difference from the rounded oracle value.  An fp32 output
    is compared with the oracle directly.
    """
    d, g = errors(got, ref)
    raw_max = float(d.max())
    if got.dtype == torch.bfloat16:
        excess = float(np.maximum(d - bf16_half_ulp(ref), 0).max())
        mean = float(np.abs(g.astype(np.float64) - rne_bf16(ref).astype(np.float64)).mean())
    else:
        excess = raw_max
        mean = float(d.mean())
    print(f"[parity] {what}: max_abs={raw_max:.3e} beyond_rounding={excess:.3e} "
          f"mean_abs={mean:.3e} n={d.size}", flush=True)
    assert excess <= MAX_ABS, f"{what}: max-abs error {excess} > {MAX_ABS}"
    assert mean <= MEAN_ABS, f"{what}: mean-abs error {mean} > {MEAN_ABS}"
    return raw_max, mean


def sample_rows(lc, hq: int, tokens, ) -> np.ndarray:
    """Oracle entries (q_row * Hq + head) for the given global q rows, all heads."""
    t = np.asarray(sorted(set(int(x) for x in tokens)), dtype=np.int64)
    return (t[:, None] * hq + np.arange(hq)[None, :]).reshape(-1), t
