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


def rounding_floor(ref: np.ndarray):
    """(max, mean) of |rne_bf16(ref) - ref|: the error a bf16 output carries
    from its own rounding even when the fp32 result before it is exact."""
    d = np.abs(rne_bf16(ref).astype(np.float64) - ref.astype(np.float64))
    return float(d.max()), float(d.mean())


def floor_breaks_gate(ref: np.ndarray) -> bool:
    fmax, fmean = rounding_floor(ref)
    return fmax > MAX_ABS or fmean > MEAN_ABS


def check_parity(got: torch.Tensor, ref: np.ndarray, what: str):
    """The gate: max-abs <= 1e-2 and mean-abs <= 1e-3 of the output against
    the unrounded fp32 oracle, for fp32 and bf16 outputs alike.

    For a bf16 output the error of rounding the oracle itself to bf16 (the
    floor no bf16 output can go below) is printed beside the raw figures and
    named in the failure message; it is never subtracted.
    """
    d, g = errors(got, ref)
    raw_max = float(d.max())
    mean = float(d.mean())
    floor = ""
    if got.dtype == torch.bfloat16:
        fmax, fmean = rounding_floor(ref)
        floor = f" bf16_floor_max={fmax:.3e} bf16_floor_mean={fmean:.3e}"
    print(f"[parity] {what}: max_abs={raw_max:.3e} mean_abs={mean:.3e}{floor} n={d.size}",
          flush=True)
    assert raw_max <= MAX_ABS, f"{what}: max-abs error {raw_max} > {MAX_ABS}{floor}"
    assert mean <= MEAN_ABS, f"{what}: mean-abs error {mean} > {MEAN_ABS}{floor}"
    return raw_max, mean


def check_parity_floor_case(got_bf16: torch.Tensor, got_f32: torch.Tensor, ref: np.ndarray,
                            what: str):
    """A case whose exact result rounded to bf16 already breaks the gate.

    No bf16 output can pass such a case, so the kernel's arithmetic is gated
    through its fp32-output form (the same main loop, a different store), and
    the bf16 output is required to be exactly that fp32 output rounded to
    nearest even.  The case and its floor are printed so that it is reported,
    not absorbed.
    """
    fmax, fmean = rounding_floor(ref)
    assert fmax > MAX_ABS or fmean > MEAN_ABS, f"{what}: not a floor case"
    print(f"[parity] {what}: bf16 rounding floor breaks the gate (floor max={fmax:.3e} "
          f"mean={fmean:.3e}, max|o|={float(np.abs(ref).max()):.3f}); gating the fp32 output "
          f"and requiring bf16 == rne(fp32)", flush=True)
    check_parity(got_f32, ref, what + " (fp32 output)")
    want = got_f32.to(torch.bfloat16)
    assert torch.equal(got_bf16.view(torch.int16), want.view(torch.int16)), \
        f"{what}: bf16 output differs from the rounded fp32 output"


def check_parity_any(run, ref: np.ndarray, what: str, out_dtype: str):
    """check_parity of run(out_dtype), or for a bf16 floor case the pair
    run("bf16"), run("fp32") through check_parity_floor_case."""
    got = run(out_dtype)
    if out_dtype == "bf16" and floor_breaks_gate(ref):
        return check_parity_floor_case(got, run("fp32"), ref, what)
    return check_parity(got, ref, what)


def sample_rows(lc, hq: int, tokens, ) -> np.ndarray:
    """Oracle entries (q_row * Hq + head) for the given global q rows, all heads."""
    t = np.asarray(sorted(set(int(x) for x in tokens)), dtype=np.int64)
    return (t[:, None] * hq + np.arange(hq)[None, :]).reshape(-1), t


def tokens_per_workgroup(hq: int, hkv: int) -> int:
    """Query tokens one prefill workgroup covers: 128 packed rows / group size."""
    return 128 // (hq // hkv)


def one_token_per_block(q_len: int, block: int, seed: int):
    """One seeded token from every block of `block` consecutive tokens (so
    every prefill workgroup of the chunk has a row checked), plus the chunk's
    first and last token."""
    g = np.random.default_rng(seed)
    toks = {0, q_len - 1}
    for b0 in range(0, q_len, block):
        toks.add(b0 + int(g.integers(0, min(block, q_len - b0))))
    return sorted(toks)


# Oracle rows computed once per process and shared by the tests of kernels
# that read the same bytes (the widened FP8 and the FP8-MMA prefill).
_ORACLE_ROWS = {}


def oracle_rows_cached(key, case_cpu, rows, launch_idx: int = 0) -> np.ndarray:
    import oracle
    k = (key, launch_idx, hash(np.asarray(rows).tobytes()))
    if k not in _ORACLE_ROWS:
        _ORACLE_ROWS[k] = oracle.attend_rows(case_cpu, rows, launch_idx=launch_idx)
    return _ORACLE_ROWS[k]
