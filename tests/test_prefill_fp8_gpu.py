"""GPU parity of attn_prefill_hd512_e4m3 (FP8-E4M3 KV cache) against the CPU oracle.

The oracle reads the same E4M3 bytes, widened exactly and multiplied by the
per-tensor scales in fp32 (vLLM flash-attention PR 199, "Summary"), so the
parity gate is the bf16 path's: only the bf16 rounding of P and the
summation order differ.  Small shapes are checked on every output, the
measured shapes on sampled rows, with the same NaN-poisoned padding,
spare pages and table padding as the bf16 tests.
"""
import numpy as np
import pytest
import torch

import attn_workloads as W
import oracle
from _gpu_helpers import (check_parity, check_parity_any, library, one_token_per_block,
                          oracle_rows_cached, run_prefill, sample_rows, sentinel_intact,
                          tokens_per_workgroup)

pytestmark = pytest.mark.gpu

FP8 = "fp8_e4m3"


@pytest.fixture(scope="module")
def A():
    return library()


def _full_check(A, case, out_dtype=None, pad_rows=5, li=0):
    out = run_prefill(A, case, li=li, out_dtype=out_dtype, pad_rows=pad_rows)
    lc = case.launches[li]
    ref = oracle.attend_all(case.to("cpu"), launch_idx=li)
    assert sentinel_intact(out[lc.total_q:]), "rows past total_q were written"
    return check_parity(out[:lc.total_q], ref, f"{case.name}[{li}] out={out.dtype}")


SMALL = [
    ([(1, 0, 1)], 8, 1),
    ([(37, 0, 37)], 8, 1),
    ([(100, 28, 128)], 4, 4),
    ([(64, 64, 200)], 16, 8),
    ([(19, 5, 24), (70, 130, 200), (1, 63, 64)], 12, 4),
    ([(130, 0, 130), (7, 300, 307)], 16, 1),
    ([(129, 2000, 2129)], 32, 4),
]


@pytest.mark.parametrize("shape", SMALL, ids=lambda s: f"{s[0]}-{s[1]}x{s[2]}")
@pytest.mark.parametrize("out_dtype", ["fp32", "bf16"])
def test_small_shapes_fp8(A, shape, out_dtype):
    seqs, hq, hkv = shape
    case = W.build_case("small_fp8", seqs=seqs, hq=hq, hkv=hkv, seed=19, out_dtype=out_dtype,
                        device="cuda", q_pad_rows=3, extra_pages=2, table_pad=2, kv_dtype=FP8)
    lc = case.launches[0]
    ref = oracle.attend_all(case.to("cpu"))

    def run(dt):
        out = run_prefill(A, case, out_dtype=dt, pad_rows=5)
        assert sentinel_intact(out[lc.total_q:]), "rows past total_q were written"
        return out[:lc.total_q]
    # the one-key shape outputs dequantised V rows (|o| up to ~3.5), whose
    # own bf16 rounding breaks the mean-abs bound: check_parity_any gates its
    # fp32 output and requires the bf16 output to be that value rounded
    check_parity_any(run, ref, f"fp8 {seqs} {hq}/{hkv} out={out_dtype}", out_dtype)


def test_chunk_prefill_2048_fp8(A):
    _full_check(A, W.chunk_prefill_2k(device="cuda", kv_dtype=FP8))


def test_chunk_prefill_8192_at_8192_fp8_every_workgroup(A):
    # one query token from every 16-token workgroup block, all 32 heads, plus
    # the first and last token (the oracle rows are shared with the FP8-MMA test)
    case = W.chunk_prefill_8k_at_8k(device="cuda", kv_dtype=FP8)
    lc = case.launches[0]
    out = run_prefill(A, case, pad_rows=64)
    assert sentinel_intact(out[lc.total_q:])
    tokens = one_token_per_block(lc.total_q, tokens_per_workgroup(32, 4), seed=5)
    rows, toks = sample_rows(lc, case.num_q_heads, tokens)
    ref = oracle_rows_cached(case.name, case.to("cpu"), rows).reshape(len(toks),
                                                                      case.num_q_heads, -1)
    check_parity(out[torch.as_tensor(toks, device="cuda")], ref,
                 f"chunk_8192_at_8192_fp8 every workgroup ({len(toks)} tokens)")


@pytest.mark.parametrize("li", range(8))
def test_long_mqa_32k_chunk_fp8_every_workgroup(A, li):
    case = W.long_mqa_32k(device="cuda", kv_dtype=FP8)
    lc = case.launches[li]
    out = run_prefill(A, case, li=li, pad_rows=3)
    assert sentinel_intact(out[lc.total_q:])
    tokens = one_token_per_block(lc.total_q, tokens_per_workgroup(16, 1), seed=6 + li)
    rows, toks = sample_rows(lc, case.num_q_heads, tokens)
    ref = oracle_rows_cached(case.name, case.to("cpu"), rows, launch_idx=li).reshape(
        len(toks), case.num_q_heads, -1)
    check_parity(out[torch.as_tensor(toks, device="cuda")], ref,
                 f"long_mqa_32k fp8 chunk {li} every workgroup ({len(toks)} tokens)")


def test_fp8_q0_v1_matches_dequantised_one(A):
    # q = 0 gives uniform weights; every V element dequantises to the same
    # value v = byte(1 / v_scale) * v_scale, so the output is v (within the
    # fp32 rounding of the final scale multiply), whatever the weights.
    case = W.long_mqa_32k(device="cuda", q_zero=True, v_one=True, kv_dtype=FP8)
    li = 3
    out = run_prefill(A, case, li=li).float().cpu().numpy()
    page0 = int(case.page_table[0, 0].item())
    code = case.v_pool.view(torch.uint8)[page0, 0, 0, 0].item()
    v = float(oracle.e4m3_to_f32(np.array([code], dtype=np.uint8))[0] * np.float32(case.v_scale))
    assert np.isfinite(out).all()
    np.testing.assert_allclose(out, v, rtol=2e-7, atol=0)


def test_fp8_deterministic(A):
    case = W.build_case("det_fp8", seqs=[(300, 100, 400)], hq=32, hkv=4, seed=23,
                        out_dtype="fp32", device="cuda", kv_dtype=FP8)
    a = run_prefill(A, case)
    b = run_prefill(A, case)
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))


def test_fp8_bad_scales(A):
    case = W.build_case("bad_fp8", seqs=[(8, 0, 8)], hq=8, hkv=1, seed=1, out_dtype="fp32",
                        device="cuda", kv_dtype=FP8)
    lc = case.launches[0]
    out = torch.zeros((lc.total_q, 8, 512), device="cuda")
    for ks, vs in ((0.0, 1.0), (1.0, -1.0), (float("nan"), 1.0)):
        with pytest.raises(A.AttnError, match="status 2"):
            A.prefill(lc.q, case.k_pool, case.v_pool, case.page_table, lc.cu_seqlens_q,
                      lc.q_start, lc.kv_len, out, total_q=lc.total_q, max_q_len=lc.max_q_len,
                      softmax_scale=case.softmax_scale, kv_dtype=FP8, k_scale=ks, v_scale=vs)
