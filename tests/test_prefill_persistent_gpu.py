"""GPU parity of the persistent, heaviest-first prefill
(attn_prefill_hd512_persistent) through the C ABI.

Every work unit computes what the one-workgroup-per-unit launch computes,
so the outputs (and LSE) must be bitwise equal to attn_prefill_hd512_ex's,
and they are also held to the parity gate against the oracle: small ragged
batches on every element, the 2048-row chunk on every element, and the
8192-row chunk on one token of every work unit.  The workspace starts
poisoned (the call resets its counter itself), and two calls in a row reuse
it.
"""
import numpy as np
import pytest
import torch

import attn_workloads as W
import oracle
from _gpu_helpers import (check_parity, library, one_token_per_block, oracle_rows_cached,
                          out_tensor, run_prefill, sample_rows, sentinel_intact,
                          tokens_per_workgroup)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def A():
    return library()


def run_persistent(A, case, out_dtype=None, pad_rows=3, sinks=None, with_lse=False):
    lc = case.launches[0]
    hq = case.num_q_heads
    out = out_tensor(lc.total_q, hq, out_dtype or case.out_dtype, pad_rows)
    lse = torch.full((lc.total_q, hq), float("nan"), device="cuda") if with_lse else None
    ws = torch.full((A.prefill_persistent_workspace_size() // 4,), 12345, dtype=torch.int32,
                    device="cuda")
    A.prefill_persistent(lc.q, case.k_pool, case.v_pool, case.page_table, lc.cu_seqlens_q,
                         lc.q_start, lc.kv_len, out, ws, total_q=lc.total_q,
                         max_q_len=lc.max_q_len, softmax_scale=case.softmax_scale,
                         kv_dtype=case.kv_dtype, k_scale=case.k_scale, v_scale=case.v_scale,
                         sinks=sinks, lse=lse)
    torch.cuda.synchronize()
    return out, lse


def _same_bits(a, b, what):
    view = torch.int32 if a.dtype == torch.float32 else torch.int16
    assert torch.equal(a.view(view), b.view(view)), f"{what}: persistent output differs"


SHAPES = [
    ([(37, 0, 37)], 8, 1),
    ([(19, 5, 24), (70, 130, 200), (1, 63, 64)], 12, 4),
    ([(130, 0, 130), (7, 300, 307)], 16, 1),
    ([(129, 2000, 2129), (300, 0, 300), (64, 64, 128)], 32, 4),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"{s[0][0]}-{s[1]}x{s[2]}")
@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8_e4m3"])
@pytest.mark.parametrize("out_dtype", ["fp32", "bf16"])
def test_persistent_small(A, shape, kv_dtype, out_dtype):
    seqs, hq, hkv = shape
    case = W.build_case("pers", seqs=seqs, hq=hq, hkv=hkv, seed=83, out_dtype=out_dtype,
                        device="cuda", kv_dtype=kv_dtype, q_pad_rows=3, extra_pages=2,
                        table_pad=2)
    lc = case.launches[0]
    sinks = torch.as_tensor(np.random.default_rng(5).uniform(-2, 4, hq).astype(np.float32),
                            device="cuda")
    got, lse = run_persistent(A, case, sinks=sinks, with_lse=True)
    assert sentinel_intact(got[lc.total_q:]), "rows past total_q were written"
    ref_out = out_tensor(lc.total_q, hq, out_dtype, 3)
    ref_lse = torch.full((lc.total_q, hq), float("nan"), device="cuda")
    A.prefill(lc.q, case.k_pool, case.v_pool, case.page_table, lc.cu_seqlens_q, lc.q_start,
              lc.kv_len, ref_out, total_q=lc.total_q, max_q_len=lc.max_q_len,
              softmax_scale=case.softmax_scale, kv_dtype=kv_dtype, k_scale=case.k_scale,
              v_scale=case.v_scale, sinks=sinks, lse=ref_lse)
    torch.cuda.synchronize()
    _same_bits(got, ref_out, f"{seqs} {kv_dtype}")
    assert torch.equal(lse.view(torch.int32), ref_lse.view(torch.int32))
    if out_dtype == "fp32":
        ref, _ = oracle.attend_all_lse(case.to("cpu"), sinks=sinks.cpu().numpy())
        check_parity(got[:lc.total_q], ref, f"persistent {seqs} {kv_dtype}")


def test_persistent_chunk_2048_all_elements(A):
    case = W.chunk_prefill_2k(device="cuda")
    got, _ = run_persistent(A, case, pad_rows=0)
    _same_bits(got, run_prefill(A, case), "chunk_2048")
    check_parity(got, oracle.attend_all(case.to("cpu")), "persistent chunk_2048")
    again, _ = run_persistent(A, case, pad_rows=0)   # the counter is reset per call
    _same_bits(again, got, "chunk_2048, second call")


def test_persistent_chunk_8192_every_unit(A):
    case = W.chunk_prefill_8k_at_8k(device="cuda")
    lc = case.launches[0]
    got, _ = run_persistent(A, case, pad_rows=64)
    assert sentinel_intact(got[lc.total_q:])
    _same_bits(got[:lc.total_q], run_prefill(A, case)[:lc.total_q], "chunk_8192")
    tokens = one_token_per_block(lc.total_q, tokens_per_workgroup(32, 4), seed=3)
    rows, toks = sample_rows(lc, case.num_q_heads, tokens)
    ref = oracle_rows_cached(case.name, case.to("cpu"), rows).reshape(len(toks),
                                                                      case.num_q_heads, -1)
    check_parity(got[torch.as_tensor(toks, device="cuda")], ref,
                 f"persistent chunk_8192 every unit ({len(toks)} tokens)")


def test_persistent_rejects_missing_or_small_workspace(A):
    case = W.build_case("pers_bad", seqs=[(8, 0, 8)], hq=8, hkv=1, seed=1, out_dtype="fp32",
                        device="cuda")
    lc = case.launches[0]
    out = torch.zeros((lc.total_q, 8, 512), device="cuda")
    small = torch.zeros(1, dtype=torch.int32, device="cuda")
    with pytest.raises(A.AttnError, match="status 4"):
        A.prefill_persistent(lc.q, case.k_pool, case.v_pool, case.page_table, lc.cu_seqlens_q,
                             lc.q_start, lc.kv_len, out, small, total_q=lc.total_q,
                             max_q_len=lc.max_q_len, softmax_scale=case.softmax_scale)
