"""GPU parity of attn_prefill_hd512 against the CPU oracle (through the C ABI).

Small shapes are compared element by element on every output; the measured
workloads at full size are compared on sampled query rows (all heads of each
sampled row, the first and last rows of the chunk included) and through
properties that hold at any size (q = 0 with V = 1 gives exactly 1).  Every
case also checks that padding rows of the output stay untouched and that
NaN-poisoned page slots, spare pages and table padding never leak in.
"""
import numpy as np
import pytest
import torch

import attn_workloads as W
import oracle
from _gpu_helpers import (check_parity, check_parity_any, check_parity_floor_case,
                          floor_breaks_gate, library, one_token_per_block,
                          oracle_rows_cached, run_prefill, sample_rows, sentinel_intact,
                          tokens_per_workgroup)

pytestmark = pytest.mark.gpu


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
    # (seqs (q_len, q_start, kv_len), hq, hkv)
    ([(1, 0, 1)], 8, 1),                          # one row, one key
    ([(37, 0, 37)], 8, 1),                        # ragged tile, partial page
    ([(100, 28, 128)], 4, 4),                     # MHA (g = 1), offset chunk
    ([(64, 64, 200)], 16, 8),                     # g = 2, keys past the chunk's end masked
    ([(19, 5, 24), (70, 130, 200), (1, 63, 64)], 12, 4),  # g = 3 (rows left unused), batch 3
    ([(130, 0, 130), (7, 300, 307)], 16, 1),      # g = 16 (8 tokens per workgroup)
    ([(129, 2000, 2129)], 32, 4),                 # g = 8, long prefix, one-row tail tile
]


@pytest.mark.parametrize("shape", SMALL, ids=lambda s: f"{s[0]}-{s[1]}x{s[2]}")
@pytest.mark.parametrize("out_dtype", ["fp32", "bf16"])
def test_small_shapes(A, shape, out_dtype):
    seqs, hq, hkv = shape
    case = W.build_case("small", seqs=seqs, hq=hq, hkv=hkv, seed=17, out_dtype=out_dtype,
                        device="cuda", q_pad_rows=3, extra_pages=2, table_pad=2)
    lc = case.launches[0]
    ref = oracle.attend_all(case.to("cpu"))

    def run(dt):
        out = run_prefill(A, case, out_dtype=dt, pad_rows=5)
        assert sentinel_intact(out[lc.total_q:]), "rows past total_q were written"
        return out[:lc.total_q]
    check_parity_any(run, ref, f"small {seqs} {hq}/{hkv} out={out_dtype}", out_dtype)


def test_tiny_prefill_mqa_256(A):
    case = W.tiny_prefill_mqa(device="cuda")
    _full_check(A, case)


@pytest.mark.parametrize("out_dtype", ["bf16", "fp32"])
def test_chunk_prefill_2048(A, out_dtype):
    case = W.chunk_prefill_2k(device="cuda")
    _full_check(A, case, out_dtype=out_dtype)


def test_chunk_prefill_8192_at_8192_every_workgroup(A):
    # one query token from every workgroup's 16-token block (all 32 heads, so
    # every (token block, KV head) workgroup of the 8192-row chunk), plus the
    # first and last token
    case = W.chunk_prefill_8k_at_8k(device="cuda")
    lc = case.launches[0]
    out = run_prefill(A, case, pad_rows=64)
    assert sentinel_intact(out[lc.total_q:])
    tokens = one_token_per_block(lc.total_q, tokens_per_workgroup(32, 4), seed=3)
    rows, toks = sample_rows(lc, case.num_q_heads, tokens)
    ref = oracle_rows_cached(case.name, case.to("cpu"), rows).reshape(len(toks),
                                                                      case.num_q_heads, -1)
    check_parity(out[torch.as_tensor(toks, device="cuda")], ref,
                 f"chunk_8192_at_8192 every workgroup ({len(toks)} tokens)")


@pytest.mark.parametrize("kv_dtype,fp8_mma", [("bf16", False), ("fp8_e4m3", False),
                                              ("fp8_e4m3", True)])
def test_chunk_prefill_8192_at_8192_late_keys_every_workgroup(A, kv_dtype, fp8_mma):
    # every row sees two or three keys far above what it saw before them
    # (38, 76 and 151 nats), so every workgroup raises its rows' softmax
    # reference two or three times; one token of every workgroup checked
    # (the rows are dominated by one key, so their outputs are that key's
    # value: over an E4M3 pool the dequantised values' own bf16 rounding can
    # break the gate, and the floor-case check then gates the fp32 output)
    case = W.chunk_prefill_8k_at_8k_late_keys(device="cuda", kv_dtype=kv_dtype)
    lc = case.launches[0]
    out = run_prefill(A, case, pad_rows=64, fp8_mma=fp8_mma)
    assert sentinel_intact(out[lc.total_q:])
    tokens = one_token_per_block(lc.total_q, tokens_per_workgroup(32, 4), seed=8)
    rows, toks = sample_rows(lc, case.num_q_heads, tokens)
    ref = oracle_rows_cached(case.name, case.to("cpu"), rows).reshape(len(toks),
                                                                      case.num_q_heads, -1)
    sel = torch.as_tensor(toks, device="cuda")
    what = f"{case.name} mma={fp8_mma} every workgroup ({len(toks)} tokens)"
    if floor_breaks_gate(ref):
        out32 = run_prefill(A, case, out_dtype="fp32", fp8_mma=fp8_mma)
        check_parity_floor_case(out[sel], out32[sel], ref, what)
    else:
        check_parity(out[sel], ref, what)


@pytest.mark.parametrize("li", range(8))
def test_long_mqa_32k_chunk_every_workgroup(A, li):
    # chunk li of the 32K prompt: one token from every 8-token workgroup block
    # (g = 16), all 16 heads, plus the chunk's first and last token
    case = W.long_mqa_32k(device="cuda")
    lc = case.launches[li]
    out = run_prefill(A, case, li=li, pad_rows=3)
    assert sentinel_intact(out[lc.total_q:])
    tokens = one_token_per_block(lc.total_q, tokens_per_workgroup(16, 1), seed=4 + li)
    rows, toks = sample_rows(lc, case.num_q_heads, tokens)
    ref = oracle_rows_cached(case.name, case.to("cpu"), rows, launch_idx=li).reshape(
        len(toks), case.num_q_heads, -1)
    check_parity(out[torch.as_tensor(toks, device="cuda")], ref,
                 f"long_mqa chunk {li} every workgroup ({len(toks)} tokens)")


def test_long_mqa_32k_q0_v1_is_exactly_one(A):
    case = W.long_mqa_32k(device="cuda", q_zero=True, v_one=True)
    for li, lc in enumerate(case.launches):
        out = run_prefill(A, case, li=li)
        assert bool((out[:lc.total_q] == 1.0).all()), f"chunk {li}: output differs from 1"


@pytest.mark.parametrize("kv_dtype,fp8_mma", [("bf16", False), ("fp8_e4m3", False),
                                              ("fp8_e4m3", True)])
def test_deterministic_bitwise(A, kv_dtype, fp8_mma):
    # ten launches of the 2048-row chunk give identical bits: the per-row
    # accumulation order is fixed, so a difference between runs would point
    # at an LDS hand-off that depends on timing
    case = W.chunk_prefill_2k(device="cuda", kv_dtype=kv_dtype)
    a = run_prefill(A, case, fp8_mma=fp8_mma)
    for i in range(9):
        b = run_prefill(A, case, fp8_mma=fp8_mma)
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"launch {i + 2} differs"


def test_empty_launch_and_bad_arguments(A):
    case = W.tiny_prefill_mqa(device="cuda")
    lc = case.launches[0]
    out = torch.zeros((lc.total_q, 8, 512), dtype=torch.float32, device="cuda")
    with pytest.raises(A.AttnError):
        A.prefill(lc.q, case.k_pool, case.v_pool, case.page_table, lc.cu_seqlens_q, lc.q_start,
                  lc.kv_len, out, total_q=lc.total_q, max_q_len=lc.total_q + 1,
                  softmax_scale=case.softmax_scale)
    A.prefill(lc.q, case.k_pool, case.v_pool, case.page_table, lc.cu_seqlens_q, lc.q_start,
              lc.kv_len, out, total_q=0, max_q_len=0, softmax_scale=case.softmax_scale)
    torch.cuda.synchronize()
    assert not out.any()


def test_many_ragged_sequences(A):
    # 40 sequences with every kind of offset: chunks at 0, mid-page, on page
    # boundaries, single rows, rows longer than one workgroup's 16 tokens
    g = np.random.default_rng(79)
    seqs = []
    for i in range(40):
        ql = int(g.integers(1, 200))
        st = int(g.choice([0, 63, 64, 65, int(g.integers(0, 3000))]))
        seqs.append((ql, st, st + ql))
    case = W.build_case("ragged40", seqs=seqs, hq=16, hkv=2, seed=79, out_dtype="fp32",
                        device="cuda", q_pad_rows=3, extra_pages=2, table_pad=2)
    _full_check(A, case, pad_rows=3)
