"""GPU checks of the prefill with the KV append fused in
(attn_prefill_hd512_append, bf16 pool) and of its E4M3 form
(attn_prefill_hd512_e4m3_mma_append: the append kernel, then the FP8-MMA
prefill), through the C ABI.

The chunk's new rows are gathered from a cache the generator built, and the
chunk's slots of both pools are then poisoned with NaN.  The fused call must
give the same output bits and the same pool bytes as attn_append_kv followed
by the prefill over the written pools (so a chunk key read from the pool
before its row was written would show up as a NaN or a changed bit), and
its output must pass the parity gate against the oracle over the built
cache.
"""
import dataclasses

import numpy as np
import pytest
import torch

import attn_workloads as W
import oracle
from oracle import kv_append
from _gpu_helpers import (check_parity, check_parity_floor_case, floor_breaks_gate, library,
                          out_tensor, sample_rows, sentinel_intact)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def A():
    return library()


def _chunk_rows(case, lc):
    """New K/V rows [total_q, Hkv, 512] of the chunk, read from the built
    pools, and the (page, slot) of each."""
    pages, slots = [], []
    for b, (ql, st) in enumerate(zip(lc.q_lens, lc.q_starts)):
        pos = torch.arange(st, st + ql, device="cuda")
        pages.append(case.page_table[b, pos // 64].long())
        slots.append(pos % 64)
    pages, slots = torch.cat(pages), torch.cat(slots)
    kn = case.k_pool[pages, :, slots, :].contiguous()
    vn = case.v_pool[pages, :, slots, :].contiguous()
    return kn, vn, pages, slots


def _poisoned_pools(case, pages, slots):
    kp, vp = case.k_pool.clone(), case.v_pool.clone()
    kp[pages, :, slots, :] = float("nan")
    vp[pages, :, slots, :] = float("nan")
    return kp, vp


def run_both(A, case, out_dtype, sinks=None, with_lse=False, pad_rows=2):
    """(fused out, fused lse, fused pools), (unfused out, lse, pools)."""
    lc = case.launches[0]
    hq = case.num_q_heads
    kn, vn, pages, slots = _chunk_rows(case, lc)
    sk = None if sinks is None else torch.as_tensor(sinks, device="cuda")
    res = []
    for fused in (True, False):
        kp, vp = _poisoned_pools(case, pages, slots)
        out = out_tensor(lc.total_q, hq, out_dtype, pad_rows)
        lse = torch.full((lc.total_q, hq), float("nan"), device="cuda") if with_lse else None
        if fused:
            A.prefill_append(lc.q, kn, vn, kp, vp, case.page_table, lc.cu_seqlens_q, lc.q_start,
                             lc.kv_len, out, total_q=lc.total_q, max_q_len=lc.max_q_len,
                             softmax_scale=case.softmax_scale, sinks=sk, lse=lse)
        else:
            A.append_kv(kn, vn, case.page_table, lc.cu_seqlens_q, lc.q_start, kp, vp)
            A.prefill(lc.q, kp, vp, case.page_table, lc.cu_seqlens_q, lc.q_start, lc.kv_len,
                      out, total_q=lc.total_q, max_q_len=lc.max_q_len,
                      softmax_scale=case.softmax_scale, sinks=sk, lse=lse)
        torch.cuda.synchronize()
        res.append((out, lse, kp, vp))
    return res


def _same_bits(a, b):
    if a.dtype == torch.uint8:
        return torch.equal(a, b)
    if a.dtype == torch.float32:
        return torch.equal(a.view(torch.int32), b.view(torch.int32))
    return torch.equal(a.view(torch.int16), b.view(torch.int16))


def assert_fused_equals_unfused(fused, unfused, what):
    (o1, l1, k1, v1), (o2, l2, k2, v2) = fused, unfused
    assert _same_bits(o1, o2), f"{what}: output bits differ from append + prefill"
    if l1 is not None:
        assert _same_bits(l1, l2), f"{what}: lse bits differ"
    assert _same_bits(k1, k2) and _same_bits(v1, v2), f"{what}: pools differ"


SHAPES = [
    # (seqs (q_len, q_start, kv_len), hq, hkv)
    ([(37, 300, 337)], 8, 1),                                     # chunk starts mid-page
    ([(100, 1000, 1100), (7, 0, 7), (64, 192, 256)], 32, 4),       # ragged, page-aligned end
    ([(129, 2000, 2129), (1, 639, 640)], 32, 4),                  # one-row tail block, q_len 1
    ([(19, 5, 24), (70, 1130, 1200)], 12, 4),                     # g = 3
    ([(130, 0, 130), (3, 4000, 4003)], 16, 1),                    # whole prompt in the chunk, g = 16
    ([(3, 4001, 4004), (9, 62, 71), (200, 57, 257)], 8, 2),       # chunks inside and across 8-key groups
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"{s[0][0][0]}x{len(s[0])}-{s[1]}x{s[2]}")
@pytest.mark.parametrize("out_dtype", ["fp32", "bf16"])
def test_fused_append_equals_append_then_prefill(A, shape, out_dtype):
    seqs, hq, hkv = shape
    case = W.build_case("fused_append", seqs=seqs, hq=hq, hkv=hkv, seed=61, out_dtype=out_dtype,
                        device="cuda", q_pad_rows=2, extra_pages=2, table_pad=2)
    fused, unfused = run_both(A, case, out_dtype)
    what = f"fused append {seqs} {hq}/{hkv} {out_dtype}"
    assert_fused_equals_unfused(fused, unfused, what)
    lc = case.launches[0]
    assert sentinel_intact(fused[0][lc.total_q:]), "rows past total_q were written"
    ref = oracle.attend_all(case.to("cpu"))
    check_parity(fused[0][:lc.total_q], ref, what)


def test_fused_append_with_sinks_and_lse(A):
    case = W.build_case("fused_append_ex", seqs=[(90, 410, 500), (33, 0, 33)], hq=16, hkv=2,
                        seed=67, out_dtype="fp32", device="cuda", q_pad_rows=2)
    sinks = np.random.default_rng(3).uniform(-2.0, 6.0, 16).astype(np.float32)
    fused, unfused = run_both(A, case, "fp32", sinks=sinks, with_lse=True)
    assert_fused_equals_unfused(fused, unfused, "fused append, sinks + lse")
    lc = case.launches[0]
    ref, ref_lse = oracle.attend_all_lse(case.to("cpu"), sinks=sinks)
    check_parity(fused[0][:lc.total_q], ref, "fused append, sinks")
    err = float(np.abs(fused[1].cpu().numpy() - ref_lse).max())
    assert err <= 2e-3, f"lse error {err}"


def test_fused_append_chunk_2k(A):
    # 2048 rows over 2048 keys: every key tile is the chunk's own, 512 workgroups
    case = W.chunk_prefill_2k(device="cuda")
    fused, unfused = run_both(A, case, "fp32", pad_rows=0)
    assert_fused_equals_unfused(fused, unfused, "fused append, chunk 2048")
    lc = case.launches[0]
    rows, toks = sample_rows(lc, case.num_q_heads, [0, 1, 63, 64, 1000, 2046, 2047])
    ref = oracle.attend_rows(case.to("cpu"), rows).reshape(len(toks), case.num_q_heads, -1)
    check_parity(fused[0][torch.as_tensor(toks, device="cuda")], ref, "fused append 2048 sampled")


def test_fused_append_chunk_8k_at_8k(A):
    # one chunk of 8192 rows at positions 8192..16383, bf16 output
    case = W.chunk_prefill_8k_at_8k(device="cuda")
    fused, unfused = run_both(A, case, "bf16", pad_rows=0)
    assert_fused_equals_unfused(fused, unfused, "fused append, chunk 8192 at 8192")
    lc = case.launches[0]
    g = np.random.default_rng(8)
    tokens = [0, 1, 4095, 8190, 8191] + g.integers(0, lc.total_q, 3).tolist()
    rows, toks = sample_rows(lc, case.num_q_heads, tokens)
    ref = oracle.attend_rows(case.to("cpu"), rows).reshape(len(toks), case.num_q_heads, -1)
    check_parity(fused[0][torch.as_tensor(toks, device="cuda")], ref,
                 "fused append 8192 at 8192 sampled")


# ---- E4M3 pool: attn_prefill_hd512_e4m3_mma_append ---------------------------
#
# The new rows are bf16 rows of a bf16 build of the same shape; the E4M3
# pool's chunk slots are poisoned with the NaN code.  The expected pool is
# the append oracle's (x / scale in fp32, saturated, nearest even) over the
# poisoned pool, and the expected output is the oracle's attention over that
# expected pool.

def _fp8_cases(name, seqs, hq, hkv, seed, out_dtype, **kw):
    """An E4M3 case and a bf16 case of the same shape (its rows are the new rows)."""
    kw.update(seqs=seqs, hq=hq, hkv=hkv, seed=seed, out_dtype=out_dtype, device="cuda")
    return (W.build_case(name, kv_dtype="fp8_e4m3", **kw), W.build_case(name, **kw))


def run_both_fp8(A, fcase, bcase, out_dtype, sinks=None, with_lse=False, pad_rows=2):
    """As run_both over the E4M3 pool: the one call against attn_append_kv
    (E4M3) + the FP8-MMA prefill; also returns the oracle's expected case
    (CPU, pools as the append oracle writes them)."""
    lc = fcase.launches[0]
    hq = fcase.num_q_heads
    kn, vn, pages, slots = _chunk_rows(bcase, bcase.launches[0])
    sk = None if sinks is None else torch.as_tensor(sinks, device="cuda")
    kw = dict(kv_dtype="fp8_e4m3", k_scale=fcase.k_scale, v_scale=fcase.v_scale)
    k0, v0 = fcase.k_pool.clone(), fcase.v_pool.clone()
    k0[pages, :, slots, :] = W.E4M3_NAN_BYTE
    v0[pages, :, slots, :] = W.E4M3_NAN_BYTE
    res = []
    for fused in (True, False):
        kp, vp = k0.clone(), v0.clone()
        out = out_tensor(lc.total_q, hq, out_dtype, pad_rows)
        lse = torch.full((lc.total_q, hq), float("nan"), device="cuda") if with_lse else None
        if fused:
            A.prefill_append(lc.q, kn, vn, kp, vp, fcase.page_table, lc.cu_seqlens_q,
                             lc.q_start, lc.kv_len, out, total_q=lc.total_q,
                             max_q_len=lc.max_q_len, softmax_scale=fcase.softmax_scale,
                             sinks=sk, lse=lse, **kw)
        else:
            A.append_kv(kn, vn, fcase.page_table, lc.cu_seqlens_q, lc.q_start, kp, vp, **kw)
            A.prefill(lc.q, kp, vp, fcase.page_table, lc.cu_seqlens_q, lc.q_start, lc.kv_len,
                      out, total_q=lc.total_q, max_q_len=lc.max_q_len,
                      softmax_scale=fcase.softmax_scale, sinks=sk, lse=lse, fp8_mma=True, **kw)
        torch.cuda.synchronize()
        res.append((out, lse, kp, vp))
    cpu = fcase.to("cpu")
    want_k, want_v = kv_append.append(
        k0.cpu().numpy(), v0.cpu().numpy(), kn.cpu(), vn.cpu(), cpu.page_table.numpy(),
        cpu.launches[0].cu_seqlens_q.numpy(), cpu.launches[0].q_start.numpy(), "fp8_e4m3",
        fcase.k_scale, fcase.v_scale)
    expect = dataclasses.replace(cpu, k_pool=torch.from_numpy(want_k),
                                 v_pool=torch.from_numpy(want_v))
    return res[0], res[1], expect


def assert_fp8_pools_written(fused, expect, what):
    _, _, kp, vp = fused
    assert torch.equal(kp.cpu(), expect.k_pool) and torch.equal(vp.cpu(), expect.v_pool), \
        f"{what}: the pool differs from the append oracle's"


@pytest.mark.parametrize("shape", SHAPES[:4], ids=lambda s: f"{s[0][0][0]}x{len(s[0])}-{s[1]}x{s[2]}")
@pytest.mark.parametrize("out_dtype", ["fp32", "bf16"])
def test_e4m3_append_prefill_equals_append_then_prefill(A, shape, out_dtype):
    seqs, hq, hkv = shape
    fcase, bcase = _fp8_cases("fused_append_fp8", seqs, hq, hkv, 61, out_dtype, q_pad_rows=2,
                              extra_pages=2, table_pad=2)
    fused, unfused, expect = run_both_fp8(A, fcase, bcase, out_dtype)
    what = f"E4M3 append + FP8-MMA prefill {seqs} {hq}/{hkv} {out_dtype}"
    assert_fused_equals_unfused(fused, unfused, what)
    assert_fp8_pools_written(fused, expect, what)
    lc = fcase.launches[0]
    assert sentinel_intact(fused[0][lc.total_q:]), "rows past total_q were written"
    ref = oracle.attend_all(expect)
    if out_dtype == "bf16" and floor_breaks_gate(ref):
        # the bf16 rounding of the exact result alone breaks the gate: the
        # same call into an fp32 output is gated, and the bf16 output must be
        # its rounding
        f32, _, _ = run_both_fp8(A, fcase, bcase, "fp32")
        check_parity_floor_case(fused[0][:lc.total_q], f32[0][:lc.total_q], ref, what)
    else:
        check_parity(fused[0][:lc.total_q], ref, what)


def test_e4m3_append_prefill_with_sinks_and_lse(A):
    fcase, bcase = _fp8_cases("fused_append_fp8_ex", [(90, 410, 500), (33, 0, 33)], 16, 2, 67,
                              "fp32", q_pad_rows=2)
    sinks = np.random.default_rng(3).uniform(-2.0, 6.0, 16).astype(np.float32)
    fused, unfused, expect = run_both_fp8(A, fcase, bcase, "fp32", sinks=sinks, with_lse=True)
    assert_fused_equals_unfused(fused, unfused, "E4M3 append + prefill, sinks + lse")
    assert_fp8_pools_written(fused, expect, "E4M3 append + prefill, sinks + lse")
    lc = fcase.launches[0]
    ref, ref_lse = oracle.attend_all_lse(expect, sinks=sinks)
    check_parity(fused[0][:lc.total_q], ref, "E4M3 append + prefill, sinks")
    err = float(np.abs(fused[1].cpu().numpy() - ref_lse).max())
    assert err <= 2e-3, f"lse error {err}"


def test_e4m3_append_prefill_chunk_2k(A):
    fcase = W.chunk_prefill_2k(device="cuda", kv_dtype="fp8_e4m3")
    bcase = W.chunk_prefill_2k(device="cuda")
    fused, unfused, expect = run_both_fp8(A, fcase, bcase, "fp32", pad_rows=0)
    assert_fused_equals_unfused(fused, unfused, "E4M3 append + prefill, chunk 2048")
    assert_fp8_pools_written(fused, expect, "E4M3 append + prefill, chunk 2048")
    lc = fcase.launches[0]
    rows, toks = sample_rows(lc, fcase.num_q_heads, [0, 1, 63, 64, 1000, 2046, 2047])
    ref = oracle.attend_rows(expect, rows).reshape(len(toks), fcase.num_q_heads, -1)
    check_parity(fused[0][torch.as_tensor(toks, device="cuda")], ref,
                 "E4M3 append + prefill 2048 sampled")


def test_e4m3_append_prefill_chunk_8k_at_8k(A):
    fcase = W.chunk_prefill_8k_at_8k(device="cuda", kv_dtype="fp8_e4m3")
    bcase = W.chunk_prefill_8k_at_8k(device="cuda")
    fused, unfused, expect = run_both_fp8(A, fcase, bcase, "bf16", pad_rows=0)
    assert_fused_equals_unfused(fused, unfused, "E4M3 append + prefill, chunk 8192 at 8192")
    assert_fp8_pools_written(fused, expect, "E4M3 append + prefill, chunk 8192 at 8192")
    lc = fcase.launches[0]
    g = np.random.default_rng(8)
    tokens = [0, 1, 4095, 8190, 8191] + g.integers(0, lc.total_q, 3).tolist()
    rows, toks = sample_rows(lc, fcase.num_q_heads, tokens)
    ref = oracle.attend_rows(expect, rows).reshape(len(toks), fcase.num_q_heads, -1)
    check_parity(fused[0][torch.as_tensor(toks, device="cuda")], ref,
                 "E4M3 append + prefill 8192 at 8192 sampled")
