"""GPU checks of the prefill with the KV append fused in
(attn_prefill_hd512_append), through the C ABI.

The chunk's new rows are gathered from a cache the generator built, and the
chunk's slots of both pools are then poisoned with NaN.  The fused call must
give the same output bits and the same pool bytes as attn_append_kv followed
by the prefill over the written pools (so a chunk key read from the pool
before its row was written would show up as a NaN or a changed bit), and
its output must pass the parity gate against the oracle over the built
cache.
"""
import numpy as np
import pytest
import torch

import attn_workloads as W
import oracle
from _gpu_helpers import check_parity, library, out_tensor, sample_rows, sentinel_intact

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
