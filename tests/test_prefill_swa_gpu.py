"""GPU parity of the sliding-window prefill (attn_prefill_swa) against the CPU
oracle, through the C ABI: head dims 256 and 512, windows from 1 key to more
than the cache, ring caches that have wrapped, ragged batches, GQA groups 1
to 16, single-token decode rows, and the 8192-row local-layer chunk sampled.
Padding rows of the output must stay untouched and NaN-poisoned slots
(spare pages, table padding, ring slots no row's band reaches) must never
leak in.
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


def run_swa(A, case, out_dtype=None, pad_rows=3):
    lc = case.launches[0]
    out = out_tensor(lc.total_q, case.num_q_heads, out_dtype or case.out_dtype, pad_rows,
                     head_dim=case.head_dim)
    A.prefill_swa(lc.q, case.k_pool, case.v_pool, case.page_table, lc.cu_seqlens_q, lc.q_start,
                  lc.kv_len, out, total_q=lc.total_q, max_q_len=lc.max_q_len,
                  softmax_scale=case.softmax_scale, window=case.window,
                  ring_pages=case.ring_pages)
    torch.cuda.synchronize()
    return out


SHAPES = [
    # (seqs (q_len, q_start, kv_len), hq, hkv, head_dim, window, ring_pages)
    ([(37, 0, 37)], 8, 1, 256, 16, 0),                       # window inside one tile
    ([(100, 300, 400), (7, 0, 7)], 32, 4, 256, 100, 0),       # window across tiles, ragged
    ([(130, 500, 630), (3, 60, 63)], 16, 1, 256, 1, 0),       # window 1: the row's own value
    ([(64, 1000, 1064)], 4, 4, 256, 2000, 0),                 # window longer than the cache
    ([(70, 4000, 4070), (19, 5, 24)], 12, 4, 256, 200, 5),    # ring of 320 slots, wrapped
    ([(129, 8000, 8129)], 32, 4, 256, 1024, 18),              # ring of 1152 slots, window 1024
    ([(50, 700, 750)], 16, 8, 512, 77, 0),                    # head dim 512 with a window
    ([(40, 2000, 2040), (1, 999, 1000)], 8, 2, 512, 300, 6),  # head dim 512 in a ring
    ([(90, 200, 290)], 8, 4, 256, 0, 0),                      # head dim 256, no window
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"{s[0][0]}-{s[1]}x{s[2]}-d{s[3]}-w{s[4]}-r{s[5]}")
@pytest.mark.parametrize("out_dtype", ["fp32", "bf16"])
def test_swa_small(A, shape, out_dtype):
    seqs, hq, hkv, d, window, ring = shape
    case = W.build_case("swa", seqs=seqs, hq=hq, hkv=hkv, seed=61, out_dtype=out_dtype,
                        device="cuda", q_pad_rows=3, extra_pages=2, table_pad=2, head_dim=d,
                        window=window, ring_pages=ring)
    lc = case.launches[0]
    out = run_swa(A, case)
    assert sentinel_intact(out[lc.total_q:]), "rows past total_q were written"
    ref = oracle.attend_all(case.to("cpu"))
    check_parity(out[:lc.total_q], ref, f"swa {seqs} {hq}/{hkv} d={d} w={window} ring={ring}")


def test_swa_decode_rows(A):
    # single-token rows at the end of long sequences, ring = the window
    lens = [1024, 1025, 5000, 64, 3]
    case = W.build_case("swa_dec", seqs=[(1, L - 1, L) for L in lens], hq=32, hkv=4, seed=67,
                        out_dtype="bf16", device="cuda", head_dim=256, window=1024,
                        ring_pages=16)
    out = run_swa(A, case)
    ref = oracle.attend_all(case.to("cpu"))
    check_parity(out[:len(lens)], ref, "swa decode rows")


def test_swa_q0_v1_is_exactly_one(A):
    case = W.build_case("swa_q0v1", seqs=[(300, 2000, 2300), (40, 0, 40)], hq=16, hkv=2,
                        seed=71, out_dtype="fp32", device="cuda", head_dim=256, window=513,
                        ring_pages=14, q_zero=True, v_one=True)
    lc = case.launches[0]
    out = run_swa(A, case, pad_rows=0)
    assert bool((out[:lc.total_q] == 1.0).all())


def test_swa_prefill_hd256_8192_at_8192_sampled(A):
    case = W.swa_prefill_hd256_8k_at_8k(device="cuda")
    lc = case.launches[0]
    out = run_swa(A, case, pad_rows=16)
    assert sentinel_intact(out[lc.total_q:])
    g = np.random.default_rng(7)
    tokens = [0, 1, 2, 1023, 1024, lc.total_q - 2, lc.total_q - 1] + \
        g.integers(0, lc.total_q, 25).tolist()
    rows, toks = sample_rows(lc, case.num_q_heads, tokens)
    ref = oracle.attend_rows(case.to("cpu"), rows).reshape(len(toks), case.num_q_heads, -1)
    check_parity(out[torch.as_tensor(toks, device="cuda")], ref, "swa 8192 @ 8192 w1024 sampled")


def test_swa_decode_b64_all_rows(A):
    case = W.swa_decode_hd256_b64(device="cuda")
    lc = case.launches[0]
    out = run_swa(A, case, pad_rows=0)
    ref = oracle.attend_all(case.to("cpu"))
    check_parity(out[:lc.total_q], ref, "swa decode b64 w1024")
