"""GPU parity of attn_append_kv against the append oracle: bit-exact pools.

Both sides start from the same NaN-poisoned pools; every slot the chunk does
not own must keep its bytes, and every owned slot must hold exactly the
oracle's bf16 bits or E4M3 codes (same fp32 division, saturation and ties to
even).
"""
import numpy as np
import pytest
import torch

import attn_workloads as W
from oracle import kv_append
from _gpu_helpers import library

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def A():
    return library()


CASES = [
    # (seqs (q_len, q_start, kv_len), hkv)
    ([(1, 0, 1)], 1),
    ([(100, 28, 128), (64, 64, 200), (7, 300, 307)], 4),
    ([(2048, 0, 2048)], 4),
    ([(5, 4091, 4096), (3, 62, 65)], 8),
]


@pytest.mark.parametrize("seqs_hkv", CASES, ids=lambda c: f"{c[0][0]}x{len(c[0])}-hkv{c[1]}")
@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8_e4m3"])
def test_append_is_bit_exact(A, seqs_hkv, kv_dtype):
    seqs, hkv = seqs_hkv
    case = W.build_case("append", seqs=seqs, hq=hkv * 2, hkv=hkv, seed=41, out_dtype="fp32",
                        device="cuda", kv_dtype=kv_dtype, extra_pages=2, table_pad=2)
    lc = case.launches[0]
    g = torch.Generator(device="cuda").manual_seed(7)
    # rows to append (bf16), with a few values far outside the E4M3 range
    kn = (torch.randn(lc.total_q, hkv, 512, device="cuda", generator=g) * 3).to(torch.bfloat16)
    vn = (torch.randn(lc.total_q, hkv, 512, device="cuda", generator=g) * 3).to(torch.bfloat16)
    kn.view(-1)[::997] = 1e4
    vn.view(-1)[::991] = -1e4
    kp, vp = case.k_pool.clone(), case.v_pool.clone()
    A.append_kv(kn, vn, case.page_table, lc.cu_seqlens_q, lc.q_start, kp, vp,
                kv_dtype=kv_dtype, k_scale=case.k_scale, v_scale=case.v_scale)
    torch.cuda.synchronize()
    view = (lambda t: t.view(torch.int16).cpu().numpy().view(np.uint16)) if kv_dtype == "bf16" \
        else (lambda t: t.cpu().numpy())
    want_k, want_v = kv_append.append(
        view(case.k_pool), view(case.v_pool), kn.cpu(), vn.cpu(), case.page_table.cpu().numpy(),
        lc.cu_seqlens_q.cpu().numpy(), lc.q_start.cpu().numpy(), kv_dtype, case.k_scale,
        case.v_scale)
    assert np.array_equal(view(kp), want_k)
    assert np.array_equal(view(vp), want_v)


def test_append_then_prefill_matches_the_prebuilt_cache(A):
    # Writing the chunk's own K/V with append_kv and attending must give the
    # same output as the cache the generator built with those values.
    case = W.build_case("append_pf", seqs=[(256, 256, 512)], hq=16, hkv=2, seed=43,
                        out_dtype="fp32", device="cuda", extra_pages=1)
    lc = case.launches[0]
    table = case.page_table
    # gather the chunk's rows (positions 256..511) from the prebuilt pools
    pos = torch.arange(256, 512, device="cuda")
    pages = table[0, pos // 64].long()
    kn = case.k_pool[pages, :, pos % 64, :].contiguous()
    vn = case.v_pool[pages, :, pos % 64, :].contiguous()
    kp, vp = case.k_pool.clone(), case.v_pool.clone()
    kp[pages, :, pos % 64, :] = float("nan")
    vp[pages, :, pos % 64, :] = float("nan")
    A.append_kv(kn, vn, table, lc.cu_seqlens_q, lc.q_start, kp, vp)
    out_a = torch.empty((lc.total_q, 16, 512), device="cuda")
    out_b = torch.empty_like(out_a)
    for pools, out in (((kp, vp), out_a), ((case.k_pool, case.v_pool), out_b)):
        A.prefill(lc.q, pools[0], pools[1], table, lc.cu_seqlens_q, lc.q_start, lc.kv_len, out,
                  total_q=lc.total_q, max_q_len=lc.max_q_len, softmax_scale=case.softmax_scale)
    torch.cuda.synchronize()
    assert torch.equal(out_a, out_b)
