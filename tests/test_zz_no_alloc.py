"""attn_decode_splitk_ex_noalloc (partials in the library's static device
scratch) against attn_decode_splitk_ex (caller workspace), through the C ABI.

Two calls in a row on one process: the batch-64 decode workload, then a
smaller call (3 sequences, 2 tokens each, an FP8 pool, sinks and the
log-sum-exp) that reuses the scratch the first call left behind.  The two
entry points run the same kernels on the same plan, so outputs and LSE must
be bitwise equal; the first call is also held to the parity gate.
"""
import numpy as np
import pytest
import torch

import attn_workloads as W
import oracle
from _gpu_helpers import check_parity, library, out_tensor

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def A():
    return library()


def _pair(A, case, q_len=1, sinks=None, with_lse=False):
    lc = case.launches[0]
    B = lc.batch
    rows = B * q_len
    hq = case.num_q_heads
    outs, lses = [], []
    for noalloc in (False, True):
        out = out_tensor(rows, hq, case.out_dtype)
        lse = torch.full((rows, hq), float("nan"), device="cuda") if with_lse else None
        kw = dict(max_kv_len=lc.max_kv_len, softmax_scale=case.softmax_scale,
                  kv_dtype=case.kv_dtype, k_scale=case.k_scale, v_scale=case.v_scale,
                  q_len=q_len, sinks=sinks, lse=lse)
        if noalloc:
            A.decode_noalloc(lc.q[:rows], case.k_pool, case.v_pool, case.page_table, lc.kv_len,
                             out, **kw)
        else:
            n = A.decode_workspace_size(B, hq, case.num_kv_heads, lc.max_kv_len, 0, q_len=q_len)
            ws = torch.full((n // 4,), float("nan"), device="cuda")
            A.decode(lc.q[:rows], case.k_pool, case.v_pool, case.page_table, lc.kv_len, out, ws,
                     **kw)
        torch.cuda.synchronize()
        outs.append(out)
        lses.append(lse)
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16)), \
        "no-alloc output differs from the workspace entry point's"
    if with_lse:
        assert torch.equal(lses[0].view(torch.int32), lses[1].view(torch.int32)), \
            "no-alloc log-sum-exp differs"
    return outs[1]


def test_noalloc_matches_workspace_entry_point_two_calls(A):
    print("[case] noalloc call 1: decode_b64 bf16", flush=True)
    big = W.decode_b64(device="cuda")
    got = _pair(A, big)
    ref = oracle.attend_all(big.to("cpu"))
    check_parity(got, ref, "noalloc decode_b64")
    del big
    print("[case] noalloc call 2: 3 sequences x 2 tokens, FP8, sinks, lse", flush=True)
    lens = [700, 64, 1500]
    small = W.build_case("noalloc_small", seqs=[(2, L - 2, L) for L in lens], hq=8, hkv=4,
                         seed=9, out_dtype="fp32", device="cuda", kv_dtype="fp8_e4m3")
    sinks = torch.as_tensor(np.float32([0.5, -1.0, 2.0, 0.0, 1.5, -0.5, 3.0, 0.25]),
                            device="cuda")
    _pair(A, small, q_len=2, sinks=sinks, with_lse=True)


@pytest.mark.parametrize("q_len", [5, 7])
def test_noalloc_wide_multi_token_decode(A, q_len):
    # g = 8: 5 tokens are three column blocks of the decode kernels, 7 tokens
    # (56 columns) run as split-K prefill, the no-alloc call with its row
    # offsets and partials in the static scratch
    print(f"[case] noalloc multi-token: 4 sequences x {q_len} tokens, 32/4 heads, bf16",
          flush=True)
    lens = [257, 1000, 64, 2049]
    case = W.build_case("noalloc_wide", seqs=[(q_len, L - q_len, L) for L in lens], hq=32,
                        hkv=4, seed=13, out_dtype="fp32", device="cuda")
    got = _pair(A, case, q_len=q_len, with_lse=True)
    ref = oracle.attend_all(case.to("cpu"))
    check_parity(got, ref, f"noalloc decode q_len={q_len} g=8")
