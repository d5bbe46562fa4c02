"""GPU behaviour on NaN inside the live key band, through the C ABI.

A NaN key row makes exactly the rows that attend to it NaN, in the oracle
(the materialised softmax) and in the kernels alike: masked scores are
replaced by -inf before the softmax.  A NaN score makes its block's sum of
p non-finite, which sends the prefill through its reference raise once for
that block (no loop), so these calls must also return.  A NaN value row makes every row
that attends to it NaN, and may also poison rows of a workgroup that loads
its 64-key tile without attending to it (masked keys enter P.V with p = 0,
and 0 x NaN = NaN); rows whose workgroup never loads that tile, and other
sequences, must be unaffected and pass the parity gate.
"""
import numpy as np
import pytest
import torch

import attn_workloads as W
import oracle
from _gpu_helpers import check_parity, library, run_decode, run_prefill

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def A():
    return library()


def _plant_nan(case, b, j, kvh, which, kv_dtype):
    page = int(case.page_table[b, j // 64])
    pool = case.k_pool if which == "k" else case.v_pool
    if kv_dtype == "bf16":
        pool[page, kvh, j % 64, :] = float("nan")
    else:
        pool[page, kvh, j % 64, :] = 0x7F     # E4M3FN NaN


def _compare(got, ref, what):
    g = got.float().cpu().numpy()
    nan_ref = np.isnan(ref).any(axis=-1)
    nan_got = np.isnan(g).any(axis=-1)
    assert nan_ref.any(), f"{what}: the fixture should poison some rows"
    assert np.array_equal(nan_ref, nan_got), f"{what}: NaN rows differ from the oracle's"
    keep = ~nan_ref
    check_parity(got[torch.as_tensor(keep, device=got.device)], ref[keep], what)


PREFILL_PATHS = [("bf16", False), ("fp8_e4m3", False), ("fp8_e4m3", True)]


@pytest.mark.parametrize("kv_dtype,mma", PREFILL_PATHS, ids=["bf16", "fp8", "fp8_mma"])
def test_prefill_nan_key_poisons_exactly_its_attenders(A, kv_dtype, mma):
    case = W.build_case("nan_pf", seqs=[(100, 200, 300), (50, 0, 50)], hq=16, hkv=2, seed=83,
                        out_dtype="fp32", device="cuda", kv_dtype=kv_dtype)
    # key 250 of sequence 0, KV head 1: chunk rows at positions >= 250 of
    # heads 8..15 see it; positions 200..249 and sequence 1 do not
    _plant_nan(case, 0, 250, 1, "k", kv_dtype)
    out = run_prefill(A, case, fp8_mma=mma)
    lc = case.launches[0]
    ref = oracle.attend_all(case.to("cpu"))
    _compare(out[:lc.total_q], ref, f"prefill NaN k {kv_dtype} mma={mma}")


@pytest.mark.parametrize("kv_dtype,mma", PREFILL_PATHS, ids=["bf16", "fp8", "fp8_mma"])
def test_prefill_nan_value_stays_in_its_tile(A, kv_dtype, mma):
    hq, hkv = 16, 2
    case = W.build_case("nan_pf_v", seqs=[(100, 150, 250), (50, 0, 50)], hq=hq, hkv=hkv,
                        seed=83, out_dtype="fp32", device="cuda", kv_dtype=kv_dtype)
    j = 230                                   # tile 3: keys 192..255
    _plant_nan(case, 0, j, 1, "v", kv_dtype)
    out = run_prefill(A, case, fp8_mma=mma)
    lc = case.launches[0]
    ref = oracle.attend_all(case.to("cpu"))
    got = out[:lc.total_q].float().cpu().numpy()
    nan_got = np.isnan(got).any(axis=-1)
    nan_ref = np.isnan(ref).any(axis=-1)
    assert nan_ref.any() and bool(nan_got[nan_ref].all()), "an attending row is not NaN"
    # a workgroup covers 128 / g consecutive tokens; one whose last token
    # lies before the NaN key's tile never loads it
    tok_per_wg = 128 // (hq // hkv)
    pos = np.concatenate([np.arange(st, st + ql) for ql, st in zip(lc.q_lens, lc.q_starts)])
    seq = np.concatenate([np.full(ql, b) for b, ql in enumerate(lc.q_lens)])
    clean = (seq != 0) | (pos + tok_per_wg <= (j // 64) * 64)
    assert clean.sum() >= 50 + 16
    assert not nan_got[clean].any(), "a row whose workgroup never loads the tile is NaN"
    keep = ~nan_got
    keep[~clean] = False
    check_parity(out[:lc.total_q][torch.as_tensor(keep, device="cuda")], ref[keep],
                 f"prefill NaN v {kv_dtype} mma={mma}, clean rows")


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8_e4m3"])
@pytest.mark.parametrize("which", ["k", "v"])
def test_decode_nan_in_a_visible_key(A, kv_dtype, which):
    # one token per sequence sees every key, so exactly the oracle's NaN rows
    case = W.build_case("nan_dec", seqs=[(1, 4999, 5000), (1, 2999, 3000), (1, 700, 701)],
                        hq=8, hkv=4, seed=89, out_dtype="bf16", device="cuda", kv_dtype=kv_dtype)
    _plant_nan(case, 1, 1234, 2, which, kv_dtype)   # sequence 1, KV head 2 (query heads 4, 5)
    out = run_decode(A, case)
    ref = oracle.attend_all(case.to("cpu"))
    _compare(out, ref, f"decode NaN {which} {kv_dtype}")
