"""GPU parity of attn_decode_splitk (split kernel + merge) against the CPU oracle.

Fixtures pin split boundaries (kv_len at a split size minus one, equal, plus
one, and shorter than one split), partial pages, batch > 1 and group sizes
1..16, for bf16 and FP8-E4M3 pools; the workspace is NaN-poisoned before each
call so that a partial that is read without being written fails the run.
The batch-64 workload is checked on every output row.
"""
import numpy as np
import pytest
import torch

import attn_workloads as W
import oracle
from _gpu_helpers import check_parity, library, run_decode, sentinel_intact

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def A():
    return library()


def _decode_case(lens, hq, hkv, kv_dtype="bf16", seed=23, **kw):
    return W.build_case("dec", seqs=[(1, L - 1, L) for L in lens], hq=hq, hkv=hkv, seed=seed,
                        out_dtype="fp32", device="cuda", kv_dtype=kv_dtype, extra_pages=2,
                        table_pad=2, **kw)


FIXTURES = [
    # (lens, hq, hkv, keys_per_split)
    ([1, 63, 64, 65], 8, 4, 256),
    ([255, 256, 257, 511, 512, 513], 8, 4, 256),
    ([1000, 3], 16, 1, 256),          # MQA, g = 16
    ([700], 4, 4, 512),               # g = 1
    ([4096, 300, 2049], 8, 4, 0),     # library default split
]


@pytest.mark.parametrize("fx", FIXTURES, ids=lambda f: f"{f[0]}-{f[1]}x{f[2]}-s{f[3]}")
@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8_e4m3"])
def test_decode_fixtures(A, fx, kv_dtype):
    lens, hq, hkv, kps = fx
    case = _decode_case(lens, hq, hkv, kv_dtype)
    out = run_decode(A, case, keys_per_split=kps)
    ref = oracle.attend_all(case.to("cpu"))
    check_parity(out, ref, f"decode {lens} {hq}/{hkv} {kv_dtype} split={kps}")


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8_e4m3"])
def test_decode_b64(A, kv_dtype):
    case = W.decode_b64(device="cuda", kv_dtype=kv_dtype)
    out = run_decode(A, case)
    ref = oracle.attend_all(case.to("cpu"))
    raw, mean = check_parity(out, ref, f"decode_b64 {kv_dtype}")
    d = out.float().cpu().numpy().astype(np.float64) - ref
    rel_l2 = np.linalg.norm(d) / np.linalg.norm(ref)
    print(f"[parity] decode_b64 {kv_dtype} rel_l2={rel_l2:.3e}")


def test_decode_q0_v1_exactly_one_at_28k(A):
    case = _decode_case([28672, 4096], 8, 4, q_zero=True, v_one=True)
    out = run_decode(A, case)
    assert bool((out == 1.0).all())


def test_decode_deterministic(A):
    case = _decode_case([5000, 12345, 64], 8, 4)
    a = run_decode(A, case, keys_per_split=512)
    b = run_decode(A, case, keys_per_split=512)
    assert torch.equal(a, b)


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8_e4m3"])
def test_decode_b64_deterministic_ten_calls(A, kv_dtype):
    # the batch-64 workload, ten calls with the library's default split: the
    # same bits every time (the merge order and every partial are fixed)
    case = W.decode_b64(device="cuda", kv_dtype=kv_dtype)
    a = run_decode(A, case, poison_ws=False)
    for i in range(9):
        b = run_decode(A, case, poison_ws=False)
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"call {i + 2} differs"


def test_decode_workspace_too_small(A):
    case = _decode_case([300], 8, 4)
    lc = case.launches[0]
    out = torch.empty((1, 8, 512), dtype=torch.float32, device="cuda")
    ws = torch.empty(16, dtype=torch.float32, device="cuda")
    with pytest.raises(A.AttnError):
        A.decode(lc.q[:1], case.k_pool, case.v_pool, case.page_table, lc.kv_len, out, ws,
                 max_kv_len=300, softmax_scale=case.softmax_scale)
