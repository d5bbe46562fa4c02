"""Physical page placement never changes a result, on the GPU path.

The method addresses keys by logical position through the page table
(Flash-Decoding for MQA in CUDA, "The starting point"), so where a page sits
in the pool is invisible to the arithmetic.  Two builds of one workload that
differ only in the page permutation (same `seed`, another `page_seed`: the
same Q, K and V, other physical ids, spare NaN pages elsewhere) must give
bitwise-identical outputs from every kernel family: bf16 prefill, the E4M3
pool widened and on the FP8 MFMA, split-K decode over both pools, and the
sliding-window layer over a ring cache.  The oracle's own pin of this
property walks logical positions too, so these tests add what it cannot:
that no kernel reads a page's contents through anything but the table.
"""
import pytest
import torch

import attn_workloads as W
from _gpu_helpers import library, out_tensor, run_decode, run_prefill, sentinel_intact

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def A():
    return library()


def _pair(**kw):
    a = W.build_case("placement", page_seed=101, device="cuda", **kw)
    b = W.build_case("placement", page_seed=202, device="cuda", **kw)
    assert not torch.equal(a.page_table, b.page_table), "the two placements must differ"
    for la, lb in zip(a.launches, b.launches):
        assert torch.equal(la.q.view(torch.int16), lb.q.view(torch.int16))
    return a, b


def _same_bits(x: torch.Tensor, y: torch.Tensor, rows: int, what: str):
    assert torch.isfinite(x[:rows].float()).all(), f"{what}: non-finite output"
    ix = x.view(torch.int16 if x.dtype == torch.bfloat16 else torch.int32)
    iy = y.view(torch.int16 if y.dtype == torch.bfloat16 else torch.int32)
    assert torch.equal(ix, iy), f"{what}: outputs differ between placements"


# (q_len, q_start, kv_len): an offset chunk, a chunk past a partial page, a
# one-row chunk at a page end, a long prefix with a one-row tail tile
PREFILL_SEQS = [(100, 28, 128), (70, 130, 200), (1, 63, 64), (129, 2000, 2129)]


@pytest.mark.parametrize("kv_dtype,fp8_mma", [("bf16", False), ("fp8_e4m3", False),
                                              ("fp8_e4m3", True)],
                         ids=["bf16", "e4m3", "e4m3-mma"])
@pytest.mark.parametrize("out_dtype", ["bf16", "fp32"])
def test_prefill_page_placement_bitwise(A, kv_dtype, fp8_mma, out_dtype):
    a, b = _pair(seqs=PREFILL_SEQS, hq=32, hkv=4, seed=29, out_dtype=out_dtype,
                 kv_dtype=kv_dtype, q_pad_rows=2)
    rows = a.launches[0].total_q
    oa = run_prefill(A, a, fp8_mma=fp8_mma, pad_rows=3)
    ob = run_prefill(A, b, fp8_mma=fp8_mma, pad_rows=3)
    assert sentinel_intact(oa[rows:]) and sentinel_intact(ob[rows:])
    _same_bits(oa, ob, rows, f"prefill {kv_dtype} mma={fp8_mma} out={out_dtype}")


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8_e4m3"])
def test_decode_page_placement_bitwise(A, kv_dtype):
    # one token per sequence at its last position; lengths across split and
    # page boundaries, one sequence shorter than a page
    seqs = [(1, n - 1, n) for n in (5000, 3001, 1793, 700, 64, 9)]
    a, b = _pair(seqs=seqs, hq=8, hkv=4, seed=31, out_dtype="bf16", kv_dtype=kv_dtype)
    oa = run_decode(A, a)
    ob = run_decode(A, b)
    _same_bits(oa, ob, len(seqs), f"decode {kv_dtype}")


def test_sliding_window_ring_page_placement_bitwise(A):
    seqs = [(100, 1900, 2000), (37, 0, 37)]
    a, b = _pair(seqs=seqs, hq=16, hkv=2, seed=37, out_dtype="bf16", head_dim=256,
                 window=300, ring_pages=7)   # 448 slots hold the window and the rows

    def run(case):
        lc = case.launches[0]
        out = out_tensor(lc.total_q, case.num_q_heads, "bf16", 3, head_dim=case.head_dim)
        A.prefill_swa(lc.q, case.k_pool, case.v_pool, case.page_table, lc.cu_seqlens_q,
                      lc.q_start, lc.kv_len, out, total_q=lc.total_q, max_q_len=lc.max_q_len,
                      softmax_scale=case.softmax_scale, window=case.window,
                      ring_pages=case.ring_pages)
        torch.cuda.synchronize()
        return out

    rows = a.launches[0].total_q
    _same_bits(run(a), run(b), rows, "sliding window, ring cache")
