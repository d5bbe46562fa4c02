"""GPU parity of the split-K prefill (attn_prefill_hd512_splitk) against the
CPU oracle, through the C ABI.

Small ragged batches are compared element by element for several range
lengths (so that ranges end inside a chunk, rows see no key of the last
ranges, and a row's count of ranges differs within one workgroup), both pool
dtypes, sinks and the log-sum-exp.  The prefix-prefill workload (512 rows over
32768 keys) is compared on sampled rows.  The workspace is poisoned with NaN
so that a partial the merge reads but the split kernel never wrote shows up.

The raise of the softmax reference (a score far above the row's first 32)
is exercised here too, on the single-pass and split-K kernels: a planted key
whose score is about 2^200 above the others would overflow fp32 without it,
and keys tens of thousands of log2 units apart need it to rise without
bound.
"""
import numpy as np
import pytest
import torch

import attn_workloads as W
import oracle
from _gpu_helpers import (check_parity, library, out_tensor, run_prefill, sample_rows,
                          sentinel_intact)

pytestmark = pytest.mark.gpu

LSE_ATOL = 2e-3


@pytest.fixture(scope="module")
def A():
    return library()


# "fp8_mma": the E4M3 pool through the FP8-MMA kernels
MODES = ["bf16", "fp8_e4m3", "fp8_mma"]


def _pool(mode):
    return ("fp8_e4m3" if mode.startswith("fp8") else "bf16"), mode == "fp8_mma"


def run_splitk(A, case, kps, out_dtype=None, sinks=None, with_lse=False, pad_rows=3,
               li=0, fp8_mma=False):
    lc = case.launches[li]
    hq = case.num_q_heads
    out = out_tensor(lc.total_q, hq, out_dtype or case.out_dtype, pad_rows)
    lse = torch.full((lc.total_q, hq), float("nan"), device="cuda") if with_lse else None
    nbytes = A.prefill_splitk_workspace_size(lc.batch, lc.max_q_len, lc.total_q, hq,
                                             case.num_kv_heads, lc.max_kv_len, kps)
    ws = torch.full((max(nbytes, 4) // 4,), float("nan"), device="cuda") if nbytes else None
    A.prefill_splitk(lc.q, case.k_pool, case.v_pool, case.page_table, lc.cu_seqlens_q,
                     lc.q_start, lc.kv_len, out, ws, total_q=lc.total_q,
                     max_q_len=lc.max_q_len, max_kv_len=lc.max_kv_len,
                     softmax_scale=case.softmax_scale, keys_per_split=kps,
                     kv_dtype=case.kv_dtype, k_scale=case.k_scale, v_scale=case.v_scale,
                     sinks=None if sinks is None else torch.as_tensor(sinks, device="cuda"),
                     lse=lse, fp8_mma=fp8_mma)
    torch.cuda.synchronize()
    return out, lse, nbytes


def _lse_check(got, ref, what):
    g = got.cpu().numpy()
    assert np.array_equal(np.isinf(g), np.isinf(ref)), f"{what}: lse infinities differ"
    fin = np.isfinite(ref)
    err = float(np.abs(g[fin] - ref[fin]).max()) if fin.any() else 0.0
    print(f"[parity] {what} lse: max_abs={err:.3e}", flush=True)
    assert err <= LSE_ATOL, f"{what}: lse error {err}"


SHAPES = [
    # (seqs (q_len, q_start, kv_len), hq, hkv, keys_per_split)
    ([(37, 300, 337)], 8, 1, 64),                          # ranges end inside the chunk
    ([(100, 1000, 1100), (7, 0, 7), (64, 191, 255)], 32, 4, 128),   # batch 3, ragged
    ([(129, 2000, 2129)], 32, 4, 256),                     # one-row tail block
    ([(19, 5, 24), (70, 1130, 1200), (1, 639, 640)], 12, 4, 192),   # g = 3
    ([(130, 700, 830), (3, 4000, 4003)], 16, 1, 512),      # g = 16
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"{s[0][0]}-{s[1]}x{s[2]}-k{s[3]}")
@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("with_sink", [False, True])
def test_splitk_small(A, shape, mode, with_sink):
    kv_dtype, mma = _pool(mode)
    seqs, hq, hkv, kps = shape
    case = W.build_case("splitk", seqs=seqs, hq=hq, hkv=hkv, seed=41, out_dtype="fp32",
                        device="cuda", kv_dtype=kv_dtype, q_pad_rows=3, extra_pages=2,
                        table_pad=2)
    sinks = (np.random.default_rng(9).uniform(-2.0, 6.0, hq).astype(np.float32)
             if with_sink else None)
    out, lse, nbytes = run_splitk(A, case, kps, sinks=sinks, with_lse=True, fp8_mma=mma)
    assert nbytes > 0, "the fixture is meant to split"
    lc = case.launches[0]
    assert sentinel_intact(out[lc.total_q:]), "rows past total_q were written"
    ref, ref_lse = oracle.attend_all_lse(case.to("cpu"), sinks=sinks)
    what = f"splitk {seqs} {hq}/{hkv} kps={kps} {mode} sink={with_sink}"
    check_parity(out[:lc.total_q], ref, what)
    _lse_check(lse, ref_lse, what)


@pytest.mark.parametrize("out_dtype", ["bf16", "fp32"])
def test_splitk_bf16_out_and_default_plan(A, out_dtype):
    case = W.build_case("splitk_b", seqs=[(200, 3000, 3200), (60, 100, 160)], hq=32, hkv=4,
                        seed=43, out_dtype=out_dtype, device="cuda", q_pad_rows=2)
    lc = case.launches[0]
    ref = oracle.attend_all(case.to("cpu"))
    out, _, nbytes = run_splitk(A, case, 0)
    assert nbytes > 0   # 13 row blocks x 4 KV heads: the default plan splits
    check_parity(out[:lc.total_q], ref, f"splitk default plan out={out_dtype}")
    assert sentinel_intact(out[lc.total_q:])


def test_splitk_single_range_runs_single_pass(A):
    # a range as long as the whole prefix: no workspace, same result bits as
    # the single-pass entry point
    case = W.build_case("splitk_1", seqs=[(100, 1000, 1100)], hq=32, hkv=4, seed=47,
                        out_dtype="bf16", device="cuda")
    out, _, nbytes = run_splitk(A, case, 1152)
    assert nbytes == 0
    single = run_prefill(A, case, pad_rows=3)
    assert torch.equal(out.view(torch.int16), single.view(torch.int16))


def test_splitk_matches_single_pass(A):
    case = W.chunk_prefill_2k(device="cuda")
    lc = case.launches[0]
    single = run_prefill(A, case, out_dtype="fp32")
    split, _, nbytes = run_splitk(A, case, 512, out_dtype="fp32")
    assert nbytes > 0
    d = (split[:lc.total_q] - single[:lc.total_q]).abs()
    print(f"[parity] splitk vs single pass, chunk 2048: max={d.max().item():.3e} "
          f"mean={d.mean().item():.3e}", flush=True)
    # the two differ only in rounding order: hold them to the parity gate
    assert d.max().item() <= 1e-2 and d.mean().item() <= 1e-3


def test_splitk_q0_v1_is_exactly_one(A):
    case = W.build_case("splitk_q0v1", seqs=[(300, 5000, 5300), (40, 0, 40)], hq=16, hkv=1,
                        seed=53, out_dtype="fp32", device="cuda", q_zero=True, v_one=True)
    lc = case.launches[0]
    out, _, nbytes = run_splitk(A, case, 256)
    assert nbytes > 0
    assert bool((out[:lc.total_q] == 1.0).all())


@pytest.mark.parametrize("mode", MODES)
def test_prefix_prefill_512_at_32k_sampled(A, mode):
    kv_dtype, mma = _pool(mode)
    case = W.prefix_prefill_512_at_32k(device="cuda", kv_dtype=kv_dtype)
    lc = case.launches[0]
    out, _, nbytes = run_splitk(A, case, 0, pad_rows=16, fp8_mma=mma)
    assert nbytes > 0
    assert sentinel_intact(out[lc.total_q:])
    g = np.random.default_rng(6)
    tokens = [0, 1, 2, 255, 256, lc.total_q - 2, lc.total_q - 1] + \
        g.integers(0, lc.total_q, 9).tolist()
    rows, toks = sample_rows(lc, case.num_q_heads, tokens)
    ref = oracle.attend_rows(case.to("cpu"), rows).reshape(len(toks), case.num_q_heads, -1)
    check_parity(out[torch.as_tensor(toks, device="cuda")], ref,
                 f"prefix_prefill_512_at_32k {mode} sampled")


def _plant_hot_key(case, b, j, kv_dtype):
    """Sets every q row to a sign vector u and key j of sequence b to +-big u,
    so that key's score is about 2^200 (log2 units) above the others'."""
    lc = case.launches[0]
    u = torch.where(torch.arange(512, device="cuda") % 3 == 0, -1.0, 1.0)
    lc.q[:lc.total_q] = u.to(torch.bfloat16)
    page = int(case.page_table[b, j // 64])
    if kv_dtype == "bf16":
        case.k_pool[page, :, j % 64, :] = (7.0 * u).to(torch.bfloat16)
    else:
        # +-448 codes: 0x7E and 0xFE
        case.k_pool[page, :, j % 64, :] = torch.where(u > 0, 0x7E, 0xFE).to(torch.uint8)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("path", ["single", "splitk"])
def test_reference_raise_on_hot_key(A, mode, path):
    kv_dtype, mma = _pool(mode)
    case = W.build_case("hot", seqs=[(70, 900, 970), (50, 0, 50)], hq=16, hkv=2, seed=59,
                        out_dtype="fp32", device="cuda", kv_dtype=kv_dtype, q_pad_rows=2)
    _plant_hot_key(case, 0, 700, kv_dtype)    # in the 11th key tile, past the first 32 keys
    _plant_hot_key(case, 1, 40, kv_dtype)     # in the first tile, second half
    lc = case.launches[0]
    if path == "single":
        out = run_prefill(A, case, pad_rows=2, fp8_mma=mma)
    else:
        out, _, nbytes = run_splitk(A, case, 128, pad_rows=2, fp8_mma=mma)
        assert nbytes > 0
    ref = oracle.attend_all(case.to("cpu"))
    assert np.isfinite(ref).all()
    check_parity(out[:lc.total_q], ref, f"hot key {mode} {path}")


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("path", ["single", "splitk"])
def test_reference_rises_past_any_range(A, mode, path):
    # Three keys per sequence, each tens of thousands of log2 units above
    # everything before it: the softmax reference must rise by far more than
    # any fixed number of bounded raises would allow.  Every q row is q_mag u
    # (u a +-1 vector); bf16 pools get keys beta u with beta = 16, 64, 256,
    # E4M3 pools the codes of 28 u, 112 u and 448 u (exact E4M3 values).  The
    # rows are then each dominated by one key, whose value is the output.
    kv_dtype, mma = _pool(mode)
    case = W.build_case("far", seqs=[(70, 900, 970), (50, 0, 50)], hq=16, hkv=2, seed=61,
                        out_dtype="fp32", device="cuda", kv_dtype=kv_dtype, q_pad_rows=2)
    lc = case.launches[0]
    u = torch.where(torch.arange(512, device="cuda") % 3 == 0, -1.0, 1.0)
    q_mag = 8.0 if kv_dtype == "bf16" else 1024.0
    lc.q[:lc.total_q] = (q_mag * u).to(torch.bfloat16)
    levels = (16.0, 64.0, 256.0) if kv_dtype == "bf16" else (28.0, 112.0, 448.0)
    for b, keys in ((0, (300, 600, 950)), (1, (5, 20, 40))):
        for j, lev in zip(keys, levels):
            page = int(case.page_table[b, j // 64])
            if kv_dtype == "bf16":
                case.k_pool[page, :, j % 64, :] = (lev * u).to(torch.bfloat16)
            else:
                case.k_pool[page, :, j % 64, :] = (lev * u).to(torch.float8_e4m3fn).view(torch.uint8)
    if path == "single":
        out = run_prefill(A, case, pad_rows=2, fp8_mma=mma)
    else:
        out, _, nbytes = run_splitk(A, case, 128, pad_rows=2, fp8_mma=mma)
        assert nbytes > 0
    ref = oracle.attend_all(case.to("cpu"))
    assert np.isfinite(ref).all()
    check_parity(out[:lc.total_q], ref, f"far keys {mode} {path}")


@pytest.mark.parametrize("mode", ["bf16", "fp8_mma"])
@pytest.mark.parametrize("path", ["single", "splitk"])
def test_context_past_the_staged_page_ids(A, path, mode):
    # 300000 keys = 4688 key tiles: past the 4096 page ids a workgroup stages
    # in LDS, so the tail tiles take the page-table path in the loop
    kv_dtype, mma = _pool(mode)
    case = W.build_case("long300k", seqs=[(64, 299936, 300000)], hq=8, hkv=1, seed=73,
                        out_dtype="fp32", device="cuda", q_pad_rows=2, kv_dtype=kv_dtype)
    lc = case.launches[0]
    if path == "single":
        out = run_prefill(A, case, pad_rows=2, fp8_mma=mma)
    else:
        out, _, nbytes = run_splitk(A, case, 0, pad_rows=2, fp8_mma=mma)
        assert nbytes > 0
    assert sentinel_intact(out[lc.total_q:])
    tokens = [0, 1, 31, 62, 63]
    rows, toks = sample_rows(lc, case.num_q_heads, tokens)
    ref = oracle.attend_rows(case.to("cpu"), rows).reshape(len(toks), case.num_q_heads, -1)
    check_parity(out[torch.as_tensor(toks, device="cuda")], ref, f"300000 keys {path} {mode}")
