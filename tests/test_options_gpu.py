"""GPU parity of the extended entry points against the CPU oracle: multi-token
decode (q_len query tokens per sequence at its last positions, up to three
blocks of 16 (token, head) columns per KV head in the decode kernels; wider
calls run as split-K prefill),
attention sinks and the log-sum-exp output, for prefill and decode, bf16 and
FP8 pools.

Outputs use the usual gate; the log-sum-exp is compared with the oracle's
(natural log) to an absolute 2e-3.  Decode fixtures put kv_len next to split
boundaries, so that the earlier tokens of a multi-token row see no key at all
in the last split and that split's partial must be empty.
"""
import numpy as np
import pytest
import torch

import attn_workloads as W
import oracle
from _gpu_helpers import check_parity, library, out_tensor

pytestmark = pytest.mark.gpu

LSE_ATOL = 2e-3


@pytest.fixture(scope="module")
def A():
    return library()


def _sinks(hq, seed=3):
    return np.random.default_rng(seed).uniform(-2.0, 6.0, hq).astype(np.float32)


def _lse_check(got, ref, what):
    g = got.cpu().numpy()
    assert np.array_equal(np.isinf(g), np.isinf(ref)), f"{what}: lse infinities differ"
    fin = np.isfinite(ref)
    err = float(np.abs(g[fin] - ref[fin]).max()) if fin.any() else 0.0
    print(f"[parity] {what} lse: max_abs={err:.3e}", flush=True)
    assert err <= LSE_ATOL, f"{what}: lse error {err}"


def _run_decode(A, case, q_len, sinks, kps, out_dtype="fp32"):
    lc = case.launches[0]
    B = lc.batch
    out = out_tensor(B * q_len, case.num_q_heads, out_dtype)
    lse = torch.full((B * q_len, case.num_q_heads), float("nan"), device="cuda")
    nbytes = A.decode_workspace_size(B, case.num_q_heads, case.num_kv_heads, lc.max_kv_len,
                                     kps, q_len=q_len)
    ws = torch.full((nbytes // 4,), float("nan"), device="cuda")
    A.decode(lc.q[:B * q_len], case.k_pool, case.v_pool, case.page_table, lc.kv_len, out, ws,
             max_kv_len=lc.max_kv_len, softmax_scale=case.softmax_scale,
             kv_dtype=case.kv_dtype, k_scale=case.k_scale, v_scale=case.v_scale,
             keys_per_split=kps, q_len=q_len,
             sinks=None if sinks is None else torch.as_tensor(sinks, device="cuda"), lse=lse)
    torch.cuda.synchronize()
    return out, lse


DECODE = [
    # (kv_lens, q_len, hq, hkv, keys_per_split)
    ([257, 258, 300, 511, 513], 2, 8, 4, 256),
    ([256, 259, 1000, 64], 3, 8, 4, 256),
    ([260, 900, 5], 5, 6, 3, 256),          # g = 2, q_len 5: 10 columns
    ([4096, 4097, 2049], 4, 16, 4, 0),      # g = 4, 16 columns, library default split
    ([777, 1024], 1, 16, 1, 256),            # g = 16, q_len 1
    # two and three 16-column blocks per split workgroup
    ([257, 1000, 64, 2049], 3, 32, 4, 256),  # g = 8, q_len 3: 24 columns
    ([5, 300, 4100], 5, 32, 4, 0),           # g = 8, q_len 5, kv_len = q_len, default split
    ([700, 129], 2, 16, 1, 256),             # g = 16, q_len 2: 32 columns
    ([100, 33], 17, 4, 4, 256),              # g = 1, q_len 17
    ([300, 48, 1100], 12, 16, 4, 512),       # g = 4, q_len 12: 48 columns
    # more than 48 columns: routed through the split-K prefill
    ([257, 1000, 7, 2049], 7, 32, 4, 256),   # g = 8, q_len 7: 56 columns
    ([700, 129], 4, 16, 1, 0),               # g = 16, q_len 4: 64 columns
    ([100, 64], 50, 4, 4, 256),              # g = 1, q_len 50
]


@pytest.mark.parametrize("fx", DECODE, ids=lambda f: f"L{f[0][0]}-q{f[1]}-{f[2]}x{f[3]}")
@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8_e4m3"])
@pytest.mark.parametrize("with_sink", [False, True])
def test_multi_token_decode(A, fx, kv_dtype, with_sink):
    lens, q_len, hq, hkv, kps = fx
    case = W.build_case("mtp", seqs=[(q_len, L - q_len, L) for L in lens], hq=hq, hkv=hkv,
                        seed=29, out_dtype="fp32", device="cuda", kv_dtype=kv_dtype,
                        extra_pages=2, table_pad=2)
    sinks = _sinks(hq) if with_sink else None
    out, lse = _run_decode(A, case, q_len, sinks, kps)
    ref, ref_lse = oracle.attend_all_lse(case.to("cpu"), sinks=sinks)
    what = f"decode q_len={q_len} {hq}/{hkv} {kv_dtype} sink={with_sink}"
    check_parity(out, ref, what)
    _lse_check(lse, ref_lse, what)


@pytest.mark.parametrize("kps", [256, 1024], ids=["split256", "split1024"])
@pytest.mark.parametrize("q_len", [1, 3, 5])
@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8_e4m3"])
def test_decode_late_dominant_keys(A, kv_dtype, q_len, kps):
    # a key 12 log2 units above what its split saw before it (two
    # sequences) and a climb to 99 (the third), inside later tiles of their
    # splits: the split kernels move their references and rescale O and l
    # after the first tile; one to three column blocks at g = 8
    case = W.decode_late_keys(device="cuda", kv_dtype=kv_dtype, q_len=q_len)
    out, lse = _run_decode(A, case, q_len, None, kps)
    ref, ref_lse = oracle.attend_all_lse(case.to("cpu"))
    what = f"decode late keys q_len={q_len} {kv_dtype} split={kps}"
    check_parity(out, ref, what)
    _lse_check(lse, ref_lse, what)


def test_multi_token_decode_bf16_out(A):
    lens = [300, 1000, 2049]
    case = W.build_case("mtp_bf16", seqs=[(4, L - 4, L) for L in lens], hq=8, hkv=4, seed=31,
                        out_dtype="bf16", device="cuda", extra_pages=1)
    out, lse = _run_decode(A, case, 4, _sinks(8, 5), 256, out_dtype="bf16")
    ref, ref_lse = oracle.attend_all_lse(case.to("cpu"), sinks=_sinks(8, 5))
    check_parity(out, ref, "decode q_len=4 bf16 out")
    _lse_check(lse, ref_lse, "decode q_len=4 bf16 out")


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8_e4m3"])
def test_multi_token_decode_b64_q5_g8(A, kv_dtype):
    # the current token plus a 4-token draft at 32/4 heads, batch 64, lengths
    # U{4096..28672}: 40 columns per KV head (three column blocks of the
    # decode kernels).  Every sequence is checked: its 5 tokens on the 8 heads of one
    # KV group (rotating over the groups) and head 0 of the others.
    case = W.decode_mtp_b64(device="cuda", kv_dtype=kv_dtype)
    lc = case.launches[0]
    q_len, hq, g = 5, case.num_q_heads, case.num_q_heads // case.num_kv_heads
    sinks = _sinks(hq, 11)
    out_bf, lse = _run_decode(A, case, q_len, sinks, 0, out_dtype="bf16")
    rows = []
    for b in range(lc.batch):
        kvh = b % case.num_kv_heads
        heads = sorted(set(range(kvh * g, kvh * g + g)) |
                       {h * g for h in range(case.num_kv_heads)})
        rows += [(b * q_len + t) * hq + h for t in range(q_len) for h in heads]
    rows = np.asarray(rows)
    ref, ref_lse = oracle.attend_rows_lse(case.to("cpu"), rows, sinks=sinks)
    what = f"decode_mtp_b64_q5_g8 {kv_dtype} ({len(rows)} rows)"
    got = out_bf.reshape(-1, out_bf.shape[-1])[torch.as_tensor(rows, device="cuda")]
    check_parity(got, ref, what)
    _lse_check(lse.reshape(-1)[torch.as_tensor(rows, device="cuda")], ref_lse, what)
    assert bool(torch.isfinite(out_bf.float()).all()), "unwritten output rows"
    # the same bits on a second call
    again, _ = _run_decode(A, case, q_len, sinks, 0, out_dtype="bf16")
    assert torch.equal(out_bf.view(torch.int16), again.view(torch.int16))


PREFILL = [
    ([(37, 0, 37)], 8, 1),
    ([(100, 28, 128), (64, 64, 200)], 16, 8),
    ([(129, 2000, 2129), (7, 300, 307)], 32, 4),
]


@pytest.mark.parametrize("shape", PREFILL, ids=lambda s: f"{s[0][0]}-{s[1]}x{s[2]}")
@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8_e4m3"])
@pytest.mark.parametrize("with_sink", [False, True])
def test_prefill_sinks_and_lse(A, shape, kv_dtype, with_sink):
    seqs, hq, hkv = shape
    case = W.build_case("pf_opt", seqs=seqs, hq=hq, hkv=hkv, seed=37, out_dtype="fp32",
                        device="cuda", kv_dtype=kv_dtype, extra_pages=2, table_pad=2)
    lc = case.launches[0]
    sinks = _sinks(hq, 7) if with_sink else None
    out = out_tensor(lc.total_q, hq, "fp32")
    lse = torch.full((lc.total_q, hq), float("nan"), device="cuda")
    A.prefill(lc.q, case.k_pool, case.v_pool, case.page_table, lc.cu_seqlens_q, lc.q_start,
              lc.kv_len, out, total_q=lc.total_q, max_q_len=lc.max_q_len,
              softmax_scale=case.softmax_scale, kv_dtype=kv_dtype, k_scale=case.k_scale,
              v_scale=case.v_scale,
              sinks=None if sinks is None else torch.as_tensor(sinks, device="cuda"), lse=lse)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.attend_all_lse(case.to("cpu"), sinks=sinks)
    what = f"prefill {seqs} {kv_dtype} sink={with_sink}"
    check_parity(out, ref, what)
    _lse_check(lse, ref_lse, what)


def test_prefill_lse_on_the_2048_chunk(A):
    case = W.chunk_prefill_2k(device="cuda")
    lc = case.launches[0]
    out = out_tensor(lc.total_q, case.num_q_heads, "bf16")
    lse = torch.empty((lc.total_q, case.num_q_heads), device="cuda")
    A.prefill(lc.q, case.k_pool, case.v_pool, case.page_table, lc.cu_seqlens_q, lc.q_start,
              lc.kv_len, out, total_q=lc.total_q, max_q_len=lc.max_q_len,
              softmax_scale=case.softmax_scale, lse=lse)
    torch.cuda.synchronize()
    g = np.random.default_rng(9)
    toks = np.unique(np.concatenate([[0, 1, lc.total_q - 1], g.integers(0, lc.total_q, 40)]))
    rows = (toks[:, None] * case.num_q_heads + np.arange(case.num_q_heads)[None, :]).reshape(-1)
    ref, ref_lse = oracle.attend_rows_lse(case.to("cpu"), rows)
    check_parity(out[torch.as_tensor(toks, device="cuda")],
                 ref.reshape(len(toks), case.num_q_heads, -1), "prefill 2048 (lse call)")
    _lse_check(lse[torch.as_tensor(toks, device="cuda")],
               ref_lse.reshape(len(toks), case.num_q_heads), "prefill 2048")
