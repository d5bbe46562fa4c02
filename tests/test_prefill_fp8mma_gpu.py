"""GPU parity of attn_prefill_hd512_e4m3_mma (FP8-E4M3 KV cache, both
products on the block-scaled FP8 matrix core) against the CPU oracle.

The oracle reads the same E4M3 bytes (vLLM flash-attention PR 199,
"Summary"); the kernel's extra rounding is Q and P as two scaled E4M3 terms
each (second review, commit 4 and finding F1), which the parity gate of the
bf16 path must absorb.  Beyond the shapes of the widened FP8 tests, the cases
the pages found the FP8-MMA form failing are run here: one late key ahead by
Delta = 12 and 13 over a long row (finding F1: the residual of small weights
was lost), |q| far above 448 (finding F2: a fixed Q scale overflows), and
q = 0 with V = 1 over 32K keys (commit 3: sub-fp32 accumulation gave 0.5).
"""
import numpy as np
import pytest
import torch

import attn_workloads as W
import oracle
from _gpu_helpers import (check_parity, check_parity_any, library, one_token_per_block,
                          oracle_rows_cached, out_tensor, sample_rows, sentinel_intact,
                          tokens_per_workgroup)

pytestmark = pytest.mark.gpu

FP8 = "fp8_e4m3"
GATE_MAX, GATE_MEAN = 1e-2, 1e-3


@pytest.fixture(scope="module")
def A():
    return library()


def run_mma(A, case, li=0, out_dtype=None, pad_rows=0, sinks=None, lse=None):
    lc = case.launches[li]
    out = out_tensor(lc.total_q, case.num_q_heads, out_dtype or case.out_dtype, pad_rows)
    A.prefill(lc.q, case.k_pool, case.v_pool, case.page_table, lc.cu_seqlens_q, lc.q_start,
              lc.kv_len, out, total_q=lc.total_q, max_q_len=lc.max_q_len,
              softmax_scale=case.softmax_scale, kv_dtype=FP8, k_scale=case.k_scale,
              v_scale=case.v_scale, sinks=sinks, lse=lse, fp8_mma=True)
    torch.cuda.synchronize()
    return out


SMALL = [
    ([(1, 0, 1)], 8, 1),
    ([(37, 0, 37)], 8, 1),
    ([(100, 28, 128)], 4, 4),
    ([(64, 64, 200)], 16, 8),
    ([(19, 5, 24), (70, 130, 200), (1, 63, 64)], 12, 4),
    ([(130, 0, 130), (7, 300, 307)], 16, 1),
    ([(129, 2000, 2129)], 32, 4),
    ([(3, 4001, 4004), (200, 57, 257)], 8, 2),
]


@pytest.mark.parametrize("shape", SMALL, ids=lambda s: f"{s[0]}-{s[1]}x{s[2]}")
@pytest.mark.parametrize("out_dtype", ["fp32", "bf16"])
def test_small_shapes_fp8_mma(A, shape, out_dtype):
    seqs, hq, hkv = shape
    case = W.build_case("small_fp8_mma", seqs=seqs, hq=hq, hkv=hkv, seed=29,
                        out_dtype=out_dtype, device="cuda", q_pad_rows=3, extra_pages=2,
                        table_pad=2, kv_dtype=FP8)
    lc = case.launches[0]
    print(f"[case] {seqs} {hq}/{hkv} {out_dtype}", flush=True)
    ref = oracle.attend_all(case.to("cpu"))

    def run(dt):
        out = run_mma(A, case, out_dtype=dt, pad_rows=5)
        assert sentinel_intact(out[lc.total_q:]), "rows past total_q were written"
        return out[:lc.total_q]
    # the one-key shape is a bf16 rounding-floor case (see the widened FP8 test)
    check_parity_any(run, ref, f"fp8 mma {seqs} out={out_dtype}", out_dtype)


def test_chunk_prefill_2048_fp8_mma(A):
    case = W.chunk_prefill_2k(device="cuda", kv_dtype=FP8)
    out = run_mma(A, case)
    check_parity(out, oracle.attend_all(case.to("cpu")), "chunk_2048 fp8 mma")


def test_chunk_prefill_8192_at_8192_fp8_mma_every_workgroup(A):
    # the widened FP8 test's tokens and oracle rows: one token from every
    # 16-token workgroup block, all 32 heads, first and last token
    case = W.chunk_prefill_8k_at_8k(device="cuda", kv_dtype=FP8)
    lc = case.launches[0]
    out = run_mma(A, case, pad_rows=64)
    assert sentinel_intact(out[lc.total_q:])
    tokens = one_token_per_block(lc.total_q, tokens_per_workgroup(32, 4), seed=5)
    rows, toks = sample_rows(lc, case.num_q_heads, tokens)
    ref = oracle_rows_cached(case.name, case.to("cpu"), rows).reshape(len(toks),
                                                                      case.num_q_heads, -1)
    check_parity(out[torch.as_tensor(toks, device="cuda")], ref,
                 f"chunk_8192_at_8192 fp8 mma every workgroup ({len(toks)} tokens)")


@pytest.mark.parametrize("li", range(8))
def test_long_mqa_32k_chunk_fp8_mma_every_workgroup(A, li):
    case = W.long_mqa_32k(device="cuda", kv_dtype=FP8)
    lc = case.launches[li]
    out = run_mma(A, case, li=li, pad_rows=3)
    assert sentinel_intact(out[lc.total_q:])
    tokens = one_token_per_block(lc.total_q, tokens_per_workgroup(16, 1), seed=6 + li)
    rows, toks = sample_rows(lc, case.num_q_heads, tokens)
    ref = oracle_rows_cached(case.name, case.to("cpu"), rows, launch_idx=li).reshape(
        len(toks), case.num_q_heads, -1)
    check_parity(out[torch.as_tensor(toks, device="cuda")], ref,
                 f"long_mqa_32k fp8 mma chunk {li} every workgroup ({len(toks)} tokens)")


def test_fp8_mma_q0_v1_is_the_dequantised_one(A):
    # q = 0: every weight is 1 (one E4M3 term, no residual); V dequantises to
    # one value v everywhere, so fp32 accumulation gives v exactly up to the
    # final scale multiply, at the prompt's last 4096-row chunk (28K-32K keys)
    case = W.long_mqa_32k(device="cuda", q_zero=True, v_one=True, kv_dtype=FP8)
    li = len(case.launches) - 1
    out = run_mma(A, case, li=li).float().cpu().numpy()
    page0 = int(case.page_table[0, 0].item())
    code = case.v_pool.view(torch.uint8)[page0, 0, 0, 0].item()
    v = float(oracle.e4m3_to_f32(np.array([code], dtype=np.uint8))[0] * np.float32(case.v_scale))
    assert np.isfinite(out).all()
    np.testing.assert_allclose(out, v, rtol=2e-7, atol=0)


@pytest.mark.parametrize("delta", [12.0, 13.0])
def test_fp8_mma_keeps_the_softmax_tail(A, delta):
    # one row over 32768 keys with logits 0 except the last key at Delta
    # (q = a e_0, keys zero in dim 0 but the last): the other keys' weights
    # are 2^-17 .. 2^-19 of the late one's and carry 1 - e^D / (n - 1 + e^D)
    # = 7 % (D = 12) and 3 % (D = 13) of the output
    n = 32768
    case = W.build_case("spike_fp8", seqs=[(1, n - 1, n)], hq=1, hkv=1, seed=31,
                        out_dtype="fp32", device="cuda", kv_dtype=FP8)
    lc = case.launches[0]
    a = 256.0                # keeps the late key's byte value (~100) inside E4M3's 448
    lc.q.zero_()
    lc.q[0, 0, 0] = a
    kp = case.k_pool.view(torch.uint8)
    kp[:, :, :, 0] = 0
    coef = delta / (case.softmax_scale * a * case.k_scale)      # key byte value in dim 0
    assert coef < 448.0
    code = int(torch.tensor(coef).to(torch.float8_e4m3fn).view(torch.uint8))
    late = n - 1
    kp[int(case.page_table[0, late // 64]), 0, late % 64, 0] = code
    out = run_mma(A, case)
    cpu = case.to("cpu")
    ref = oracle.attend_all(cpu)
    check_parity(out, ref, f"late key Delta={delta}")
    # against the closed form of the same bytes
    d = float(oracle.e4m3_to_f32(np.array([code], dtype=np.uint8))[0]) * case.k_scale * a * \
        case.softmax_scale
    j = torch.arange(n)
    vb = cpu.v_pool.view(torch.uint8)[cpu.page_table[0, j // 64].long(), 0, j % 64]
    V = oracle.e4m3_to_f32(vb.numpy()).astype(np.float64) * case.v_scale
    w = np.exp(d)
    expect = (V[:-1].sum(axis=0) + w * V[-1]) / (n - 1 + w)
    got = out[0, 0].double().cpu().numpy()
    assert np.abs(got - expect).max() <= GATE_MAX


def test_fp8_mma_q_far_above_448(A):
    # finding F2: a fixed-scale E4M3 split of Q overflows past |q| = 448; the
    # per-32-dim scales here take any finite bf16 Q.  Q x 256 (exact in bf16)
    # with softmax_scale / 256 keeps the logits of the unscaled case.  (The
    # split keeps about 8 significant bits of Q, so at logits hundreds of
    # nats apart its rounding moves scores by tenths of a nat; the range
    # itself, any finite score spread, is the far-keys test's subject.)
    case = W.build_case("bigq_fp8", seqs=[(150, 300, 450), (40, 0, 40)], hq=16, hkv=2, seed=37,
                        out_dtype="fp32", device="cuda", kv_dtype=FP8)
    lc = case.launches[0]
    lc.q.mul_(256.0)
    case.softmax_scale /= 256.0
    assert float(lc.q[:lc.total_q].float().abs().max()) > 448
    out = run_mma(A, case)
    check_parity(out[:lc.total_q], oracle.attend_all(case.to("cpu")), "|q| > 448")


def test_fp8_mma_sinks_and_lse(A):
    case = W.build_case("sink_fp8_mma", seqs=[(90, 410, 500), (33, 0, 33), (129, 64, 193)],
                        hq=16, hkv=2, seed=41, out_dtype="fp32", device="cuda", kv_dtype=FP8)
    lc = case.launches[0]
    sinks = np.random.default_rng(4).uniform(-2.0, 6.0, 16).astype(np.float32)
    lse = torch.full((lc.total_q, 16), float("nan"), device="cuda")
    out = run_mma(A, case, sinks=torch.as_tensor(sinks, device="cuda"), lse=lse)
    ref, ref_lse = oracle.attend_all_lse(case.to("cpu"), sinks=sinks)
    check_parity(out[:lc.total_q], ref, "fp8 mma sinks")
    err = float(np.abs(lse.cpu().numpy() - ref_lse).max())
    assert err <= 2e-3, f"lse error {err}"


def test_fp8_mma_deterministic(A):
    case = W.build_case("det_fp8_mma", seqs=[(300, 100, 400)], hq=32, hkv=4, seed=23,
                        out_dtype="fp32", device="cuda", kv_dtype=FP8)
    a = run_mma(A, case)
    b = run_mma(A, case)
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))


def test_fp8_mma_close_to_the_widened_path(A):
    # the two FP8 paths read the same bytes; their difference is the E4M3
    # split of Q and P against bf16 P
    case = W.build_case("cmp_fp8", seqs=[(256, 512, 768)], hq=32, hkv=4, seed=43,
                        out_dtype="fp32", device="cuda", kv_dtype=FP8)
    lc = case.launches[0]
    got = run_mma(A, case)
    out = out_tensor(lc.total_q, 32, "fp32", 0)
    A.prefill(lc.q, case.k_pool, case.v_pool, case.page_table, lc.cu_seqlens_q, lc.q_start,
              lc.kv_len, out, total_q=lc.total_q, max_q_len=lc.max_q_len,
              softmax_scale=case.softmax_scale, kv_dtype=FP8, k_scale=case.k_scale,
              v_scale=case.v_scale)
    torch.cuda.synchronize()
    diff = (got - out).abs()
    assert float(diff.max()) <= GATE_MAX and float(diff.mean()) <= GATE_MEAN


def test_fp8_mma_rejects_a_bf16_pool(A):
    case = W.build_case("bf16_pool", seqs=[(8, 0, 8)], hq=8, hkv=1, seed=1, out_dtype="fp32",
                        device="cuda")
    lc = case.launches[0]
    out = torch.zeros((lc.total_q, 8, 512), device="cuda")
    with pytest.raises(A.AttnError):
        A.prefill(lc.q, case.k_pool, case.v_pool, case.page_table, lc.cu_seqlens_q, lc.q_start,
                  lc.kv_len, out, total_q=lc.total_q, max_q_len=lc.max_q_len,
                  softmax_scale=case.softmax_scale, fp8_mma=True)
