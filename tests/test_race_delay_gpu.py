"""Race stand-in: the small parity shapes on the delay-injected build.

libattn_hd512_delay.so is the same sources built with ATTN_RACE_DELAY: every
wave sleeps for a time set by its index, its workgroup and the call site
after each LDS refill load and before each workgroup barrier, so the waves
reach every hand-off (tile refills, score and probability exchanges, the
output staging, the persistent queue) in other orders and at other distances
than in the normal build.  A missing wait or barrier then changes the
results.  The kernels are deterministic, so each case must give the normal
build's bits exactly, and it is also held to the parity gate against the
oracle.  Every kernel family that stages data through LDS is covered: the
bf16, widened-FP8 and FP8-MMA prefills (plain, with sinks and log-sum-exp,
split-K, persistent, append fused, sliding window) and the split-K decode
(one, two and three column blocks, both pools, and the call routed to the
split-K prefill).
"""
import numpy as np
import pytest
import torch

import attn_workloads as W
import oracle
from _gpu_helpers import check_parity, library, out_tensor

pytestmark = pytest.mark.gpu

PREFILL_SEQS = [(37, 0, 37), (100, 28, 128), (129, 2000, 2129)]


@pytest.fixture(scope="module")
def A():
    return library()


def _both(A, run):
    """run() on the normal build, then on the delay-injected one."""
    from attention_hd512_gqa_amd import _lib
    first = run()
    torch.cuda.synchronize()
    with _lib.delay_injected():
        second = run()
        torch.cuda.synchronize()
    return first, second


def _same_bits(a, b, what):
    view = torch.int32 if a.dtype == torch.float32 else torch.int16
    assert torch.equal(a.view(view), b.view(view)), \
        f"{what}: the delay-injected build gives other bits"


def _case(name, seqs, hq, hkv, kv="bf16", seed=41, **kw):
    kw.setdefault("extra_pages", 2)
    kw.setdefault("table_pad", 2)
    return W.build_case(name, seqs=seqs, hq=hq, hkv=hkv, seed=seed, out_dtype="fp32",
                        device="cuda", kv_dtype=kv, **kw)


@pytest.mark.parametrize("kv,mma", [("bf16", False), ("fp8_e4m3", False), ("fp8_e4m3", True)],
                         ids=["bf16", "fp8", "fp8mma"])
@pytest.mark.parametrize("hq,hkv", [(32, 4), (16, 1), (4, 4)])
def test_prefill_delayed(A, kv, mma, hq, hkv):
    what = f"prefill {kv} mma={mma} {hq}/{hkv}"
    print(f"[case] delay {what}", flush=True)
    case = _case("race_pf", PREFILL_SEQS, hq, hkv, kv)
    lc = case.launches[0]
    sinks = np.random.default_rng(5).uniform(-2.0, 6.0, hq).astype(np.float32)

    def run():
        out = out_tensor(lc.total_q, hq, "fp32")
        lse = torch.full((lc.total_q, hq), float("nan"), device="cuda")
        A.prefill(lc.q, case.k_pool, case.v_pool, case.page_table, lc.cu_seqlens_q,
                  lc.q_start, lc.kv_len, out, total_q=lc.total_q, max_q_len=lc.max_q_len,
                  softmax_scale=case.softmax_scale, kv_dtype=kv, k_scale=case.k_scale,
                  v_scale=case.v_scale, fp8_mma=mma, lse=lse,
                  sinks=torch.as_tensor(sinks, device="cuda"))
        return torch.cat([out.reshape(lc.total_q, -1), lse], dim=1)

    a, b = _both(A, run)
    _same_bits(a, b, what)
    ref, _ = oracle.attend_all_lse(case.to("cpu"), sinks=sinks)
    check_parity(b[:, :-hq].reshape(lc.total_q, hq, -1), ref, what + " (delayed)")


@pytest.mark.parametrize("kv,mma", [("bf16", False), ("fp8_e4m3", True)], ids=["bf16", "fp8mma"])
def test_splitk_prefill_delayed(A, kv, mma):
    what = f"split-K prefill {kv}"
    print(f"[case] delay {what}", flush=True)
    case = _case("race_sk", [(5, 3000, 3005), (64, 100, 164), (17, 700, 717)], 32, 4, kv)
    lc = case.launches[0]
    nb = A.prefill_splitk_workspace_size(lc.batch, lc.max_q_len, lc.total_q, 32, 4,
                                         lc.max_kv_len, 256)
    ws = torch.empty(nb // 4, device="cuda")

    def run():
        out = out_tensor(lc.total_q, 32, "fp32")
        A.prefill_splitk(lc.q, case.k_pool, case.v_pool, case.page_table, lc.cu_seqlens_q,
                         lc.q_start, lc.kv_len, out, ws, total_q=lc.total_q,
                         max_q_len=lc.max_q_len, max_kv_len=lc.max_kv_len,
                         softmax_scale=case.softmax_scale, keys_per_split=256, kv_dtype=kv,
                         k_scale=case.k_scale, v_scale=case.v_scale, fp8_mma=mma)
        return out

    a, b = _both(A, run)
    _same_bits(a, b, what)
    check_parity(b, oracle.attend_all(case.to("cpu")), what + " (delayed)")


def test_persistent_prefill_delayed(A):
    what = "persistent prefill bf16"
    print(f"[case] delay {what}", flush=True)
    case = _case("race_pers", PREFILL_SEQS + [(300, 0, 300)], 32, 4)
    lc = case.launches[0]
    ws = torch.empty(max(A.prefill_persistent_workspace_size() // 4, 1), dtype=torch.int32,
                     device="cuda")

    def run():
        out = out_tensor(lc.total_q, 32, "fp32")
        A.prefill_persistent(lc.q, case.k_pool, case.v_pool, case.page_table, lc.cu_seqlens_q,
                             lc.q_start, lc.kv_len, out, ws, total_q=lc.total_q,
                             max_q_len=lc.max_q_len, softmax_scale=case.softmax_scale)
        return out

    a, b = _both(A, run)
    _same_bits(a, b, what)
    check_parity(b, oracle.attend_all(case.to("cpu")), what + " (delayed)")


def test_fused_append_prefill_delayed(A):
    what = "prefill with the append fused"
    print(f"[case] delay {what}", flush=True)
    case = _case("race_app", PREFILL_SEQS, 32, 4)
    lc = case.launches[0]
    pages, slots = [], []
    for b, (ql, st) in enumerate(zip(lc.q_lens, lc.q_starts)):
        pos = torch.arange(st, st + ql, device="cuda")
        pages.append(case.page_table[b, pos // 64].long())
        slots.append(pos % 64)
    pages, slots = torch.cat(pages), torch.cat(slots)
    kn = case.k_pool[pages, :, slots, :].contiguous()
    vn = case.v_pool[pages, :, slots, :].contiguous()

    def run():
        kp, vp = case.k_pool.clone(), case.v_pool.clone()
        kp[pages, :, slots, :] = float("nan")
        vp[pages, :, slots, :] = float("nan")
        out = out_tensor(lc.total_q, 32, "fp32")
        A.prefill_append(lc.q, kn, vn, kp, vp, case.page_table, lc.cu_seqlens_q, lc.q_start,
                         lc.kv_len, out, total_q=lc.total_q, max_q_len=lc.max_q_len,
                         softmax_scale=case.softmax_scale)
        return out

    a, b = _both(A, run)
    _same_bits(a, b, what)
    check_parity(b, oracle.attend_all(case.to("cpu")), what + " (delayed)")


def test_sliding_window_prefill_delayed(A):
    what = "sliding-window prefill, head dim 256, ring cache"
    print(f"[case] delay {what}", flush=True)
    case = _case("race_swa", [(100, 500, 600), (64, 0, 64)], 16, 2, head_dim=256, window=200,
                 ring_pages=6)
    lc = case.launches[0]

    def run():
        out = out_tensor(lc.total_q, 16, "fp32", head_dim=256)
        A.prefill_swa(lc.q, case.k_pool, case.v_pool, case.page_table, lc.cu_seqlens_q,
                      lc.q_start, lc.kv_len, out, total_q=lc.total_q, max_q_len=lc.max_q_len,
                      softmax_scale=case.softmax_scale, window=case.window,
                      ring_pages=case.ring_pages)
        return out

    a, b = _both(A, run)
    _same_bits(a, b, what)
    check_parity(b, oracle.attend_all(case.to("cpu")), what + " (delayed)")


DECODE = [
    # (kv_lens, q_len, hq, hkv, keys_per_split)
    ([1, 63, 64, 65, 300, 2049], 1, 8, 4, 256),   # one column block
    ([257, 1000, 64, 2049], 3, 32, 4, 256),       # two blocks
    ([5, 300, 4100], 5, 32, 4, 0),                # three blocks, default split
    ([257, 1000, 7, 2049], 7, 32, 4, 256),        # 56 columns: split-K prefill
]


@pytest.mark.parametrize("fx", DECODE, ids=lambda f: f"q{f[1]}-{f[2]}x{f[3]}")
@pytest.mark.parametrize("kv", ["bf16", "fp8_e4m3"])
def test_decode_delayed(A, fx, kv):
    lens, q_len, hq, hkv, kps = fx
    what = f"decode q_len={q_len} {hq}/{hkv} {kv}"
    print(f"[case] delay {what}", flush=True)
    case = _case("race_dec", [(q_len, L - q_len, L) for L in lens], hq, hkv, kv)
    lc = case.launches[0]
    rows = lc.batch * q_len
    nb = A.decode_workspace_size(lc.batch, hq, hkv, lc.max_kv_len, kps, q_len=q_len)
    ws = torch.empty(nb // 4, device="cuda")

    def run():
        out = out_tensor(rows, hq, "fp32")
        A.decode(lc.q[:rows], case.k_pool, case.v_pool, case.page_table, lc.kv_len, out, ws,
                 max_kv_len=lc.max_kv_len, softmax_scale=case.softmax_scale, kv_dtype=kv,
                 k_scale=case.k_scale, v_scale=case.v_scale, keys_per_split=kps, q_len=q_len)
        return out

    a, b = _both(A, run)
    _same_bits(a, b, what)
    check_parity(b, oracle.attend_all(case.to("cpu")), what + " (delayed)")


@pytest.mark.parametrize("q_len", [1, 5])
@pytest.mark.parametrize("kv", ["bf16", "fp8_e4m3"])
def test_decode_late_keys_delayed(A, q_len, kv):
    # the reference moves after a split's first tile (the per-column maxima
    # exchanged, O and l rescaled, the probabilities written again)
    what = f"decode late keys q_len={q_len} {kv}"
    print(f"[case] delay {what}", flush=True)
    case = W.decode_late_keys(device="cuda", kv_dtype=kv, q_len=q_len)
    lc = case.launches[0]
    rows = lc.batch * q_len
    nb = A.decode_workspace_size(lc.batch, 32, 4, lc.max_kv_len, 256, q_len=q_len)
    ws = torch.empty(nb // 4, device="cuda")

    def run():
        out = out_tensor(rows, 32, "fp32")
        A.decode(lc.q[:rows], case.k_pool, case.v_pool, case.page_table, lc.kv_len, out, ws,
                 max_kv_len=lc.max_kv_len, softmax_scale=case.softmax_scale, kv_dtype=kv,
                 k_scale=case.k_scale, v_scale=case.v_scale, keys_per_split=256, q_len=q_len)
        return out

    a, b = _both(A, run)
    _same_bits(a, b, what)
    check_parity(b, oracle.attend_all(case.to("cpu")), what + " (delayed)")
