"""Seeded random shapes through every prefill entry point and the split-K
decode, against the oracle.

Each case draws a ragged batch (1-4 sequences, chunk lengths 1-150 at
offsets 0-2000), a GQA group g in {1, 2, 3, 4, 8, 16} over 1, 2 or 4 KV
heads, the pool and output dtypes, and one entry point: the plain or _ex
prefill (random sinks, log-sum-exp), the split-K prefill (random range
length or the default plan), the prefill with the KV append fused (bf16
pool; also bitwise against append_kv + prefill), or the sliding-window
prefill (head dim 256 or 512, random window, unbounded or ring cache); 24
more draw the FP8-MMA prefill with random sinks and log-sum-exp.
Decode cases draw 1-8 sequences of 1-6000 keys, 1 to 16 / g tokens each,
the range length (or the default plan), both pools, sinks and the
log-sum-exp.  Every element of every written row is held to the parity
gate; rows past the written ones must stay untouched.
"""
import numpy as np
import pytest
import torch

import attn_workloads as W
import oracle
from _gpu_helpers import (check_parity, check_parity_floor_case, floor_breaks_gate, library,
                          out_tensor, sentinel_intact)

pytestmark = pytest.mark.gpu

N_CASES = 64
LSE_ATOL = 2e-3


@pytest.fixture(scope="module")
def A():
    return library()


def draw(i):
    g_rng = np.random.default_rng(1000 + i)
    mode = ["prefill", "splitk", "append", "swa"][i % 4]
    batch = int(g_rng.integers(1, 5))
    seqs = []
    for _ in range(batch):
        ql = int(g_rng.integers(1, 151))
        st = int(g_rng.integers(0, 2001)) if g_rng.random() < 0.8 else 0
        seqs.append((ql, st, st + ql))
    g = int(g_rng.choice([1, 2, 3, 4, 8, 16]))
    hkv = int(g_rng.choice([1, 2, 4]))
    while g * hkv > 32:
        hkv //= 2
    kv = "bf16" if mode in ("append", "swa") else str(g_rng.choice(["bf16", "fp8_e4m3"]))
    out = str(g_rng.choice(["fp32", "bf16"]))
    extra = {}
    if mode == "prefill":
        extra["sinks"] = g_rng.random() < 0.5
        extra["lse"] = g_rng.random() < 0.5
    elif mode == "splitk":
        extra["kps"] = int(g_rng.choice([0, 64, 128, 320, 1024]))
        extra["sinks"] = g_rng.random() < 0.5
    elif mode == "swa":
        d = int(g_rng.choice([256, 512]))
        window = int(g_rng.integers(1, 1500))
        max_ql = max(s[0] for s in seqs)
        ring = 0
        if g_rng.random() < 0.5:
            # the ring must hold every row's band: q_len + window - 1 slots
            ring = -(-(max_ql + window - 1) // 64) + int(g_rng.integers(0, 3))
            max_pages = max(-(-s[2] // 64) for s in seqs)
            if ring >= max_pages:
                ring = 0
        extra.update(d=d, window=window, ring=ring)
    return mode, seqs, g * hkv, hkv, kv, out, extra


def _gate(launch, out, rows, hq, out_dtype, ref, what, head_dim=W.HEAD_DIM):
    """The parity gate on out[:rows]; for a bf16 output whose own rounding
    breaks the gate (see check_parity_floor_case), the same call is launched
    again into an fp32 output and the pair is checked."""
    if out_dtype == "bf16" and floor_breaks_gate(ref):
        out32 = out_tensor(rows, hq, "fp32", 0, head_dim=head_dim)
        launch(out32)
        torch.cuda.synchronize()
        check_parity_floor_case(out[:rows], out32[:rows], ref, what)
    else:
        check_parity(out[:rows], ref, what)


def _check_lse(got, ref, what):
    gl = got.cpu().numpy()
    assert np.array_equal(np.isinf(gl), np.isinf(ref)), f"{what}: lse infinities differ"
    fin = np.isfinite(ref)
    err = float(np.abs(gl[fin] - ref[fin]).max()) if fin.any() else 0.0
    assert err <= LSE_ATOL, f"{what}: lse error {err}"


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_shape(A, i):
    mode, seqs, hq, hkv, kv, out_dtype, ex = draw(i)
    what = f"case {i}: {mode} {seqs} {hq}/{hkv} {kv} out={out_dtype} {ex}"
    print(f"[case] {what}", flush=True)
    kw = dict(seqs=seqs, hq=hq, hkv=hkv, seed=2000 + i, out_dtype=out_dtype, device="cuda",
              kv_dtype=kv, q_pad_rows=2, extra_pages=2, table_pad=2)
    if mode == "swa":
        kw.update(head_dim=ex["d"], window=ex["window"], ring_pages=ex["ring"])
    case = W.build_case(f"rand{i}", **kw)
    lc = case.launches[0]
    d = case.head_dim
    out = out_tensor(lc.total_q, hq, out_dtype, 2, head_dim=d)
    common = dict(total_q=lc.total_q, max_q_len=lc.max_q_len, softmax_scale=case.softmax_scale)
    sinks = None
    lse = None
    if ex.get("sinks"):
        sinks = np.random.default_rng(i).uniform(-2.0, 6.0, hq).astype(np.float32)
    sk = None if sinks is None else torch.as_tensor(sinks, device="cuda")
    if mode == "prefill":
        if ex.get("lse"):
            lse = torch.full((lc.total_q, hq), float("nan"), device="cuda")

        def launch(o, lse_out=None):
            A.prefill(lc.q, case.k_pool, case.v_pool, case.page_table, lc.cu_seqlens_q,
                      lc.q_start, lc.kv_len, o, kv_dtype=kv, k_scale=case.k_scale,
                      v_scale=case.v_scale, sinks=sk, lse=lse_out, **common)
        launch(out, lse)
    elif mode == "splitk":
        nb = A.prefill_splitk_workspace_size(lc.batch, lc.max_q_len, lc.total_q, hq, hkv,
                                             lc.max_kv_len, ex["kps"])
        ws = torch.full((max(nb, 4) // 4,), float("nan"), device="cuda") if nb else None

        def launch(o):
            A.prefill_splitk(lc.q, case.k_pool, case.v_pool, case.page_table,
                             lc.cu_seqlens_q, lc.q_start, lc.kv_len, o, ws,
                             max_kv_len=lc.max_kv_len, keys_per_split=ex["kps"], kv_dtype=kv,
                             k_scale=case.k_scale, v_scale=case.v_scale, sinks=sk, **common)
        launch(out)
    elif mode == "append":
        # the chunk's own rows, gathered from the built cache; their slots
        # are then poisoned in the pools the two calls start from
        pages, slots = [], []
        for b, (ql, st) in enumerate(zip(lc.q_lens, lc.q_starts)):
            pos = torch.arange(st, st + ql, device="cuda")
            pages.append(case.page_table[b, pos // 64].long())
            slots.append(pos % 64)
        pages, slots = torch.cat(pages), torch.cat(slots)
        kn = case.k_pool[pages, :, slots, :].contiguous()
        vn = case.v_pool[pages, :, slots, :].contiguous()
        pools = []
        for _ in range(2):
            kp, vp = case.k_pool.clone(), case.v_pool.clone()
            kp[pages, :, slots, :] = float("nan")
            vp[pages, :, slots, :] = float("nan")
            pools.append((kp, vp))
        def launch(o):
            A.prefill_append(lc.q, kn, vn, pools[0][0], pools[0][1], case.page_table,
                             lc.cu_seqlens_q, lc.q_start, lc.kv_len, o, **common)
        launch(out)
        out2 = out_tensor(lc.total_q, hq, out_dtype, 2, head_dim=d)
        A.append_kv(kn, vn, case.page_table, lc.cu_seqlens_q, lc.q_start, pools[1][0],
                    pools[1][1])
        A.prefill(lc.q, pools[1][0], pools[1][1], case.page_table, lc.cu_seqlens_q,
                  lc.q_start, lc.kv_len, out2, **common)
        torch.cuda.synchronize()
        view = torch.int32 if out.dtype == torch.float32 else torch.int16
        assert torch.equal(out.view(view), out2.view(view)), f"{what}: fused != append + prefill"
        assert torch.equal(pools[0][0].view(torch.int16), pools[1][0].view(torch.int16))
        assert torch.equal(pools[0][1].view(torch.int16), pools[1][1].view(torch.int16))
    else:
        def launch(o):
            A.prefill_swa(lc.q, case.k_pool, case.v_pool, case.page_table, lc.cu_seqlens_q,
                          lc.q_start, lc.kv_len, o, window=case.window,
                          ring_pages=case.ring_pages, **common)
        launch(out)
    torch.cuda.synchronize()
    assert sentinel_intact(out[lc.total_q:]), f"{what}: rows past total_q were written"
    cpu = case.to("cpu")
    if sinks is not None or lse is not None:
        ref, ref_lse = oracle.attend_all_lse(cpu, sinks=sinks)
    else:
        ref, ref_lse = oracle.attend_all(cpu), None
    _gate(launch, out, lc.total_q, hq, out_dtype, ref, what, head_dim=d)
    if lse is not None:
        _check_lse(lse, ref_lse, what)


def draw_decode(i):
    g_rng = np.random.default_rng(5000 + i)
    g = int(g_rng.choice([1, 2, 4, 8, 16]))
    hkv = int(g_rng.choice([1, 2, 4]))
    q_len = int(g_rng.integers(1, min(16 // g, 5) + 1))
    batch = int(g_rng.integers(1, 9))
    lens = [int(g_rng.integers(q_len, 6001)) for _ in range(batch)]
    kps = int(g_rng.choice([0, 64, 256, 1024]))
    kv = str(g_rng.choice(["bf16", "fp8_e4m3"]))
    out = str(g_rng.choice(["fp32", "bf16"]))
    sinks = bool(g_rng.random() < 0.5)
    return lens, q_len, g * hkv, hkv, kps, kv, out, sinks


@pytest.mark.parametrize("i", range(32))
def test_random_decode_shape(A, i):
    lens, q_len, hq, hkv, kps, kv, out_dtype, with_sinks = draw_decode(i)
    what = f"decode case {i}: lens={lens} q_len={q_len} {hq}/{hkv} kps={kps} {kv} {out_dtype}"
    print(f"[case] {what}", flush=True)
    case = W.build_case(f"rdec{i}", seqs=[(q_len, L - q_len, L) for L in lens], hq=hq, hkv=hkv,
                        seed=6000 + i, out_dtype=out_dtype, device="cuda", kv_dtype=kv)
    lc = case.launches[0]
    B = lc.batch
    out = out_tensor(B * q_len, hq, out_dtype, 2)
    lse = torch.full((B * q_len, hq), float("nan"), device="cuda")
    sinks = np.random.default_rng(i).uniform(-2.0, 6.0, hq).astype(np.float32) if with_sinks \
        else None
    nbytes = A.decode_workspace_size(B, hq, hkv, lc.max_kv_len, kps, q_len=q_len)
    ws = torch.full((nbytes // 4,), float("nan"), device="cuda")
    def launch(o, lse_out=None):
        A.decode(lc.q[:B * q_len], case.k_pool, case.v_pool, case.page_table, lc.kv_len, o, ws,
                 max_kv_len=lc.max_kv_len, softmax_scale=case.softmax_scale, kv_dtype=kv,
                 k_scale=case.k_scale, v_scale=case.v_scale, keys_per_split=kps, q_len=q_len,
                 sinks=None if sinks is None else torch.as_tensor(sinks, device="cuda"),
                 lse=lse_out)
    launch(out, lse)
    torch.cuda.synchronize()
    assert sentinel_intact(out[B * q_len:]), f"{what}: rows past the batch were written"
    ref, ref_lse = oracle.attend_all_lse(case.to("cpu"), sinks=sinks)
    _gate(launch, out, B * q_len, hq, out_dtype, ref, what)
    _check_lse(lse, ref_lse, what)


@pytest.mark.parametrize("i", range(24))
def test_random_fp8_mma_shape(A, i):
    # the FP8-MMA prefill (attn_prefill_hd512_e4m3_mma) over the same kind of
    # ragged batches, with random sinks and log-sum-exp
    g_rng = np.random.default_rng(9000 + i)
    batch = int(g_rng.integers(1, 5))
    seqs = []
    for _ in range(batch):
        ql = int(g_rng.integers(1, 151))
        st = int(g_rng.integers(0, 2001)) if g_rng.random() < 0.8 else 0
        seqs.append((ql, st, st + ql))
    g = int(g_rng.choice([1, 2, 3, 4, 8, 16]))
    hkv = int(g_rng.choice([1, 2, 4]))
    while g * hkv > 32:
        hkv //= 2
    hq = g * hkv
    out_dtype = str(g_rng.choice(["fp32", "bf16"]))
    with_extras = bool(g_rng.random() < 0.5)
    what = f"fp8 mma case {i}: {seqs} {hq}/{hkv} out={out_dtype} extras={with_extras}"
    print(f"[case] {what}", flush=True)
    case = W.build_case(f"rmma{i}", seqs=seqs, hq=hq, hkv=hkv, seed=9500 + i,
                        out_dtype=out_dtype, device="cuda", kv_dtype="fp8_e4m3", q_pad_rows=2,
                        extra_pages=2, table_pad=2)
    lc = case.launches[0]
    out = out_tensor(lc.total_q, hq, out_dtype, 2)
    sinks = np.random.default_rng(i).uniform(-2.0, 6.0, hq).astype(np.float32) \
        if with_extras else None
    lse = torch.full((lc.total_q, hq), float("nan"), device="cuda") if with_extras else None
    def launch(o, lse_out=None):
        A.prefill(lc.q, case.k_pool, case.v_pool, case.page_table, lc.cu_seqlens_q,
                  lc.q_start, lc.kv_len, o, total_q=lc.total_q, max_q_len=lc.max_q_len,
                  softmax_scale=case.softmax_scale, kv_dtype="fp8_e4m3", k_scale=case.k_scale,
                  v_scale=case.v_scale, fp8_mma=True, lse=lse_out,
                  sinks=None if sinks is None else torch.as_tensor(sinks, device="cuda"))
    launch(out, lse)
    torch.cuda.synchronize()
    assert sentinel_intact(out[lc.total_q:]), f"{what}: rows past total_q were written"
    cpu = case.to("cpu")
    if with_extras:
        ref, ref_lse = oracle.attend_all_lse(cpu, sinks=sinks)
        _check_lse(lse, ref_lse, what)
    else:
        ref = oracle.attend_all(cpu)
    _gate(launch, out, lc.total_q, hq, out_dtype, ref, what)
