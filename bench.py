#!/usr/bin/env python3
"""Benchmark of the hd512 paged GQA attention path on one MI355X.

Headline (one JSON line on stdout): causal prefill TFLOP/s of one 8192-row
chunk at positions 8192..16383 over 16384 paged keys, 32 query heads over 4
KV heads, head_dim 512, bf16 in and out -- the shape the pegainfer issue 1051
("Description") measures -- with its fraction of a bf16 GEMM measured in the
same process and of the chip's dense bf16 MFMA peak.  One step is one prefill
launch; inputs are resident in HBM before the timed region.

Also reported: split-K decode (batch 64, 8 query heads over 4 KV heads,
lengths U{4096..28672}, bf16 and FP8-E4M3 pools) in us per call and GB/s of
live KV bytes against an HBM read probe taken in the same process; the other
prefill workloads; and the CPU oracle timed on a bounded sample of the
headline workload (a baseline, not a target).

The headline is timed as the contract asks: K launches after W warmup
launches, events on the launch stream, cut into 7 windows (median, min, max
reported beside the mean) with clock stamps around them.  Every other figure
is the median of 7 replays of a HIP graph holding 8-100 calls, so that the
host's launch overhead (about 0.17 ms per call from Python) does not enter
the shorter launches.

FLOP convention: 4 * head_dim per visible (query, key) pair and head.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA (no sparsity)
PEAK_HBM_GBPS = 8000.0        # MI355X HBM3E

# HBM bytes per launch of the headline prefill kernel, from two rocprofv3
# counter runs (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch) of this script,
# each scaled by what the same counter reads for the 1 GiB device-to-device
# copy this script makes (profiles/prefill_hd512_chunk8192_at_8192.md).  The
# figure is only valid for the kernel sources it was taken with: their
# SHA-256 is checked at run time and traffic is reported as null otherwise.
TRAFFIC_RECORD = {
    "sources": ["attention_hd512_gqa_amd/csrc/prefill_hd512.hip",
                "attention_hd512_gqa_amd/csrc/prefill_common.h",
                "attention_hd512_gqa_amd/csrc/device_common.h"],
    "sha256": "554357e1e25d8eadaf453c310006660510032aed151989912676826fc6366efd",
    "fetch_bytes": 1988078376,
    "write_bytes": 268435456,
    "profile": "profiles/prefill_hd512_chunk8192_at_8192.md",
}


def recorded_traffic():
    import hashlib
    h = hashlib.sha256()
    for rel in TRAFFIC_RECORD["sources"]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    digest = h.hexdigest()
    if TRAFFIC_RECORD["sha256"] != digest or TRAFFIC_RECORD["fetch_bytes"] is None:
        return None, digest
    return TRAFFIC_RECORD["fetch_bytes"] + TRAFFIC_RECORD["write_bytes"], digest


def clock_summary(stamps):
    """Mean shader clock over the region between two clock-stamp launches.

    stamps[0] and stamps[1] hold, per workgroup, (where: XCD << 32 | HW_ID,
    shader-cycle counter, 100 MHz counter).  The cycle counter is not
    synchronised between compute units, so stamps are paired by compute unit
    (XCD, shader engine, shader array, CU): cycles over ticks, times 100 MHz,
    is that unit's mean clock; the median, min and max over the units that
    hold a stamp of both launches are reported.
    """
    def where(w):
        w = int(w)
        return (w >> 32, (w >> 8) & 0xFF)   # XCD; CU | SH << 4 | SE << 5
    first = {}
    for row in stamps[0]:
        first.setdefault(where(row[0]), row)
    clocks = []
    for row in stamps[1]:
        k = where(row[0])
        if k in first:
            a = first.pop(k)
            ticks = int(row[2]) - int(a[2])
            if ticks > 0:
                clocks.append((int(row[1]) - int(a[1])) / ticks * 100.0)
    if not clocks:
        return None
    clocks.sort()
    return {"median_mhz": clocks[len(clocks) // 2], "min_mhz": clocks[0], "max_mhz": clocks[-1],
            "compute_units": len(clocks),
            "how": "s_memtime cycles / s_memrealtime 100 MHz ticks per compute unit across "
                   "the timed steps"}


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=30)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-decode", action="store_true")
    p.add_argument("--no-extra", action="store_true", help="skip the other prefill workloads")
    p.add_argument("--no-gemm", action="store_true", help="skip the same-process GEMM roofline")
    p.add_argument("--cpu-seconds", type=float, default=15.0,
                   help="target wall time of the CPU-oracle sample")
    return p.parse_args()


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} (WORLD_SIZE={world}) is not "
              "supported: this library has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import attention_hd512_gqa_amd as A
    import attn_workloads as W

    A.lib()
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()

    def timed(fn, n, warmup):
        """Mean ms per call of fn over n calls after warmup, events on the launch stream."""
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    def graph_time(fn, calls=20, windows=7):
        """ms per call of fn: `calls` calls captured in one HIP graph (so the
        host's launch overhead is not measured), replayed `windows` times;
        median, min and max over the windows.  fn launches on torch's current
        stream, which is the capture stream while the graph is recorded."""
        fn()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(calls):
                fn()
        g.replay()
        torch.cuda.synchronize()
        ts = []
        for _ in range(windows):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            g.replay()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) / calls)
        del g
        ts.sort()
        return {"ms": ts[len(ts) // 2], "ms_min": ts[0], "ms_max": ts[-1],
                "how": f"median of {windows} replays of a graph of {calls} calls"}

    # ---- same-process bf16 GEMM roofline ---------------------------------
    def gemm_rate():
        best = 0.0
        for n in (8192, 16384):
            a = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
            b = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
            ms = timed(lambda: torch.matmul(a, b), 10 if n == 8192 else 4, 3)
            best = max(best, 2.0 * n ** 3 / (ms * 1e-3) / 1e12)
            del a, b
        torch.cuda.empty_cache()
        return best

    gemm_before = 0.0 if args.no_gemm else gemm_rate()
    log(f"bf16 GEMM roofline (torch.matmul, before): {gemm_before:.1f} TFLOP/s")

    # ---- same-process HBM read probe --------------------------------------
    hbm_bytes = 8 << 30
    buf = torch.empty(hbm_bytes, dtype=torch.uint8, device="cuda")
    sink = torch.empty(A.hbm_probe_sink_words(hbm_bytes), dtype=torch.int32, device="cuda")
    ms = timed(lambda: A.hbm_read_probe(buf, sink), 10, 3)
    hbm_read = hbm_bytes / (ms * 1e-3) / 1e9
    del buf, sink
    torch.cuda.empty_cache()
    log(f"HBM read probe over 8 GiB: {hbm_read:.0f} GB/s")
    # 1 GiB device-to-device copy: a rate for reference and, under rocprofv3,
    # the calibration of the FETCH_SIZE / WRITE_SIZE counters (1 GiB each way)
    cal_bytes = 1 << 30
    src = torch.empty(cal_bytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    ms = timed(lambda: dst.copy_(src), 5, 2)
    d2d = 2 * cal_bytes / (ms * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    log(f"D2D copy of 1 GiB: {d2d:.0f} GB/s (read + write)")

    # ---- headline: prefill of one 8192-row chunk at 8192..16383 ------------
    case = W.chunk_prefill_8k_at_8k(device="cuda")
    lc = case.launches[0]
    out = torch.empty((lc.total_q, case.num_q_heads, W.HEAD_DIM), dtype=torch.bfloat16,
                      device="cuda")
    flops = W.prefill_flops(lc.q_lens, lc.q_starts, lc.kv_lens, case.num_q_heads)

    def prefill_step(c=case, l=lc, o=out):
        A.prefill(l.q, c.k_pool, c.v_pool, c.page_table, l.cu_seqlens_q, l.q_start, l.kv_len, o,
                  total_q=l.total_q, max_q_len=l.max_q_len, softmax_scale=c.softmax_scale,
                  stream=stream)

    for _ in range(args.warmup):
        prefill_step()
    # the K timed steps, cut into up to 7 windows by events on the launch
    # stream (the median window is reported beside the K-step mean), with
    # clock stamps just outside the timed region
    n_win = max(1, min(7, args.steps))
    bounds = [round(i * args.steps / n_win) for i in range(n_win + 1)]
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n_win + 1)]
    stamps = torch.zeros((2, 256, 3), dtype=torch.int64, device="cuda")
    torch.cuda.synchronize()
    A.clock_stamps(stamps[0], stream=stream)
    ev[0].record(stream)
    for w in range(n_win):
        for _ in range(bounds[w + 1] - bounds[w]):
            prefill_step()
        ev[w + 1].record(stream)
    A.clock_stamps(stamps[1], stream=stream)
    torch.cuda.synchronize()
    ms_step = ev[0].elapsed_time(ev[-1]) / args.steps
    tflops = flops / (ms_step * 1e-3) / 1e12
    win_ms = sorted(ev[w].elapsed_time(ev[w + 1]) / (bounds[w + 1] - bounds[w])
                    for w in range(n_win))
    clock = clock_summary(stamps.cpu().numpy())
    log(f"prefill chunk 8192@8192: {ms_step:.3f} ms/launch, {tflops:.1f} TFLOP/s; windows "
        f"{win_ms[0]:.3f}/{win_ms[len(win_ms) // 2]:.3f}/{win_ms[-1]:.3f} ms (min/median/max); "
        f"shader clock {clock['median_mhz'] if clock else float('nan'):.0f} MHz (median over CUs)")
    assert torch.isfinite(out.float()).all()

    extra = {}
    if not args.no_extra:
        def rate(flop, t):
            return dict(t, tflops=flop / (t["ms"] * 1e-3) / 1e12)

        def pf(c, l, o, **kw):
            # a prefill launch on torch's current stream (graph capture)
            return lambda: A.prefill(l.q, c.k_pool, c.v_pool, c.page_table, l.cu_seqlens_q,
                                     l.q_start, l.kv_len, o, total_q=l.total_q,
                                     max_q_len=l.max_q_len, softmax_scale=c.softmax_scale,
                                     kv_dtype=c.kv_dtype, k_scale=c.k_scale, v_scale=c.v_scale,
                                     **kw)
        wsp = torch.empty(A.prefill_persistent_workspace_size() // 4, dtype=torch.int32,
                          device="cuda")

        def pers(c, l, o):
            return lambda: A.prefill_persistent(l.q, c.k_pool, c.v_pool, c.page_table,
                                                l.cu_seqlens_q, l.q_start, l.kv_len, o, wsp,
                                                total_q=l.total_q, max_q_len=l.max_q_len,
                                                softmax_scale=c.softmax_scale,
                                                kv_dtype=c.kv_dtype, k_scale=c.k_scale,
                                                v_scale=c.v_scale)
        # the headline chunk, graph-timed too, next to the timing above
        extra["chunk_prefill_8192_at_8192_graph"] = rate(flops, graph_time(pf(case, lc, out), 8))
        extra["chunk_prefill_8192_at_8192_persistent"] = rate(
            flops, graph_time(pers(case, lc, out), 8))
        # 2048 rows at offset 0: one-workgroup-per-unit and persistent launches
        c2 = W.chunk_prefill_2k(device="cuda")
        l2 = c2.launches[0]
        o2 = torch.empty((l2.total_q, c2.num_q_heads, W.HEAD_DIM), dtype=torch.bfloat16,
                         device="cuda")
        f2 = W.prefill_flops(l2.q_lens, l2.q_starts, l2.kv_lens, c2.num_q_heads)
        extra["chunk_prefill_2048"] = rate(f2, graph_time(pf(c2, l2, o2)))
        extra["chunk_prefill_2048_persistent"] = rate(f2, graph_time(pers(c2, l2, o2)))
        del c2, o2
        # the 32K long-MQA prompt as eight chunks: each chunk, and the prompt
        c4 = W.long_mqa_32k(device="cuda")
        o4 = torch.empty((4096, c4.num_q_heads, W.HEAD_DIM), dtype=torch.float32, device="cuda")
        per_chunk, per_chunk_p, total, total_p, f4 = [], [], 0.0, 0.0, 0
        for l4 in c4.launches:
            fc = W.prefill_flops(l4.q_lens, l4.q_starts, l4.kv_lens, c4.num_q_heads)
            t = rate(fc, graph_time(pf(c4, l4, o4), 8))
            tp = rate(fc, graph_time(pers(c4, l4, o4), 8))
            per_chunk.append({"ms": t["ms"], "tflops": t["tflops"]})
            per_chunk_p.append({"ms": tp["ms"], "tflops": tp["tflops"]})
            total += t["ms"]
            total_p += tp["ms"]
            f4 += fc
        extra["long_mqa_32k_8x4096"] = {"ms_per_prompt": total,
                                        "tflops": f4 / (total * 1e-3) / 1e12,
                                        "per_chunk": per_chunk}
        extra["long_mqa_32k_8x4096_persistent"] = {"ms_per_prompt": total_p,
                                                   "tflops": f4 / (total_p * 1e-3) / 1e12,
                                                   "per_chunk": per_chunk_p}
        del c4, o4
        # the tiny MQA prefill (256 rows, one workgroup per 16 tokens)
        c1 = W.tiny_prefill_mqa(device="cuda")
        l1 = c1.launches[0]
        o1 = torch.empty((l1.total_q, c1.num_q_heads, W.HEAD_DIM), dtype=torch.float32,
                         device="cuda")
        f1 = W.prefill_flops(l1.q_lens, l1.q_starts, l1.kv_lens, c1.num_q_heads)
        t1 = rate(f1, graph_time(pf(c1, l1, o1), 100))
        extra["tiny_prefill_mqa_256"] = dict(t1, us_per_launch=t1["ms"] * 1e3,
                                             note="16 workgroups on 256 compute units")
        del c1, o1
        torch.cuda.empty_cache()
        # late dominant keys: every workgroup raises its rows' softmax
        # reference two or three times (the cost of the overflow path)
        for kv_dtype, mma in (("bf16", False), ("fp8_e4m3", True)):
            cl = W.chunk_prefill_8k_at_8k_late_keys(device="cuda", kv_dtype=kv_dtype)
            ll = cl.launches[0]
            extra[cl.name + ("_mma" if mma else "")] = rate(
                flops, graph_time(pf(cl, ll, out, fp8_mma=mma), 8))
            del cl
        torch.cuda.empty_cache()
        # the headline chunk over an FP8-E4M3 cache (same values, per-tensor scales)
        c8 = W.chunk_prefill_8k_at_8k(device="cuda", kv_dtype="fp8_e4m3")
        l8 = c8.launches[0]
        t8 = rate(flops, graph_time(pf(c8, l8, out), 8))
        extra["chunk_prefill_8192_at_8192_fp8"] = t8
        # the same bytes with both products on the block-scaled FP8 MFMA
        t8m = rate(flops, graph_time(pf(c8, l8, out, fp8_mma=True), 8))
        t8m["frac_of_fp8_dense_peak"] = t8m["tflops"] / 5000.0
        extra["chunk_prefill_8192_at_8192_fp8_mma"] = t8m
        log(f"FP8 pool: widened {t8['ms']:.3f} ms, FP8 MFMA {t8m['ms']:.3f} ms "
            f"({t8m['tflops']:.1f} TFLOP/s)")
        del c8
        torch.cuda.empty_cache()
        # a short chunk over a long prefix: single pass against split-K (the
        # E4M3 pool on both FP8 kernels)
        for kv_dtype, mma in (("bf16", False), ("fp8_e4m3", False), ("fp8_e4m3", True)):
            cp = W.prefix_prefill_512_at_32k(device="cuda", kv_dtype=kv_dtype)
            lp = cp.launches[0]
            op = torch.empty((lp.total_q, cp.num_q_heads, W.HEAD_DIM), dtype=torch.bfloat16,
                             device="cuda")
            fp = W.prefill_flops(lp.q_lens, lp.q_starts, lp.kv_lens, cp.num_q_heads)
            nb = A.prefill_splitk_workspace_size(lp.batch, lp.max_q_len, lp.total_q,
                                                 cp.num_q_heads, cp.num_kv_heads,
                                                 lp.max_kv_len, 0)
            ws = torch.empty((max(nb, 4) // 4,), dtype=torch.float32, device="cuda")

            def split(c=cp, l=lp, o=op, w=ws):
                A.prefill_splitk(l.q, c.k_pool, c.v_pool, c.page_table, l.cu_seqlens_q,
                                 l.q_start, l.kv_len, o, w, total_q=l.total_q,
                                 max_q_len=l.max_q_len, max_kv_len=l.max_kv_len,
                                 softmax_scale=c.softmax_scale, kv_dtype=c.kv_dtype,
                                 k_scale=c.k_scale, v_scale=c.v_scale, fp8_mma=mma)
            t_1 = graph_time(pf(cp, lp, op, fp8_mma=mma))
            t_s = graph_time(split)
            extra[cp.name + ("_mma" if mma else "")] = {
                "single_pass_ms": t_1["ms"], "single_pass_tflops": fp / (t_1["ms"] * 1e-3) / 1e12,
                "splitk_ms": t_s["ms"], "splitk_tflops": fp / (t_s["ms"] * 1e-3) / 1e12,
                "splitk_workspace_bytes": nb, "how": t_s["how"]}
            del cp, op, ws
            torch.cuda.empty_cache()
        # sliding-window (local) layers: head dim 256, window 1024, ring caches
        cs = W.swa_prefill_hd256_8k_at_8k(device="cuda")
        ls = cs.launches[0]
        os_ = torch.empty((ls.total_q, cs.num_q_heads, cs.head_dim), dtype=torch.bfloat16,
                          device="cuda")

        def swa(c, l, o):
            return lambda: A.prefill_swa(l.q, c.k_pool, c.v_pool, c.page_table, l.cu_seqlens_q,
                                         l.q_start, l.kv_len, o, total_q=l.total_q,
                                         max_q_len=l.max_q_len, softmax_scale=c.softmax_scale,
                                         window=c.window, ring_pages=c.ring_pages)
        f_w = W.prefill_flops(ls.q_lens, ls.q_starts, ls.kv_lens, cs.num_q_heads,
                              head_dim=cs.head_dim, window=cs.window)
        extra[cs.name] = dict(rate(f_w, graph_time(swa(cs, ls, os_))), flop_per_launch=f_w)
        del cs, os_
        cd = W.swa_decode_hd256_b64(device="cuda")
        ld = cd.launches[0]
        od = torch.empty((ld.total_q, cd.num_q_heads, cd.head_dim), dtype=torch.bfloat16,
                         device="cuda")
        t_d = graph_time(swa(cd, ld, od), 100)
        nb_d = W.decode_kv_bytes(ld.kv_lens, cd.num_kv_heads, cd.head_dim, 2, cd.window)
        extra[cd.name] = dict(t_d, us_per_call=t_d["ms"] * 1e3, kv_bytes=nb_d,
                              GB_per_s=nb_d / (t_d["ms"] * 1e-3) / 1e9)
        del cd, od
        torch.cuda.empty_cache()
        log(f"other prefill workloads: {json.dumps(extra)}")

    # ---- split-K decode ------------------------------------------------------
    decode = {}
    if not args.no_decode:
        for kv_dtype in ("bf16", "fp8_e4m3"):
            dc = W.decode_b64(device="cuda", kv_dtype=kv_dtype)
            dl = dc.launches[0]
            dout = torch.empty((dl.batch, dc.num_q_heads, W.HEAD_DIM), dtype=torch.bfloat16,
                               device="cuda")
            ws = torch.empty(A.decode_workspace_size(dl.batch, dc.num_q_heads, dc.num_kv_heads,
                                                     dl.max_kv_len) // 4,
                             dtype=torch.float32, device="cuda")
            qd = dl.q[:dl.batch].contiguous()

            def decode_call():
                A.decode(qd, dc.k_pool, dc.v_pool, dc.page_table, dl.kv_len, dout, ws,
                         max_kv_len=dl.max_kv_len, softmax_scale=dc.softmax_scale,
                         kv_dtype=dc.kv_dtype, k_scale=dc.k_scale, v_scale=dc.v_scale)
            # median of 7 replays of a graph of 20 calls (P3's 7 windows)
            for _ in range(10):
                decode_call()
            t = graph_time(decode_call)
            us = t["ms"] * 1e3
            nbytes = W.decode_kv_bytes(dl.kv_lens, dc.num_kv_heads, W.HEAD_DIM,
                                       1 if kv_dtype == "fp8_e4m3" else 2)
            gbps = nbytes / (us * 1e-6) / 1e9
            decode[kv_dtype] = {
                "workload": dc.name, "us_per_call": us, "us_min": t["ms_min"] * 1e3,
                "us_max": t["ms_max"] * 1e3, "kv_bytes": nbytes, "GB_per_s": gbps,
                "frac_of_hbm_probe": gbps / hbm_read, "frac_of_hbm_peak": gbps / PEAK_HBM_GBPS,
                "kernels": "split + merge, one stream", "how": t["how"]}
            log(f"decode {kv_dtype}: {us:.1f} us/call, {gbps:.0f} GB/s "
                f"({100 * gbps / hbm_read:.1f}% of probe)")
            del dc, dout, ws, qd
            torch.cuda.empty_cache()

    # ---- multi-token decode at g = 8 (routed through the split-K prefill) -----
    decode_mtp = {}
    if not args.no_decode:
        for kv_dtype in ("bf16", "fp8_e4m3"):
            mc = W.decode_mtp_b64(device="cuda", kv_dtype=kv_dtype)
            ml = mc.launches[0]
            q_len = ml.max_q_len
            mout = torch.empty((ml.total_q, mc.num_q_heads, W.HEAD_DIM), dtype=torch.bfloat16,
                               device="cuda")
            mws = torch.empty(A.decode_workspace_size(ml.batch, mc.num_q_heads, mc.num_kv_heads,
                                                      ml.max_kv_len, q_len=q_len) // 4,
                              dtype=torch.float32, device="cuda")

            def mtp_call():
                A.decode(ml.q, mc.k_pool, mc.v_pool, mc.page_table, ml.kv_len, mout, mws,
                         max_kv_len=ml.max_kv_len, softmax_scale=mc.softmax_scale,
                         kv_dtype=mc.kv_dtype, k_scale=mc.k_scale, v_scale=mc.v_scale,
                         q_len=q_len)
            for _ in range(5):
                mtp_call()
            t = graph_time(mtp_call)
            us = t["ms"] * 1e3
            nbytes = W.decode_kv_bytes(ml.kv_lens, mc.num_kv_heads, W.HEAD_DIM,
                                       1 if kv_dtype == "fp8_e4m3" else 2)
            mflops = W.prefill_flops(ml.q_lens, ml.q_starts, ml.kv_lens, mc.num_q_heads)
            gbps = nbytes / (us * 1e-6) / 1e9
            decode_mtp[kv_dtype] = {
                "workload": mc.name, "q_len": q_len, "us_per_call": us,
                "us_min": t["ms_min"] * 1e3, "us_max": t["ms_max"] * 1e3, "kv_bytes": nbytes,
                "GB_per_s": gbps, "frac_of_hbm_probe": gbps / hbm_read,
                "useful_TFLOP_per_s": mflops / (us * 1e-6) / 1e12,
                "kernels": "split (tile kernel, 3 column blocks of 16) + merge",
                "how": t["how"]}
            log(f"decode q_len={q_len} g=8 {kv_dtype}: {us:.1f} us/call, {gbps:.0f} GB/s "
                f"({100 * gbps / hbm_read:.1f}% of probe), "
                f"{mflops / (us * 1e-6) / 1e12:.0f} useful TFLOP/s")
            del mc, ml, mout, mws
            torch.cuda.empty_cache()

    # ---- paged KV append of the headline chunk (HBM-bound data movement) -----
    append = {}
    if not args.no_decode:
        for kv_dtype in ("bf16", "fp8_e4m3"):
            ac = W.chunk_prefill_8k_at_8k(device="cuda", kv_dtype=kv_dtype)
            al = ac.launches[0]
            kn = torch.randn(al.total_q, ac.num_kv_heads, W.HEAD_DIM, device="cuda").to(torch.bfloat16)
            vn = torch.randn_like(kn)
            kp, vp = ac.k_pool.clone(), ac.v_pool.clone()

            def append_call():
                A.append_kv(kn, vn, ac.page_table, al.cu_seqlens_q, al.q_start, kp, vp,
                            kv_dtype=kv_dtype, k_scale=ac.k_scale, v_scale=ac.v_scale)
            ms = graph_time(append_call, 100)["ms"]
            moved = 2 * kn.numel() * 2 + 2 * kn.numel() * (2 if kv_dtype == "bf16" else 1)
            append[kv_dtype] = {"us_per_call": ms * 1e3, "bytes": moved,
                                "GB_per_s": moved / (ms * 1e-3) / 1e9}
            log(f"append_kv {kv_dtype} (8192 rows x {ac.num_kv_heads} KV heads): "
                f"{ms * 1e3:.1f} us, {moved / (ms * 1e-3) / 1e9:.0f} GB/s")
            if kv_dtype == "bf16":
                # the append fused into the prefill launch against the two
                # launches, with the chunk's own rows as the new rows
                pos = torch.arange(al.q_starts[0], al.q_starts[0] + al.total_q, device="cuda")
                pg = ac.page_table[0, pos // 64].long()
                kn = ac.k_pool[pg, :, pos % 64, :].contiguous()
                vn = ac.v_pool[pg, :, pos % 64, :].contiguous()
                ao = torch.empty((al.total_q, ac.num_q_heads, W.HEAD_DIM),
                                 dtype=torch.bfloat16, device="cuda")

                def fused_call():
                    A.prefill_append(al.q, kn, vn, kp, vp, ac.page_table, al.cu_seqlens_q,
                                     al.q_start, al.kv_len, ao, total_q=al.total_q,
                                     max_q_len=al.max_q_len, softmax_scale=ac.softmax_scale)

                def unfused_call():
                    append_call()
                    A.prefill(al.q, kp, vp, ac.page_table, al.cu_seqlens_q, al.q_start,
                              al.kv_len, ao, total_q=al.total_q, max_q_len=al.max_q_len,
                              softmax_scale=ac.softmax_scale)
                ms_f = graph_time(fused_call, 8)["ms"]
                ms_u = graph_time(unfused_call, 8)["ms"]
                append["prefill_with_append_bf16"] = {
                    "fused_ms": ms_f, "append_then_prefill_ms": ms_u,
                    "fused_tflops": flops / (ms_f * 1e-3) / 1e12}
                log(f"prefill 8192@8192 with the append fused: {ms_f:.3f} ms "
                    f"({flops / (ms_f * 1e-3) / 1e12:.1f} TFLOP/s); append_kv + prefill: "
                    f"{ms_u:.3f} ms")
                del ao
            del ac, kn, vn, kp, vp
            torch.cuda.empty_cache()

    gemm_after = 0.0 if args.no_gemm else gemm_rate()
    log(f"bf16 GEMM roofline (after): {gemm_after:.1f} TFLOP/s")
    gemm = max(gemm_before, gemm_after)

    # ---- CPU oracle on a bounded sample of the headline workload ------------
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        host = case.to("cpu")
        cores = len(os.sched_getaffinity(0))
        hq = case.num_q_heads

        def run_tokens(tokens):
            rows = (np.asarray(tokens)[:, None] * hq + np.arange(hq)[None, :]).reshape(-1)
            t0 = time.perf_counter()
            oracle.attend_rows(host, rows, threads=cores)
            wall = time.perf_counter() - t0
            pairs = sum(min(lc.q_starts[0] + t + 1, lc.kv_lens[0]) for t in tokens) * hq
            return wall, pairs * 4 * W.HEAD_DIM

        probe_tokens = [lc.total_q - 1 - 64 * i for i in range(4)]
        wall, f = run_tokens(probe_tokens)
        rate = f / wall
        n_tok = max(4, min(lc.total_q, int(args.cpu_seconds * rate / (f / len(probe_tokens)))))
        tokens = sorted(set(np.linspace(0, lc.total_q - 1, n_tok).astype(int).tolist()))
        wall, f = run_tokens(tokens)
        cpu = {"value": f / wall / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
               "sample": f"{len(tokens)} query rows spread over the 8192-row chunk, all "
                         f"{hq} heads ({f / 1e9:.1f} GFLOP algorithmic, {wall:.1f} s wall, "
                         f"fp32 C oracle, {cores} threads)"}
        log(f"CPU oracle: {cpu['value'] * 1e3:.2f} GFLOP/s on {cores} threads")

    traffic, digest = recorded_traffic()
    # unique bytes of one launch: Q, the visible K and V rows of each KV head, O
    algo_bytes = (lc.total_q * case.num_q_heads * W.HEAD_DIM * 2 * 2
                  + 2 * lc.kv_lens[0] * case.num_kv_heads * W.HEAD_DIM * 2)
    result = {
        "metric": "hd512 causal prefill TFLOP/s + % of same-process bf16 MFMA GEMM peak",
        "value": tflops,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 Q/K/V, shuffled 64-token page table)",
        "config": {"workload": case.name, "q_rows": lc.total_q, "q_start": lc.q_starts[0],
                   "kv_len": lc.kv_lens[0], "q_heads": case.num_q_heads,
                   "kv_heads": case.num_kv_heads, "head_dim": W.HEAD_DIM,
                   "page_size": W.PAGE_SIZE, "out_dtype": "bf16", "flop_per_launch": flops},
        "windows": {"n": n_win, "median_ms": win_ms[len(win_ms) // 2], "min_ms": win_ms[0],
                    "max_ms": win_ms[-1],
                    "median_tflops": flops / (win_ms[len(win_ms) // 2] * 1e-3) / 1e12,
                    "how": "the K timed steps cut into windows by events; ms per launch"},
        "clock": clock,
        "gemm_roofline": {"tflops": gemm, "before": gemm_before, "after": gemm_after,
                          "frac": (tflops / gemm) if gemm else None,
                          "how": "torch.matmul bf16 8192^3 and 16384^3, best"},
        "roofline": {"bound": "mfma", "achieved": tflops, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": tflops / PEAK_BF16_TFLOPS, "traffic": traffic,
                     "traffic_unit": "HBM bytes per launch (FETCH + WRITE, calibrated)",
                     "traffic_algorithmic_bytes": algo_bytes,
                     "traffic_source": TRAFFIC_RECORD["profile"] if traffic else None,
                     "kernel": "prefill_hd512_kernel", "kernel_sources_sha256": digest},
        "hbm": {"read_probe_GB_per_s": hbm_read, "probe_bytes": hbm_bytes,
                "d2d_copy_GB_per_s": d2d},
        "decode": decode,
        "decode_multi_token": decode_mtp,
        "append_kv": append,
        "prefill_other": extra,
        "cpu_baseline": cpu,
    }
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
