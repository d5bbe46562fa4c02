"""Float64 brute force for tiny inputs -- TEST INFRASTRUCTURE ONLY.

Independent of oracle_attn.c: it de-pages the pools with numpy indexing into
dense per-sequence K and V (through the ring when the cache is one: key j at
slot j % C, keys older than the last C marked NaN), builds the full score
matrix of each (sequence, head) with an explicit causal mask aligned at
absolute positions, cut to the last `window` positions when there is a
window, and applies softmax and the value product in float64.  It pins the C
oracle on small shapes; it is far too slow and memory-hungry for the measured
workloads.
"""
from __future__ import annotations

from typing import List, Tuple

import numpy as np
import torch


def _to_f64(pool: torch.Tensor, kv_dtype: str, scale: float) -> np.ndarray:
    if kv_dtype == "bf16":
        return pool.float().double().numpy()
    return pool.view(torch.float8_e4m3fn).float().double().numpy() * float(scale)


def depage(case, launch_idx: int = 0) -> List[Tuple[np.ndarray, np.ndarray]]:
    """Dense (K_b, V_b), each float64 [kv_len_b, Hkv, D], for every sequence."""
    lc = case.launches[launch_idx]
    table = case.page_table.cpu().numpy()
    P = int(case.k_pool.shape[2])
    kp = _to_f64(case.k_pool.cpu(), case.kv_dtype, case.k_scale)
    vp = _to_f64(case.v_pool.cpu(), case.kv_dtype, case.v_scale)
    C = int(getattr(case, "ring_pages", 0) or 0) * P
    out = []
    for b, L in enumerate(lc.kv_lens):
        j = np.arange(L)
        c = j % C if C else j
        pages = table[b, c // P]
        slots = c % P
        K, V = kp[pages, :, slots, :], vp[pages, :, slots, :]
        if C and L > C:            # overwritten by later keys of the ring
            K[:L - C] = np.nan
            V[:L - C] = np.nan
        out.append((K, V))
    return out


def attention(case, launch_idx: int = 0) -> np.ndarray:
    """float64 [total_q, Hq, D] outputs of one launch."""
    return attention_lse(case, launch_idx)[0]


def attention_lse(case, launch_idx: int = 0, sinks=None):
    """float64 outputs [total_q, Hq, D] and log-sum-exps [total_q, Hq] of one
    launch; `sinks` (one logit per query head, or None) joins each softmax as a
    term with no value row."""
    lc = case.launches[launch_idx]
    q = lc.q[:lc.total_q].float().double().numpy()
    g = case.num_q_heads // case.num_kv_heads
    out = np.zeros_like(q)
    lse = np.full(q.shape[:2], -np.inf)
    dense = depage(case, launch_idx)
    row0 = 0
    for b, (ql, st, L) in enumerate(zip(lc.q_lens, lc.q_starts, lc.kv_lens)):
        K, V = dense[b]
        pos = st + np.arange(ql)[:, None]          # absolute query positions
        keys = np.arange(L)[None, :]
        visible = keys <= pos                         # causal, bottom-right aligned
        W = int(getattr(case, "window", 0) or 0)
        if W:
            visible &= keys > pos - W                  # the last W positions
        for h in range(case.num_q_heads):
            kvh = h // g
            s = (q[row0:row0 + ql, h, :] @ K[:, kvh, :].T) * float(np.float32(case.softmax_scale))
            s = np.where(visible, s, -np.inf)
            if sinks is not None:   # one more softmax column, weight only
                s = np.concatenate([s, np.full((ql, 1), float(sinks[h]))], axis=1)
            mx = s.max(axis=1, keepdims=True) if s.shape[1] else np.full((ql, 1), -np.inf)
            ok = ~np.isneginf(mx[:, 0])   # a row with a visible key (NaN stays NaN)
            w = np.exp(s - np.where(np.isfinite(mx), mx, 0.0))
            den = w.sum(axis=1)
            # rows the ring no longer holds are NaN: a visible one poisons its
            # score, a masked one must not leak through a zero weight
            vals = np.nan_to_num(V[:, kvh, :], nan=0.0)
            num = w[:, :L] @ vals if L else np.zeros((ql, vals.shape[-1]))
            out[row0:row0 + ql, h, :] = np.where(ok[:, None], num / np.where(ok, den, 1.0)[:, None], 0.0)
            lse[row0:row0 + ql, h] = np.where(ok, mx[:, 0] + np.log(np.where(ok, den, 1.0)), -np.inf)
        row0 += ql
    return out, lse
