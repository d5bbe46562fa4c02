"""Float64 brute force for tiny inputs -- TEST INFRASTRUCTURE ONLY.

Independent of oracle_attn.c: it de-pages the pools with numpy indexing into
dense per-sequence K and V, builds the full score matrix of each (sequence,
head) with an explicit causal mask aligned at absolute positions, and applies
softmax and the value product in float64.  It pins the C oracle on small
shapes; it is far too slow and memory-hungry for the measured workloads.
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
    out = []
    for b, L in enumerate(lc.kv_lens):
        j = np.arange(L)
        pages = table[b, j // P]
        slots = j % P
        out.append((kp[pages, :, slots, :], vp[pages, :, slots, :]))
    return out


def attention(case, launch_idx: int = 0) -> np.ndarray:
    """float64 [total_q, Hq, D] outputs of one launch."""
    lc = case.launches[launch_idx]
    q = lc.q[:lc.total_q].float().double().numpy()
    g = case.num_q_heads // case.num_kv_heads
    out = np.zeros_like(q)
    dense = depage(case, launch_idx)
    row0 = 0
    for b, (ql, st, L) in enumerate(zip(lc.q_lens, lc.q_starts, lc.kv_lens)):
        K, V = dense[b]
        pos = st + np.arange(ql)[:, None]          # absolute query positions
        keys = np.arange(L)[None, :]
        visible = keys <= pos                         # causal, bottom-right aligned
        for h in range(case.num_q_heads):
            kvh = h // g
            s = (q[row0:row0 + ql, h, :] @ K[:, kvh, :].T) * float(np.float32(case.softmax_scale))
            s = np.where(visible, s, -np.inf)
            mx = s.max(axis=1, keepdims=True)
            w = np.exp(s - mx)
            out[row0:row0 + ql, h, :] = (w @ V[:, kvh, :]) / w.sum(axis=1, keepdims=True)
        row0 += ql
    return out
