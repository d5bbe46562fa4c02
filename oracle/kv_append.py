"""Oracle of the paged KV append -- TEST INFRASTRUCTURE ONLY.

Only the tests may import it; the library never does.  Plain numpy written
from the definition: token i of sequence b sits at position
p = q_start[b] + i and its key and value rows (every KV head) go to page
page_table[b][p // page_size], slot p % page_size (one page per key tile of
the attention kernels: pegainfer issue 1051, "Proposed Plan").  Positions
outside the table and page ids outside the pool are skipped.

An FP8-E4M3 pool stores x / scale saturated to +-448 and rounded to the
nearest E4M3FN value, ties to the even code, found here by exhaustive search
over the 254 finite codes decoded with this package's own decoder.

Parity status: pinned by tests/test_kv_append_oracle.py against torch's
float8_e4m3fn conversion (values inside the range), round trips of every
finite code and exact midpoints, and a brute-force per-element scatter.
"""
from __future__ import annotations

import numpy as np
import torch

from . import e4m3_to_f32

_POS = np.arange(0x7F, dtype=np.uint8)            # 0x00 .. 0x7E: finite, >= 0
_POS_VAL = e4m3_to_f32(_POS).astype(np.float64)   # ascending


def e4m3_encode(x: np.ndarray, scale: float) -> np.ndarray:
    """Codes of x / scale (fp32 division), saturated to +-448, nearest, ties to even."""
    y = (np.asarray(x, dtype=np.float32) / np.float32(scale)).astype(np.float32)
    nan = np.isnan(y)
    y = np.where(nan, 0.0, np.clip(y, -448.0, 448.0)).astype(np.float64)
    a = np.abs(y)
    hi = np.clip(np.searchsorted(_POS_VAL, a, side="left"), 0, len(_POS_VAL) - 1)
    lo = np.clip(hi - 1, 0, len(_POS_VAL) - 1)
    d_lo = np.abs(a - _POS_VAL[lo])
    d_hi = np.abs(_POS_VAL[hi] - a)
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (_POS[hi] % 2 == 0) & (hi != lo))
    code = np.where(pick_hi, _POS[hi], _POS[lo]).astype(np.uint8)
    code = np.where(np.signbit(y), code | np.uint8(0x80), code).astype(np.uint8)
    return np.where(nan, np.uint8(0x7F), code).astype(np.uint8)


def append(k_pool: np.ndarray, v_pool: np.ndarray, k_new: torch.Tensor, v_new: torch.Tensor,
           page_table: np.ndarray, cu_seqlens: np.ndarray, q_start: np.ndarray, kv_dtype: str,
           k_scale: float = 1.0, v_scale: float = 1.0):
    """Returns copies of the pools (uint16 bf16 bits or uint8 E4M3 codes,
    [pages, Hkv, page_size, D]) with the new rows written."""
    kp, vp = k_pool.copy(), v_pool.copy()
    page_size = kp.shape[2]
    max_pages = page_table.shape[1]
    kn = k_new.contiguous().view(torch.int16).numpy().view(np.uint16)
    vn = v_new.contiguous().view(torch.int16).numpy().view(np.uint16)
    if kv_dtype == "fp8_e4m3":
        kf = k_new.float().numpy()
        vf = v_new.float().numpy()
    for b in range(len(q_start)):
        for tok in range(int(cu_seqlens[b]), int(cu_seqlens[b + 1])):
            p = int(q_start[b]) + tok - int(cu_seqlens[b])
            if p < 0 or p // page_size >= max_pages:
                continue
            page = int(page_table[b, p // page_size])
            if page < 0 or page >= kp.shape[0]:
                continue
            s = p % page_size
            if kv_dtype == "bf16":
                kp[page, :, s, :] = kn[tok]
                vp[page, :, s, :] = vn[tok]
            else:
                kp[page, :, s, :] = e4m3_encode(kf[tok], k_scale)
                vp[page, :, s, :] = e4m3_encode(vf[tok], v_scale)
    return kp, vp
