"""CPU oracle for paged hd512 causal GQA attention -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the bench's CPU-baseline leg may import
this package.  The library under test never imports it, and the two share no
code: the C source here (oracle_attn.c) is the plain fp32 definition, and
brute.py is an independent float64 brute force for tiny inputs.

Parity status: every function here is pinned by the CPU test suite
(tests/test_oracle_pins.py, tests/test_oracle_sinks_lse.py,
tests/test_oracle_window.py) against brute
force, closed forms, a library routine special case (torch's CPU
scaled_dot_product_attention with an explicit mask) and torch's
float8_e4m3fn decoding; the log-sum-exp and sink outputs against the float64
brute force, the equal-scores and single-key closed forms and the split-K
merge identity; the sliding window and the ring cache against the float64
brute force (which de-pages through the ring independently), the window-1
identity o = V[pos], the q = 0 mean over the band, a window covering every
key equal to no window, and a wrapped ring equal to the unbounded layout.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence, Tuple

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle_attn.c")
_LIB_PATH = os.path.join(_HERE, "liboracle_attn.so")
_lib = None

KV_FORMATS = {"bf16": 0, "fp8_e4m3": 1}


def build(force: bool = True) -> str:
    """Compile oracle_attn.c with gcc (OpenMP, -O2, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                               "-Wall", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        L = ctypes.CDLL(_LIB_PATH)
        P, I, I64, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float
        common = [P, I64, P, P, I, F, F, P, I, I, P, P, P, I, I, I, I, I, F]
        L.oracle_attn_rows.argtypes = common + [P, I64, P, I]
        L.oracle_attn_rows.restype = I
        L.oracle_attn_rows_ex.argtypes = common + [P, P, I64, P, P, I]
        L.oracle_attn_rows_ex.restype = I
        L.oracle_attn_rows_full.argtypes = common + [I, I, P, P, I64, P, P, I]
        L.oracle_attn_rows_full.restype = I
        L.oracle_merge_ex.argtypes = [P, P, P, I, I, F, P, P]
        L.oracle_merge_ex.restype = None
        L.oracle_attn_partial.argtypes = common + [I64, I, I, I, P, P, P]
        L.oracle_attn_partial.restype = I
        L.oracle_merge.argtypes = [P, P, P, I, I, P]
        L.oracle_merge.restype = None
        L.oracle_e4m3_to_f32.argtypes = [P, P, I64]
        L.oracle_bf16_to_f32.argtypes = [P, P, I64]
        _lib = L
    return _lib


def default_threads() -> int:
    """OpenMP threads of an oracle call: the CPUs this process may run on,
    at most 16 (a one-GPU share of the host; the row results do not depend
    on the count)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _cpu(t: torch.Tensor) -> torch.Tensor:
    assert t.device.type == "cpu", "oracle inputs must be host tensors"
    return t.contiguous()


def _common_args(case, launch_idx: int, keep):
    lc = case.launches[launch_idx]
    q = _cpu(lc.q).view(torch.int16)
    kp, vp = _cpu(case.k_pool), _cpu(case.v_pool)
    table = _cpu(case.page_table).to(torch.int32)
    cu = _cpu(lc.cu_seqlens_q).to(torch.int32)
    qs = _cpu(lc.q_start).to(torch.int32)
    kl = _cpu(lc.kv_len).to(torch.int32)
    keep.extend([q, kp, vp, table, cu, qs, kl])
    D = int(q.shape[-1])
    page_size = int(kp.shape[2])
    return [q.data_ptr(), int(q.shape[0]), kp.data_ptr(), vp.data_ptr(),
            KV_FORMATS[case.kv_dtype], float(case.k_scale), float(case.v_scale),
            table.data_ptr(), int(table.shape[1]), int(kp.shape[0]), cu.data_ptr(),
            qs.data_ptr(), kl.data_ptr(), lc.batch, case.num_q_heads, case.num_kv_heads, D,
            page_size, float(case.softmax_scale)]


def _window_args(case):
    """(window, ring slots) of a case: 0 for none / an unbounded cache."""
    ring = int(getattr(case, "ring_pages", 0) or 0)
    return int(getattr(case, "window", 0) or 0), ring * int(case.k_pool.shape[2])


def attend_rows(case, rows: Sequence[int], launch_idx: int = 0,
                threads: Optional[int] = None) -> np.ndarray:
    """Outputs of the given entries (q_row * Hq + head) as float32 [n, D]."""
    keep = []
    args = _common_args(case, launch_idx, keep)
    D = args[16]
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    out = np.zeros((len(r), D), dtype=np.float32)
    nthreads = threads if threads is not None else default_threads()
    window, ring_slots = _window_args(case)
    if window or ring_slots:
        rc = lib().oracle_attn_rows_full(*args, window, ring_slots, None, r.ctypes.data,
                                         len(r), out.ctypes.data, None, int(nthreads))
    else:
        rc = lib().oracle_attn_rows(*args, r.ctypes.data, len(r), out.ctypes.data,
                                    int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle_attn_rows failed with code {rc}")
    return out


def attend_rows_lse(case, rows: Sequence[int], launch_idx: int = 0,
                    sinks: Optional[Sequence[float]] = None,
                    threads: Optional[int] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Outputs [n, D] and log-sum-exps [n] (natural log) of the given entries
    (q_row * Hq + head), with optional per-query-head sink logits."""
    keep = []
    args = _common_args(case, launch_idx, keep)
    D = args[16]
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    out = np.zeros((len(r), D), dtype=np.float32)
    lse = np.zeros(len(r), dtype=np.float32)
    snk = None
    if sinks is not None:
        snk = np.ascontiguousarray(np.asarray(sinks, dtype=np.float32))
        assert snk.shape == (case.num_q_heads,)
    nthreads = threads if threads is not None else default_threads()
    window, ring_slots = _window_args(case)
    rc = lib().oracle_attn_rows_full(*args, window, ring_slots,
                                     snk.ctypes.data if snk is not None else None,
                                     r.ctypes.data, len(r), out.ctypes.data, lse.ctypes.data,
                                     int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle_attn_rows_ex failed with code {rc}")
    return out, lse


def attend_all_lse(case, launch_idx: int = 0, sinks=None,
                   threads: Optional[int] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Every output [total_q, Hq, D] and log-sum-exp [total_q, Hq] of one launch."""
    lc = case.launches[launch_idx]
    n = lc.total_q * case.num_q_heads
    out, lse = attend_rows_lse(case, range(n), launch_idx, sinks, threads)
    return out.reshape(lc.total_q, case.num_q_heads, -1), lse.reshape(lc.total_q, -1)


def attend_all(case, launch_idx: int = 0, threads: Optional[int] = None) -> np.ndarray:
    """Every output of one launch as float32 [total_q, Hq, D]."""
    lc = case.launches[launch_idx]
    n = lc.total_q * case.num_q_heads
    out = attend_rows(case, range(n), launch_idx, threads)
    return out.reshape(lc.total_q, case.num_q_heads, -1)


def partial(case, q_row: int, head: int, k0: int, k1: int,
            launch_idx: int = 0) -> Tuple[np.ndarray, float, float]:
    """Unnormalised (O, m, l) of one row over keys [k0, k1); m in natural-log units
    (unbounded cache, no window)."""
    if any(_window_args(case)):
        raise ValueError("partial() covers the unbounded cache without a window only")
    keep = []
    args = _common_args(case, launch_idx, keep)
    D = args[16]
    O = np.zeros(D, dtype=np.float32)
    m = ctypes.c_float()
    l = ctypes.c_float()
    rc = lib().oracle_attn_partial(*args, int(q_row), int(head), int(k0), int(k1),
                                   O.ctypes.data, ctypes.addressof(m), ctypes.addressof(l))
    if rc != 0:
        raise ValueError(f"oracle_attn_partial failed with code {rc}")
    return O, m.value, l.value


def merge(O: np.ndarray, m: np.ndarray, l: np.ndarray) -> np.ndarray:
    """Combine partials O [n, D], m [n], l [n] into one normalised row."""
    O = np.ascontiguousarray(O, dtype=np.float32)
    m = np.ascontiguousarray(m, dtype=np.float32)
    l = np.ascontiguousarray(l, dtype=np.float32)
    out = np.zeros(O.shape[1], dtype=np.float32)
    lib().oracle_merge(O.ctypes.data, m.ctypes.data, l.ctypes.data, int(O.shape[0]),
                       int(O.shape[1]), out.ctypes.data)
    return out


def merge_lse(O: np.ndarray, m: np.ndarray, l: np.ndarray,
              sink: Optional[float] = None) -> Tuple[np.ndarray, float]:
    """merge() with an optional sink logit; also returns the log-sum-exp."""
    O = np.ascontiguousarray(O, dtype=np.float32)
    m = np.ascontiguousarray(m, dtype=np.float32)
    l = np.ascontiguousarray(l, dtype=np.float32)
    out = np.zeros(O.shape[1], dtype=np.float32)
    lse = ctypes.c_float()
    lib().oracle_merge_ex(O.ctypes.data, m.ctypes.data, l.ctypes.data, int(O.shape[0]),
                          int(O.shape[1]), float("nan") if sink is None else float(sink),
                          out.ctypes.data, ctypes.addressof(lse))
    return out, lse.value


def e4m3_to_f32(codes: np.ndarray) -> np.ndarray:
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.zeros(c.shape, dtype=np.float32)
    lib().oracle_e4m3_to_f32(c.ctypes.data, out.ctypes.data, c.size)
    return out


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.zeros(b.shape, dtype=np.float32)
    lib().oracle_bf16_to_f32(b.ctypes.data, out.ctypes.data, b.size)
    return out
