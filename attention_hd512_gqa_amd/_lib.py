"""ctypes binding of libattn_hd512.so: argument marshalling only.

Every step of the attention runs in the library's HIP kernels; this module
checks tensor dtypes, devices and contiguity, then passes raw device
pointers, sizes and the current HIP stream.  Torch only owns the memory.
If the library is not built, every call raises: there is no fallback.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libattn_hd512.so")
# the same kernels with wave-dependent sleeps around every LDS hand-off
DELAY_LIB_PATH = os.path.join(_HERE, "libattn_hd512_delay.so")

ATTN_BF16, ATTN_FP32, ATTN_FP8_E4M3 = 0, 1, 2
_DTYPE_CODES = {torch.bfloat16: ATTN_BF16, torch.float32: ATTN_FP32}
_KV_CODES = {"bf16": ATTN_BF16, "fp8_e4m3": ATTN_FP8_E4M3}

_lib = None
_delay_lib = None


class AttnError(RuntimeError):
    pass


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        _lib = _load(LIB_PATH)
    return _lib


@contextlib.contextmanager
def delay_injected():
    """Within the block every call of this module runs on the delay-injected
    build (libattn_hd512_delay.so), whose kernels sleep for wave-dependent
    times after every LDS refill load and before every workgroup barrier;
    the race tests check that it reproduces the normal build's results."""
    global _lib, _delay_lib
    if _delay_lib is None:
        _delay_lib = _load(DELAY_LIB_PATH)
    saved = lib()
    _lib = _delay_lib
    try:
        yield
    finally:
        _lib = saved


def _load(path: str) -> ctypes.CDLL:
    """Opens one build of the library and declares every entry point."""
    if not os.path.exists(path):
        raise AttnError(f"{path} is missing: build it with "
                        "`python -m attention_hd512_gqa_amd.build`")
    L = ctypes.CDLL(path)
    P, I, F, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    L.attn_prefill_hd512.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, I, F, P, I, P]
    L.attn_prefill_hd512.restype = I
    L.attn_prefill_hd512_e4m3.argtypes = [P, P, P, F, F, P, P, P, P, I, I, I, I, I, I, I, I,
                                          I, F, P, I, P]
    L.attn_prefill_hd512_e4m3.restype = I
    L.attn_prefill_hd512_ex.argtypes = [P, P, P, I, F, F, P, P, P, P, I, I, I, I, I, I, I,
                                        I, I, F, P, P, I, P, P]
    L.attn_prefill_hd512_ex.restype = I
    L.attn_prefill_hd512_e4m3_mma.argtypes = [P, P, P, F, F, P, P, P, P, I, I, I, I, I, I,
                                              I, I, I, F, P, P, I, P, P]
    L.attn_prefill_hd512_e4m3_mma.restype = I
    L.attn_prefill_hd512_append.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, I, I,
                                            I, I, I, F, P, P, I, P, P]
    L.attn_prefill_hd512_append.restype = I
    L.attn_prefill_hd512_e4m3_mma_append.argtypes = [P, P, P, P, P, F, F, P, P, P, P, I, I, I,
                                                     I, I, I, I, I, I, F, P, P, I, P, P]
    L.attn_prefill_hd512_e4m3_mma_append.restype = I
    L.attn_prefill_hd512_persistent_workspace_size.argtypes = []
    L.attn_prefill_hd512_persistent_workspace_size.restype = SZ
    L.attn_prefill_hd512_persistent.argtypes = [P, P, P, I, F, F, P, P, P, P, I, I, I, I, I,
                                                I, I, I, I, F, P, P, SZ, P, I, P, P]
    L.attn_prefill_hd512_persistent.restype = I
    L.attn_prefill_swa.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, I, I, I, F,
                                   P, I, P]
    L.attn_prefill_swa.restype = I
    L.attn_prefill_hd512_splitk_workspace_size.argtypes = [I, I, I, I, I, I, I]
    L.attn_prefill_hd512_splitk_workspace_size.restype = SZ
    L.attn_prefill_hd512_splitk.argtypes = [P, P, P, I, F, F, P, P, P, P, I, I, I, I, I, I,
                                            I, I, I, I, I, F, P, P, SZ, P, I, P, P]
    L.attn_prefill_hd512_splitk.restype = I
    L.attn_prefill_hd512_splitk_e4m3_mma.argtypes = [P, P, P, F, F, P, P, P, P, I, I, I, I,
                                                     I, I, I, I, I, I, I, F, P, P, SZ, P, I,
                                                     P, P]
    L.attn_prefill_hd512_splitk_e4m3_mma.restype = I
    L.attn_decode_splitk_ex_workspace_size.argtypes = [I, I, I, I, I, I]
    L.attn_decode_splitk_ex_workspace_size.restype = SZ
    L.attn_decode_splitk_ex.argtypes = [P, P, P, I, F, F, P, P, I, I, I, I, I, I, I, I, I, I,
                                        F, P, P, SZ, P, I, P, P]
    L.attn_decode_splitk_ex.restype = I
    L.attn_decode_splitk_ex_noalloc.argtypes = [P, P, P, I, F, F, P, P, I, I, I, I, I, I, I,
                                                I, I, I, F, P, P, I, P, P]
    L.attn_decode_splitk_ex_noalloc.restype = I
    L.attn_append_kv.argtypes = [P, P, I, F, F, P, P, P, I, I, I, I, I, I, I, P, P, P]
    L.attn_append_kv.restype = I
    L.attn_decode_splitk_workspace_size.argtypes = [I, I, I, I, I]
    L.attn_decode_splitk_workspace_size.restype = SZ
    L.attn_decode_splitk.argtypes = [P, P, P, I, F, F, P, P, I, I, I, I, I, I, I, I, I, F,
                                     P, SZ, P, I, P]
    L.attn_decode_splitk.restype = I
    L.attn_hbm_read_probe.argtypes = [P, SZ, P, P]
    L.attn_hbm_read_probe.restype = I
    L.attn_hbm_probe_sink_words.argtypes = [SZ]
    L.attn_hbm_probe_sink_words.restype = SZ
    L.attn_clock_stamps.argtypes = [P, I, P]
    L.attn_clock_stamps.restype = I
    L.attn_status_string.argtypes = [I]
    L.attn_status_string.restype = ctypes.c_char_p
    return L


def status_string(code: int) -> str:
    return lib().attn_status_string(int(code)).decode()


def _check(code: int, what: str):
    if code != 0:
        raise AttnError(f"{what}: {status_string(code)} (status {code})")


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _dev(t: torch.Tensor, name: str, dtype=None) -> int:
    if not t.is_cuda:
        raise AttnError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise AttnError(f"{name} must be contiguous")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise AttnError(f"{name} has dtype {t.dtype}, expected {dtype}")
    return t.data_ptr()


def _opt(t, name, dtype, numel):
    if t is None:
        return None
    if t.numel() != numel:
        raise AttnError(f"{name} must have {numel} elements, has {t.numel()}")
    return _dev(t, name, dtype)


def prefill(q, k_pages, v_pages, page_table, cu_seqlens_q, q_start, kv_lens, out, *,
            total_q: int, max_q_len: int, softmax_scale: float, kv_dtype: str = "bf16",
            k_scale: float = 1.0, v_scale: float = 1.0, sinks=None, lse=None,
            fp8_mma: bool = False, stream=None) -> None:
    """Chunked causal prefill over a bf16 pool (attn_prefill_hd512) or an
    FP8-E4M3 pool with per-tensor scales (attn_prefill_hd512_e4m3); with
    per-head sink logits `sinks` (fp32 [Hq]) or a log-sum-exp output `lse`
    (fp32 [total_q, Hq]) it calls attn_prefill_hd512_ex.  fp8_mma (FP8 pool
    only) runs both products on the block-scaled FP8 matrix core instead
    (attn_prefill_hd512_e4m3_mma).  Sizes are host ints: no sync."""
    num_pages, hkv, page, d = k_pages.shape
    hq = q.shape[1]
    batch = kv_lens.shape[0]
    meta = (_dev(page_table, "page_table", torch.int32),
            _dev(cu_seqlens_q, "cu_seqlens_q", torch.int32), _dev(q_start, "q_start", torch.int32),
            _dev(kv_lens, "kv_lens", torch.int32), int(batch), int(total_q), int(max_q_len),
            int(hq), int(hkv), int(d), int(page), int(num_pages), int(page_table.shape[1]),
            float(softmax_scale), _dev(out, "out", (torch.bfloat16, torch.float32)),
            _DTYPE_CODES[out.dtype], _stream(stream))
    if kv_dtype not in _KV_CODES:
        raise AttnError(f"unsupported kv_dtype {kv_dtype!r}")
    kvt = torch.bfloat16 if kv_dtype == "bf16" else torch.uint8
    if fp8_mma:
        if kv_dtype != "fp8_e4m3":
            raise AttnError("fp8_mma needs kv_dtype 'fp8_e4m3'")
        code = lib().attn_prefill_hd512_e4m3_mma(
            _dev(q, "q", torch.bfloat16), _dev(k_pages, "k_pages", kvt),
            _dev(v_pages, "v_pages", kvt), float(k_scale), float(v_scale), *meta[:14],
            _opt(sinks, "sinks", torch.float32, hq), meta[14], meta[15],
            _opt(lse, "lse", torch.float32, int(total_q) * hq), meta[16])
        _check(code, "attn_prefill_hd512_e4m3_mma")
    elif sinks is not None or lse is not None:
        code = lib().attn_prefill_hd512_ex(
            _dev(q, "q", torch.bfloat16), _dev(k_pages, "k_pages", kvt),
            _dev(v_pages, "v_pages", kvt), _KV_CODES[kv_dtype], float(k_scale), float(v_scale),
            *meta[:14], _opt(sinks, "sinks", torch.float32, hq), meta[14], meta[15],
            _opt(lse, "lse", torch.float32, int(total_q) * hq), meta[16])
        _check(code, "attn_prefill_hd512_ex")
    elif kv_dtype == "bf16":
        code = lib().attn_prefill_hd512(
            _dev(q, "q", torch.bfloat16), _dev(k_pages, "k_pages", torch.bfloat16),
            _dev(v_pages, "v_pages", torch.bfloat16), *meta)
        _check(code, "attn_prefill_hd512")
    elif kv_dtype == "fp8_e4m3":
        code = lib().attn_prefill_hd512_e4m3(
            _dev(q, "q", torch.bfloat16), _dev(k_pages, "k_pages", torch.uint8),
            _dev(v_pages, "v_pages", torch.uint8), float(k_scale), float(v_scale), *meta)
        _check(code, "attn_prefill_hd512_e4m3")


def prefill_append(q, k_new, v_new, k_pages, v_pages, page_table, cu_seqlens_q, q_start,
                   kv_lens, out, *, total_q: int, max_q_len: int, softmax_scale: float,
                   kv_dtype: str = "bf16", k_scale: float = 1.0, v_scale: float = 1.0,
                   sinks=None, lse=None, stream=None) -> None:
    """Chunked causal prefill with the chunk's KV append: the bf16 rows
    k_new, v_new [total_q, Hkv, 512] are written into their page slots and
    the chunk attends to them, giving the same result as append_kv followed
    by prefill.  bf16 pool: one fused launch (attn_prefill_hd512_append).
    E4M3 pool (kv_dtype "fp8_e4m3"): the rows are encoded with k_scale and
    v_scale and the prefill runs on the FP8 matrix core
    (attn_prefill_hd512_e4m3_mma_append: the append kernel, then the
    FP8-MMA prefill, on one stream)."""
    num_pages, hkv, page, d = k_pages.shape
    hq = q.shape[1]
    batch = kv_lens.shape[0]
    if kv_dtype not in _KV_CODES:
        raise AttnError(f"unsupported kv_dtype {kv_dtype!r}")
    fp8 = kv_dtype == "fp8_e4m3"
    kvt = torch.uint8 if fp8 else torch.bfloat16
    head = (_dev(q, "q", torch.bfloat16), _dev(k_new, "k_new", torch.bfloat16),
            _dev(v_new, "v_new", torch.bfloat16), _dev(k_pages, "k_pages", kvt),
            _dev(v_pages, "v_pages", kvt))
    rest = (_dev(page_table, "page_table", torch.int32),
            _dev(cu_seqlens_q, "cu_seqlens_q", torch.int32), _dev(q_start, "q_start", torch.int32),
            _dev(kv_lens, "kv_lens", torch.int32), int(batch), int(total_q), int(max_q_len),
            int(hq), int(hkv), int(d), int(page), int(num_pages), int(page_table.shape[1]),
            float(softmax_scale), _opt(sinks, "sinks", torch.float32, hq),
            _dev(out, "out", (torch.bfloat16, torch.float32)), _DTYPE_CODES[out.dtype],
            _opt(lse, "lse", torch.float32, int(total_q) * hq), _stream(stream))
    if fp8:
        code = lib().attn_prefill_hd512_e4m3_mma_append(*head, float(k_scale), float(v_scale),
                                                          *rest)
        _check(code, "attn_prefill_hd512_e4m3_mma_append")
    else:
        code = lib().attn_prefill_hd512_append(*head, *rest)
        _check(code, "attn_prefill_hd512_append")


def prefill_persistent_workspace_size() -> int:
    return int(lib().attn_prefill_hd512_persistent_workspace_size())


def prefill_persistent(q, k_pages, v_pages, page_table, cu_seqlens_q, q_start, kv_lens, out,
                       workspace, *, total_q: int, max_q_len: int, softmax_scale: float,
                       kv_dtype: str = "bf16", k_scale: float = 1.0, v_scale: float = 1.0,
                       sinks=None, lse=None, stream=None) -> None:
    """prefill() with persistent heaviest-first scheduling
    (attn_prefill_hd512_persistent): one workgroup per compute unit taking
    work units from a counter in `workspace` (a device tensor of at least
    prefill_persistent_workspace_size() bytes).  Bitwise the same results."""
    num_pages, hkv, page, d = k_pages.shape
    hq = q.shape[1]
    batch = kv_lens.shape[0]
    if kv_dtype not in _KV_CODES:
        raise AttnError(f"unsupported kv_dtype {kv_dtype!r}")
    kvt = torch.bfloat16 if kv_dtype == "bf16" else torch.uint8
    code = lib().attn_prefill_hd512_persistent(
        _dev(q, "q", torch.bfloat16), _dev(k_pages, "k_pages", kvt),
        _dev(v_pages, "v_pages", kvt), _KV_CODES[kv_dtype], float(k_scale), float(v_scale),
        _dev(page_table, "page_table", torch.int32),
        _dev(cu_seqlens_q, "cu_seqlens_q", torch.int32), _dev(q_start, "q_start", torch.int32),
        _dev(kv_lens, "kv_lens", torch.int32), int(batch), int(total_q), int(max_q_len),
        int(hq), int(hkv), int(d), int(page), int(num_pages), int(page_table.shape[1]),
        float(softmax_scale), _opt(sinks, "sinks", torch.float32, hq), _dev(workspace, "workspace"),
        workspace.numel() * workspace.element_size(),
        _dev(out, "out", (torch.bfloat16, torch.float32)), _DTYPE_CODES[out.dtype],
        _opt(lse, "lse", torch.float32, int(total_q) * hq), _stream(stream))
    _check(code, "attn_prefill_hd512_persistent")


def prefill_swa(q, k_pages, v_pages, page_table, cu_seqlens_q, q_start, kv_lens, out, *,
                total_q: int, max_q_len: int, softmax_scale: float, window: int,
                ring_pages: int = 0, stream=None) -> None:
    """Chunked causal prefill of a sliding-window layer (attn_prefill_swa): a
    row at position p sees keys max(0, p - window + 1) .. p (window 0: no
    window), over a bf16 pool of head dim 256 or 512, optionally a ring cache
    of ring_pages pages per sequence (key j at slot j % (64 ring_pages))."""
    num_pages, hkv, page, d = k_pages.shape
    hq = q.shape[1]
    batch = kv_lens.shape[0]
    code = lib().attn_prefill_swa(
        _dev(q, "q", torch.bfloat16), _dev(k_pages, "k_pages", torch.bfloat16),
        _dev(v_pages, "v_pages", torch.bfloat16), _dev(page_table, "page_table", torch.int32),
        _dev(cu_seqlens_q, "cu_seqlens_q", torch.int32), _dev(q_start, "q_start", torch.int32),
        _dev(kv_lens, "kv_lens", torch.int32), int(batch), int(total_q), int(max_q_len),
        int(hq), int(hkv), int(d), int(page), int(num_pages), int(page_table.shape[1]),
        int(window), int(ring_pages), float(softmax_scale),
        _dev(out, "out", (torch.bfloat16, torch.float32)), _DTYPE_CODES[out.dtype],
        _stream(stream))
    _check(code, "attn_prefill_swa")


def prefill_splitk_workspace_size(batch: int, max_q_len: int, total_q: int, num_q_heads: int,
                                  num_kv_heads: int, max_kv_len: int,
                                  keys_per_split: int = 0) -> int:
    """Bytes of workspace attn_prefill_hd512_splitk needs (0: a single pass)."""
    return int(lib().attn_prefill_hd512_splitk_workspace_size(
        int(batch), int(max_q_len), int(total_q), int(num_q_heads), int(num_kv_heads),
        int(max_kv_len), int(keys_per_split)))


def prefill_splitk(q, k_pages, v_pages, page_table, cu_seqlens_q, q_start, kv_lens, out,
                   workspace, *, total_q: int, max_q_len: int, max_kv_len: int,
                   softmax_scale: float, keys_per_split: int = 0, kv_dtype: str = "bf16",
                   k_scale: float = 1.0, v_scale: float = 1.0, sinks=None, lse=None,
                   fp8_mma: bool = False, stream=None) -> None:
    """Chunked causal prefill with the key range split across workgroups
    (attn_prefill_hd512_splitk): split kernel then merge kernel, for short
    chunks over long prefixes.  fp8_mma (FP8 pool only) runs each range on
    the block-scaled FP8 matrix core (attn_prefill_hd512_splitk_e4m3_mma).
    `workspace` may be None when prefill_splitk_workspace_size(...) is 0."""
    num_pages, hkv, page, d = k_pages.shape
    hq = q.shape[1]
    batch = kv_lens.shape[0]
    if kv_dtype not in _KV_CODES:
        raise AttnError(f"unsupported kv_dtype {kv_dtype!r}")
    kvt = torch.bfloat16 if kv_dtype == "bf16" else torch.uint8
    if workspace is None:
        ws, ws_bytes = None, 0
    else:
        ws, ws_bytes = _dev(workspace, "workspace"), workspace.numel() * workspace.element_size()
    if fp8_mma and kv_dtype != "fp8_e4m3":
        raise AttnError("fp8_mma needs kv_dtype 'fp8_e4m3'")
    fn = lib().attn_prefill_hd512_splitk_e4m3_mma if fp8_mma else lib().attn_prefill_hd512_splitk
    head = (_dev(q, "q", torch.bfloat16), _dev(k_pages, "k_pages", kvt),
            _dev(v_pages, "v_pages", kvt)) + (() if fp8_mma else (_KV_CODES[kv_dtype],))
    code = fn(
        *head, float(k_scale), float(v_scale),
        _dev(page_table, "page_table", torch.int32),
        _dev(cu_seqlens_q, "cu_seqlens_q", torch.int32), _dev(q_start, "q_start", torch.int32),
        _dev(kv_lens, "kv_lens", torch.int32), int(batch), int(total_q), int(max_q_len),
        int(hq), int(hkv), int(d), int(page), int(num_pages), int(page_table.shape[1]),
        int(max_kv_len), int(keys_per_split), float(softmax_scale),
        _opt(sinks, "sinks", torch.float32, hq), ws, ws_bytes,
        _dev(out, "out", (torch.bfloat16, torch.float32)), _DTYPE_CODES[out.dtype],
        _opt(lse, "lse", torch.float32, int(total_q) * hq), _stream(stream))
    _check(code, "attn_prefill_hd512_splitk_e4m3_mma" if fp8_mma else "attn_prefill_hd512_splitk")


def decode_workspace_size(batch: int, num_q_heads: int, num_kv_heads: int, max_kv_len: int,
                          keys_per_split: int = 0, q_len: int = 1) -> int:
    return int(lib().attn_decode_splitk_ex_workspace_size(
        int(batch), int(q_len), int(num_q_heads), int(num_kv_heads), int(max_kv_len),
        int(keys_per_split)))


def decode(q, k_pages, v_pages, page_table, kv_lens, out, workspace, *, max_kv_len: int,
           softmax_scale: float, kv_dtype: str = "bf16", k_scale: float = 1.0,
           v_scale: float = 1.0, keys_per_split: int = 0, q_len: int = 1, sinks=None,
           lse=None, stream=None) -> None:
    """Split-K decode (split kernel then merge kernel).  q holds q_len tokens per
    sequence, [batch * q_len, Hq, 512], at positions kv_len - q_len ..; with
    q_len > 1, sinks (fp32 [Hq]) or lse (fp32 [batch * q_len, Hq]) it calls
    attn_decode_splitk_ex, else attn_decode_splitk."""
    num_pages, hkv, page, d = k_pages.shape
    hq = q.shape[1]
    batch = kv_lens.shape[0]
    if q.shape[0] != batch * q_len:
        raise AttnError(f"q has {q.shape[0]} rows, expected batch * q_len = {batch * q_len}")
    kvt = torch.bfloat16 if kv_dtype == "bf16" else torch.uint8
    head = (_dev(q, "q", torch.bfloat16), _dev(k_pages, "k_pages", kvt),
            _dev(v_pages, "v_pages", kvt), _KV_CODES[kv_dtype], float(k_scale), float(v_scale),
            _dev(page_table, "page_table", torch.int32), _dev(kv_lens, "kv_lens", torch.int32))
    ws = (_dev(workspace, "workspace"), workspace.numel() * workspace.element_size(),
          _dev(out, "out", (torch.bfloat16, torch.float32)), _DTYPE_CODES[out.dtype])
    if q_len != 1 or sinks is not None or lse is not None:
        code = lib().attn_decode_splitk_ex(
            *head, int(batch), int(q_len), int(hq), int(hkv), int(d), int(page), int(num_pages),
            int(page_table.shape[1]), int(max_kv_len), int(keys_per_split), float(softmax_scale),
            _opt(sinks, "sinks", torch.float32, hq), *ws,
            _opt(lse, "lse", torch.float32, int(batch) * int(q_len) * hq), _stream(stream))
        _check(code, "attn_decode_splitk_ex")
    else:
        code = lib().attn_decode_splitk(
            *head, int(batch), int(hq), int(hkv), int(d), int(page), int(num_pages),
            int(page_table.shape[1]), int(max_kv_len), int(keys_per_split), float(softmax_scale),
            *ws, _stream(stream))
        _check(code, "attn_decode_splitk")


def decode_noalloc(q, k_pages, v_pages, page_table, kv_lens, out, *, max_kv_len: int,
                   softmax_scale: float, kv_dtype: str = "bf16", k_scale: float = 1.0,
                   v_scale: float = 1.0, keys_per_split: int = 0, q_len: int = 1, sinks=None,
                   lse=None, stream=None) -> None:
    """decode() without a workspace argument (attn_decode_splitk_ex_noalloc):
    the partials go to the library's static device scratch (64 MiB), so the
    call allocates nothing.  Calls that overlap on one GPU share that scratch
    and race."""
    num_pages, hkv, page, d = k_pages.shape
    hq = q.shape[1]
    batch = kv_lens.shape[0]
    if q.shape[0] != batch * q_len:
        raise AttnError(f"q has {q.shape[0]} rows, expected batch * q_len = {batch * q_len}")
    kvt = torch.bfloat16 if kv_dtype == "bf16" else torch.uint8
    code = lib().attn_decode_splitk_ex_noalloc(
        _dev(q, "q", torch.bfloat16), _dev(k_pages, "k_pages", kvt),
        _dev(v_pages, "v_pages", kvt), _KV_CODES[kv_dtype], float(k_scale), float(v_scale),
        _dev(page_table, "page_table", torch.int32), _dev(kv_lens, "kv_lens", torch.int32),
        int(batch), int(q_len), int(hq), int(hkv), int(d), int(page), int(num_pages),
        int(page_table.shape[1]), int(max_kv_len), int(keys_per_split), float(softmax_scale),
        _opt(sinks, "sinks", torch.float32, hq),
        _dev(out, "out", (torch.bfloat16, torch.float32)), _DTYPE_CODES[out.dtype],
        _opt(lse, "lse", torch.float32, int(batch) * int(q_len) * hq), _stream(stream))
    _check(code, "attn_decode_splitk_ex_noalloc")


def append_kv(k_new, v_new, page_table, cu_seqlens, q_start, k_pages, v_pages, *,
              kv_dtype: str = "bf16", k_scale: float = 1.0, v_scale: float = 1.0,
              stream=None) -> None:
    """Paged KV append (attn_append_kv): writes the bf16 rows k_new, v_new
    [total_q, Hkv, 512] into their page slots, as bf16 or as E4M3 codes
    (x / scale, saturated, round to nearest even)."""
    num_pages, hkv, page, d = k_pages.shape
    batch = q_start.shape[0]
    kvt = torch.bfloat16 if kv_dtype == "bf16" else torch.uint8
    code = lib().attn_append_kv(
        _dev(k_new, "k_new", torch.bfloat16), _dev(v_new, "v_new", torch.bfloat16),
        _KV_CODES[kv_dtype], float(k_scale), float(v_scale),
        _dev(page_table, "page_table", torch.int32), _dev(cu_seqlens, "cu_seqlens", torch.int32),
        _dev(q_start, "q_start", torch.int32), int(batch), int(k_new.shape[0]), int(hkv), int(d),
        int(page), int(num_pages), int(page_table.shape[1]), _dev(k_pages, "k_pages", kvt),
        _dev(v_pages, "v_pages", kvt), _stream(stream))
    _check(code, "attn_append_kv")


def hbm_read_probe(buf: torch.Tensor, sink: torch.Tensor, stream=None) -> None:
    """Stream `buf` once (measurement helper for the HBM read roofline)."""
    nbytes = buf.numel() * buf.element_size()
    code = lib().attn_hbm_read_probe(_dev(buf, "buf"), nbytes, _dev(sink, "sink"), _stream(stream))
    _check(code, "attn_hbm_read_probe")


def hbm_probe_sink_words(nbytes: int) -> int:
    return int(lib().attn_hbm_probe_sink_words(int(nbytes)))


def clock_stamps(stamps: torch.Tensor, stream=None) -> None:
    """Enqueue one clock-stamp workgroup per row of `stamps` (int64 [n, 3]):
    XCD id, shader-clock cycle counter, 100 MHz counter (measurement helper)."""
    if stamps.dtype != torch.int64 or stamps.dim() != 2 or stamps.shape[1] != 3:
        raise AttnError("stamps must be an int64 tensor of shape [n, 3]")
    code = lib().attn_clock_stamps(_dev(stamps, "stamps"), int(stamps.shape[0]), _stream(stream))
    _check(code, "attn_clock_stamps")
