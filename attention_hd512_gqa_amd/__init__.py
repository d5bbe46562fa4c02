"""MI355X-native head-dim-512 paged causal GQA attention: Python binding.

The kernels and the C ABI live in libattn_hd512.so (include/attn_hd512.h);
this package only marshals torch tensors into that ABI.
"""
from ._lib import (ATTN_BF16, ATTN_FP32, ATTN_FP8_E4M3, AttnError, LIB_PATH, append_kv,
                   clock_stamps, decode, decode_noalloc, decode_workspace_size,
                   hbm_probe_sink_words, hbm_read_probe, lib, prefill, prefill_append,
                   prefill_persistent, prefill_persistent_workspace_size, prefill_splitk,
                   prefill_splitk_workspace_size, prefill_swa, status_string)

__all__ = ["ATTN_BF16", "ATTN_FP32", "ATTN_FP8_E4M3", "AttnError", "LIB_PATH", "append_kv",
           "clock_stamps", "decode", "decode_noalloc", "decode_workspace_size",
           "hbm_probe_sink_words", "hbm_read_probe", "lib", "prefill", "prefill_append",
           "prefill_persistent", "prefill_persistent_workspace_size", "prefill_splitk",
           "prefill_splitk_workspace_size", "prefill_swa", "status_string"]
