"""C ABI checks that need no GPU: exported symbols and host-side validation.

Every call below carries at least one argument that the host checks reject,
so no kernel is ever launched (the pointers are never dereferenced).
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn_hd512.h")


@pytest.fixture(scope="module")
def L():
    import attention_hd512_gqa_amd as A
    if not os.path.exists(A.LIB_PATH):
        from attention_hd512_gqa_amd import build
        build.build()
    return A.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("attn_prefill_hd512", "attn_prefill_hd512_e4m3", "attn_decode_splitk",
              "attn_decode_splitk_workspace_size",
              "attn_status_string", "attn_hbm_read_probe", "attn_hbm_probe_sink_words"):
        assert n in names


def test_every_declared_symbol_is_exported(L):
    for n in declared_functions():
        assert hasattr(L, n), f"{n} is declared in the header but not exported"


def test_status_strings(L):
    for code in range(6):
        assert L.attn_status_string(code)
    assert L.attn_status_string(99) == b"unknown status"


FAKE = 0x1000  # never dereferenced: each call fails validation first


def prefill(L, **over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, pt=FAKE, cu=FAKE, qs=FAKE, kl=FAKE, batch=1, total_q=4,
             max_q_len=4, hq=8, hkv=1, d=512, page=64, num_pages=4, max_pages=4, scale=0.04,
             out=FAKE, out_dtype=1, stream=None)
    a.update(over)
    return L.attn_prefill_hd512(a["q"], a["k"], a["v"], a["pt"], a["cu"], a["qs"], a["kl"],
                                a["batch"], a["total_q"], a["max_q_len"], a["hq"], a["hkv"],
                                a["d"], a["page"], a["num_pages"], a["max_pages"], a["scale"],
                                a["out"], a["out_dtype"], a["stream"])


def test_prefill_validation(L):
    assert prefill(L, q=None) == 1
    assert prefill(L, out=None) == 1
    assert prefill(L, batch=0) == 2
    assert prefill(L, hq=6, hkv=4) == 2
    assert prefill(L, d=256) == 3
    assert prefill(L, page=16) == 3
    assert prefill(L, out_dtype=2) == 3
    assert prefill(L, hq=256, hkv=1) == 3
    assert prefill(L, scale=float("nan")) == 2
    assert prefill(L, max_q_len=5) == 2          # larger than total_q
    assert prefill(L, total_q=0, max_q_len=0) == 0  # empty call: nothing to launch


def prefill_e4m3(L, **over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, ks=0.01, vs=0.01, pt=FAKE, cu=FAKE, qs=FAKE, kl=FAKE,
             batch=1, total_q=4, max_q_len=4, hq=8, hkv=1, d=512, page=64, num_pages=4,
             max_pages=4, scale=0.04, out=FAKE, out_dtype=1, stream=None)
    a.update(over)
    return L.attn_prefill_hd512_e4m3(a["q"], a["k"], a["v"], a["ks"], a["vs"], a["pt"], a["cu"],
                                     a["qs"], a["kl"], a["batch"], a["total_q"], a["max_q_len"],
                                     a["hq"], a["hkv"], a["d"], a["page"], a["num_pages"],
                                     a["max_pages"], a["scale"], a["out"], a["out_dtype"],
                                     a["stream"])


def test_prefill_e4m3_validation(L):
    assert prefill_e4m3(L, v=None) == 1
    assert prefill_e4m3(L, ks=0.0) == 2
    assert prefill_e4m3(L, vs=-1.0) == 2
    assert prefill_e4m3(L, ks=float("nan")) == 2
    assert prefill_e4m3(L, batch=0) == 2
    assert prefill_e4m3(L, d=256) == 3
    assert prefill_e4m3(L, out_dtype=2) == 3
    assert prefill_e4m3(L, total_q=0, max_q_len=0) == 0


def decode(L, **over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, kvd=0, ks=1.0, vs=1.0, pt=FAKE, kl=FAKE, batch=2, hq=8,
             hkv=4, d=512, page=64, num_pages=8, max_pages=4, max_kv=256, kps=0, scale=0.04,
             ws=FAKE, ws_bytes=1 << 30, out=FAKE, out_dtype=0, stream=None)
    a.update(over)
    return L.attn_decode_splitk(a["q"], a["k"], a["v"], a["kvd"], a["ks"], a["vs"], a["pt"],
                                a["kl"], a["batch"], a["hq"], a["hkv"], a["d"], a["page"],
                                a["num_pages"], a["max_pages"], a["max_kv"], a["kps"],
                                a["scale"], a["ws"], a["ws_bytes"], a["out"], a["out_dtype"],
                                a["stream"])


def test_decode_validation(L):
    assert decode(L, v=None) == 1
    assert decode(L, kps=100) == 2                 # not a multiple of 64
    assert decode(L, max_kv=257) == 2              # beyond max_pages * 64
    assert decode(L, hq=6) == 2
    assert decode(L, d=128) == 3
    assert decode(L, hq=256, hkv=1) == 3           # group of 256 > 128 (routed, refused)
    assert decode(L, kvd=1) == 3                   # fp32 pool
    assert decode(L, out_dtype=2) == 3
    assert decode(L, kvd=2, ks=0.0) == 2           # FP8 needs positive scales
    assert decode(L, ws=None) == 4
    assert decode(L, ws_bytes=16) == 4


def decode_ex(L, **over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, kvd=0, ks=1.0, vs=1.0, pt=FAKE, kl=FAKE, batch=2, q_len=2,
             hq=8, hkv=4, d=512, page=64, num_pages=8, max_pages=4, max_kv=256, kps=0,
             scale=0.04, sinks=None, ws=FAKE, ws_bytes=1 << 30, out=FAKE, out_dtype=0,
             lse=None, stream=None)
    a.update(over)
    return L.attn_decode_splitk_ex(a["q"], a["k"], a["v"], a["kvd"], a["ks"], a["vs"], a["pt"],
                                   a["kl"], a["batch"], a["q_len"], a["hq"], a["hkv"], a["d"],
                                   a["page"], a["num_pages"], a["max_pages"], a["max_kv"],
                                   a["kps"], a["scale"], a["sinks"], a["ws"], a["ws_bytes"],
                                   a["out"], a["out_dtype"], a["lse"], a["stream"])


def test_decode_ex_validation(L):
    assert decode_ex(L, q=None) == 1
    assert decode_ex(L, q_len=0) == 2
    # 25 tokens x g = 2 = 50 columns > 48: the call becomes a split-K
    # prefill, whose checks (pool dtype, workspace) still run before any launch
    assert decode_ex(L, q_len=25, kvd=1) == 3
    assert decode_ex(L, q_len=25, ws_bytes=16) == 4
    assert decode_ex(L, q_len=25, ws=None) == 4
    # 9 tokens x g = 2 = 18 columns: two column blocks of the decode kernel
    assert decode_ex(L, q_len=9, kvd=1) == 3
    assert decode_ex(L, q_len=9, ws_bytes=16) == 4
    assert decode_ex(L, kvd=1) == 3
    assert decode_ex(L, ws_bytes=16) == 4


def test_prefill_ex_validation(L):
    def pf(**over):
        a = dict(kvd=0, ks=1.0, vs=1.0, batch=1, total_q=4, max_q_len=4, hq=8, hkv=1, d=512,
                 page=64, out_dtype=1)
        a.update(over)
        return L.attn_prefill_hd512_ex(FAKE, FAKE, FAKE, a["kvd"], a["ks"], a["vs"], FAKE, FAKE,
                                       FAKE, FAKE, a["batch"], a["total_q"], a["max_q_len"],
                                       a["hq"], a["hkv"], a["d"], a["page"], 4, 4, 0.04, None,
                                       FAKE, a["out_dtype"], None, None)
    assert pf(kvd=1) == 3
    assert pf(kvd=2, ks=0.0) == 2
    assert pf(d=128) == 3
    assert pf(total_q=0, max_q_len=0) == 0


def test_prefill_swa_validation(L):
    def sw(**over):
        a = dict(q=FAKE, batch=1, total_q=4, max_q_len=4, hq=8, hkv=1, d=256, page=64,
                 max_pages=4, window=16, ring=0, out_dtype=1)
        a.update(over)
        return L.attn_prefill_swa(a["q"], FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, a["batch"],
                                  a["total_q"], a["max_q_len"], a["hq"], a["hkv"], a["d"],
                                  a["page"], 4, a["max_pages"], a["window"], a["ring"], 0.06,
                                  FAKE, a["out_dtype"], None)
    assert sw(q=None) == 1
    assert sw(d=128) == 3
    assert sw(page=16) == 3
    assert sw(window=-1) == 2
    assert sw(ring=-1) == 2
    assert sw(ring=5) == 2                 # longer than the table
    assert sw(window=0, ring=2) == 2       # a ring needs a window
    assert sw(out_dtype=2) == 3
    assert sw(hq=6, hkv=4) == 2
    assert sw(total_q=0, max_q_len=0) == 0
    # head dim 256 and windows are refused by the head-dim-512 entry points
    assert prefill(L, d=256) == 3


def test_prefill_append_validation(L):
    def pa(**over):
        a = dict(kn=FAKE, vn=FAKE, batch=1, total_q=4, max_q_len=4, hq=8, hkv=1, d=512,
                 page=64, out_dtype=1)
        a.update(over)
        return L.attn_prefill_hd512_append(
            FAKE, a["kn"], a["vn"], FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, a["batch"],
            a["total_q"], a["max_q_len"], a["hq"], a["hkv"], a["d"], a["page"], 4, 4, 0.04,
            None, FAKE, a["out_dtype"], None, None)
    assert pa(kn=None) == 1
    assert pa(vn=None) == 1
    assert pa(d=256) == 3
    assert pa(page=16) == 3
    assert pa(hq=6, hkv=4) == 2
    assert pa(out_dtype=2) == 3
    # new-row buffers past 32-bit buffer offsets
    assert pa(total_q=1 << 22, max_q_len=4) == 2
    assert pa(total_q=0, max_q_len=0) == 0


def test_prefill_e4m3_mma_append_validation(L):
    # every check of the append and of the prefill runs before the first
    # launch; only rejected calls and the empty one are made here
    def pa(**over):
        a = dict(kn=FAKE, vn=FAKE, ks=1.0, vs=1.0, batch=1, total_q=4, max_q_len=4, hq=8,
                 hkv=1, d=512, page=64, out_dtype=1)
        a.update(over)
        return L.attn_prefill_hd512_e4m3_mma_append(
            FAKE, a["kn"], a["vn"], FAKE, FAKE, a["ks"], a["vs"], FAKE, FAKE, FAKE, FAKE,
            a["batch"], a["total_q"], a["max_q_len"], a["hq"], a["hkv"], a["d"], a["page"], 4,
            4, 0.04, None, FAKE, a["out_dtype"], None, None)
    assert pa(kn=None) == 1
    assert pa(vn=None) == 1
    assert pa(ks=0.0) == 2
    assert pa(vs=-1.0) == 2
    assert pa(d=256) == 3
    assert pa(page=16) == 3
    assert pa(hq=6, hkv=4) == 2
    assert pa(out_dtype=2) == 3
    assert pa(max_q_len=5) == 2            # larger than total_q
    assert pa(total_q=0, max_q_len=0) == 0


def test_prefill_splitk_validation(L):
    def pf(**over):
        a = dict(kvd=0, ks=1.0, vs=1.0, batch=1, total_q=4, max_q_len=4, hq=8, hkv=1, d=512,
                 page=64, max_pages=4, max_kv=256, kps=64, ws=FAKE, ws_bytes=16, out_dtype=1)
        a.update(over)
        return L.attn_prefill_hd512_splitk(
            FAKE, FAKE, FAKE, a["kvd"], a["ks"], a["vs"], FAKE, FAKE, FAKE, FAKE, a["batch"],
            a["total_q"], a["max_q_len"], a["hq"], a["hkv"], a["d"], a["page"], 4,
            a["max_pages"], a["max_kv"], a["kps"], 0.04, None, a["ws"], a["ws_bytes"], FAKE,
            a["out_dtype"], None, None)
    assert pf() == 4                       # four 64-key ranges need a workspace
    assert pf(ws=None) == 4
    assert pf(kps=100) == 2                # not a multiple of 64
    assert pf(kps=-64) == 2
    assert pf(max_kv=0) == 2
    assert pf(max_kv=257) == 2             # beyond max_pages * 64
    assert pf(kvd=1) == 3
    assert pf(kvd=2, ks=0.0) == 2
    assert pf(d=256) == 3
    assert pf(total_q=0, max_q_len=0) == 0


def test_prefill_splitk_workspace_size(L):
    f = L.attn_prefill_hd512_splitk_workspace_size
    # 512 rows x g = 8 -> 32 row blocks x 4 KV heads = 128 workgroups; two
    # ranges fill the 256 compute units in one round
    assert f(1, 512, 512, 32, 4, 32768, 0) == 2 * 512 * 32 * (512 + 2) * 4
    # 256 rows: 64 workgroups, four ranges
    assert f(1, 256, 256, 32, 4, 32768, 0) == 4 * 256 * 32 * (512 + 2) * 4
    assert f(1, 512, 512, 32, 4, 32768, 4096) == 8 * 512 * 32 * (512 + 2) * 4
    assert f(1, 512, 600, 32, 4, 32768, 4096) == 8 * 600 * 32 * (512 + 2) * 4
    # enough workgroups already: a single pass, no workspace
    assert f(1, 8192, 8192, 32, 4, 16384, 0) == 0
    assert f(1, 512, 512, 32, 4, 32768, 32768) == 0
    assert f(1, 512, 512, 32, 4, 32768, 100) == 0      # invalid: not a multiple of 64
    assert f(1, 512, 256, 32, 4, 32768, 0) == 0        # invalid: total_q < max_q_len


def test_append_validation(L):
    def ap(**over):
        a = dict(kn=FAKE, kvd=0, ks=1.0, vs=1.0, batch=1, total_q=4, hkv=2, d=512, page=64,
                 num_pages=4, max_pages=4)
        a.update(over)
        return L.attn_append_kv(a["kn"], FAKE, a["kvd"], a["ks"], a["vs"], FAKE, FAKE, FAKE,
                                a["batch"], a["total_q"], a["hkv"], a["d"], a["page"],
                                a["num_pages"], a["max_pages"], FAKE, FAKE, None)
    assert ap(kn=None) == 1
    assert ap(kvd=1) == 3
    assert ap(kvd=2, vs=0.0) == 2
    assert ap(d=256) == 3
    assert ap(batch=0) == 2
    assert ap(total_q=0) == 0


def test_workspace_size(L):
    n = L.attn_decode_splitk_workspace_size(64, 8, 4, 28672, 1024)
    assert n == 64 * 8 * 28 * 4 * (512 + 2) * 4   # 4 partials per split
    assert L.attn_decode_splitk_workspace_size(64, 8, 4, 28672, 100) == 0
    assert L.attn_decode_splitk_workspace_size(0, 8, 4, 28672, 0) == 0
    assert L.attn_decode_splitk_workspace_size(64, 8, 4, 28672, 0) > 0
    assert L.attn_decode_splitk_ex_workspace_size(64, 3, 8, 4, 28672, 1024) == 3 * n
    assert L.attn_decode_splitk_ex_workspace_size(64, 0, 8, 4, 28672, 1024) == 0


def test_decode_noalloc_validation(L):
    def call(q=FAKE, batch=64, q_len=1, hq=8, hkv=4, max_kv=28672, kps=0, kv=0, d=512):
        return L.attn_decode_splitk_ex_noalloc(q, FAKE, FAKE, kv, 1.0, 1.0, FAKE, FAKE, batch,
                                               q_len, hq, hkv, d, 64, 16384, 448, max_kv, kps,
                                               0.04, None, FAKE, 0, None, None)
    assert call(q=None) == 1
    assert call(d=256) == 3
    # partials past the 64 MiB scratch: refused before any device call
    assert call(batch=4096, max_kv=28672, kps=64) == 4
    assert call(q_len=3, hq=8, hkv=4, batch=4096, kps=1024) == 4


def test_prefill_persistent_validation(L):
    assert L.attn_prefill_hd512_persistent_workspace_size() >= 4
    def call(ws=FAKE, nbytes=256, kv=0, d=512):
        return L.attn_prefill_hd512_persistent(FAKE, FAKE, FAKE, kv, 1.0, 1.0, FAKE, FAKE, FAKE,
                                               FAKE, 1, 4, 4, 8, 1, d, 64, 4, 1, 0.04, None, ws,
                                               nbytes, FAKE, 1, None, None)
    assert call(ws=None) == 1
    assert call(nbytes=2) == 4
    assert call(kv=7) == 3
    assert call(d=256) == 3


def test_wide_multi_token_decode_workspace(L):
    # up to 48 (token, head) columns per KV head the decode kernels run:
    # (O, m, l) partials per split and column, 4 slots per column reserved.
    # The default ranges: 1792 keys at batch 64, max 28672 keys (16 splits)
    # for one 16-column block, twice that for two or three (8 splits)
    dec = L.attn_decode_splitk_ex_workspace_size(64, 5, 32, 4, 28672, 0)   # 40 columns
    assert dec == 64 * 5 * 32 * 8 * 4 * 514 * 4
    one = L.attn_decode_splitk_ex_workspace_size(64, 1, 8, 4, 28672, 0)    # 2 columns
    assert one == 64 * 1 * 8 * 16 * 4 * 514 * 4
    # 7 tokens x g = 8 = 56 columns: routed through the split-K prefill; its
    # workspace is the row offsets and chunk starts (2 batch + 1 ints, padded
    # to 256 bytes) plus the prefill's partials for batch x q_len rows
    routed = L.attn_decode_splitk_ex_workspace_size(64, 7, 32, 4, 28672, 0)
    part = L.attn_prefill_hd512_splitk_workspace_size(64, 7, 448, 32, 4, 28672, 1792)
    assert routed == 768 + part and part == 16 * 448 * 32 * 514 * 4
    assert L.attn_decode_splitk_ex_workspace_size(64, 7, 32, 4, 28672, 4096) == \
        768 + L.attn_prefill_hd512_splitk_workspace_size(64, 7, 448, 32, 4, 28672, 4096)


def test_probe_validation(L):
    assert L.attn_hbm_read_probe(None, 1024, FAKE, None) == 1
    assert L.attn_hbm_read_probe(FAKE, 1000, FAKE, None) == 2
    assert L.attn_hbm_probe_sink_words(1 << 20) >= 1
    assert L.attn_clock_stamps(None, 8, None) == 1
    assert L.attn_clock_stamps(FAKE, 0, None) == 2
    assert L.attn_clock_stamps(FAKE, 65537, None) == 2


def test_prefill_fp8_mma_validation(L):
    def pm(**over):
        a = dict(q=FAKE, ks=1.0, vs=1.0, batch=1, total_q=4, max_q_len=4, hq=8, hkv=1, d=512,
                 page=64, out_dtype=1)
        a.update(over)
        return L.attn_prefill_hd512_e4m3_mma(
            a["q"], FAKE, FAKE, a["ks"], a["vs"], FAKE, FAKE, FAKE, FAKE, a["batch"],
            a["total_q"], a["max_q_len"], a["hq"], a["hkv"], a["d"], a["page"], 4, 4, 0.04,
            None, FAKE, a["out_dtype"], None, None)
    assert pm(q=None) == 1
    assert pm(ks=0.0) == 2
    assert pm(vs=-1.0) == 2
    assert pm(d=256) == 3
    assert pm(page=16) == 3
    assert pm(hq=6, hkv=4) == 2
    assert pm(out_dtype=2) == 3
    assert pm(total_q=0, max_q_len=0) == 0


def test_prefill_splitk_fp8_mma_validation(L):
    def ps(**over):
        a = dict(ks=1.0, batch=1, total_q=4, max_q_len=4, hq=8, hkv=1, d=512, page=64,
                 mkv=64, kps=64, ws=None, wsb=0)
        a.update(over)
        return L.attn_prefill_hd512_splitk_e4m3_mma(
            FAKE, FAKE, FAKE, a["ks"], 1.0, FAKE, FAKE, FAKE, FAKE, a["batch"], a["total_q"],
            a["max_q_len"], a["hq"], a["hkv"], a["d"], a["page"], 4, 4, a["mkv"], a["kps"], 0.04,
            None, a["ws"], a["wsb"], FAKE, 1, None, None)
    assert ps(ks=0.0) == 2
    assert ps(kps=100) == 2          # not a multiple of 64
    assert ps(mkv=0) == 2
    assert ps(d=256) == 3
    assert ps(total_q=0, max_q_len=0) == 0
