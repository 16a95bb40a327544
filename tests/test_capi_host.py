"""Host-side checks of the C ABI (no GPU needed): the library loads, exports every
symbol include/dsa.h declares, sizes workspaces, and rejects bad arguments before
launching anything."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HDR = os.path.join(ROOT, "include", "dsa.h")


def _declared():
    txt = open(HDR).read()
    pat = r"^(?:dsa_status_t|size_t|int64_t|const char\s*\*)\s*(\w+)\s*\("
    return sorted(set(re.findall(pat, txt, flags=re.M)))


def test_library_exports_every_declared_symbol():
    import sparse_attention_decode_indexer_amd as dsa
    names = _declared()
    assert set(dsa.EXPORTS) == set(names), names
    lib = C.CDLL(dsa.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    import sparse_attention_decode_indexer_amd as dsa
    for s in range(8):
        assert dsa.dsa_status_string(s)
    assert dsa.dsa_status_string(0) == "ok"


def test_workspace_sizes_are_monotone_and_cover_candidates():
    import sparse_attention_decode_indexer_amd as dsa
    small = dsa.dsa_workspace_bytes(dsa.WS_INDEX_TOPK, 8, 65536, 2048)
    big = dsa.dsa_workspace_bytes(dsa.WS_INDEX_TOPK, 8, 1 << 20, 2048)
    assert 0 < small < big
    assert big >= 8 * (1 << 20) * 8            # every position can be a candidate
    assert dsa.dsa_workspace_bytes(dsa.WS_SPARSE_ATTN, 8, 1 << 20, 2048) >= 8 * 32 * 8 * 130 * 4
    assert dsa.dsa_workspace_bytes(dsa.WS_LAYER_DSA, 8, 1 << 20, 2048) > big
    assert dsa.dsa_workspace_bytes(dsa.WS_LAYER_SWA, 8, 1 << 20, 128) > 0
    assert dsa.dsa_workspace_bytes(dsa.WS_TOPK, 0, 100, 10) == 0


def test_long_context_limit_and_spill_workspace(monkeypatch):
    """Past 4096 keys per CU the selection keeps the rest of each chunk's scores in the
    workspace: the context limit is 65536 keys per CU, and the workspace is the control
    block, the count and bound slots, one candidate slot per key and chunk position of
    each of 8 tokens, and the spilled scores (fp32, 8 tokens x workgroups x (chunk - 4096))."""
    import sparse_attention_decode_indexer_amd as dsa
    assert dsa.dsa_max_context() % 65536 == 0 and dsa.dsa_max_context() >= 65536
    monkeypatch.setenv("DSA_NUM_CU", "4")          # geometry cut for 4 CUs
    assert dsa.dsa_max_context() == 4 * 65536
    L = 40000                                      # chunk = roundup(10000, 512) = 10240
    ctl, slots = 16384, 8 * 1024 * 16

    def ws(nwg, chunk):                            # nwg = max(chunks, T): one workgroup per token at least
        return ctl + slots + 8 * nwg * chunk * 8 + (8 * nwg * (chunk - 4096) * 4 if chunk > 4096 else 0)

    assert dsa.dsa_workspace_bytes(dsa.WS_INDEX_TOPK, 8, L, 2048) == ws(8, 10240)
    assert dsa.dsa_workspace_bytes(dsa.WS_TOPK, 3, L, 100) == ws(4, 10240)
    # up to 4096 keys per CU nothing spills
    assert dsa.dsa_workspace_bytes(dsa.WS_INDEX_TOPK, 2, 16384, 2048) == ws(4, 4096)
    assert dsa.dsa_workspace_bytes(dsa.WS_LAYER_DSA, 8, L, 2048) > ws(8, 10240)


FAKE = 0x10000          # aligned, never dereferenced: every call below fails validation first
MIS = 0x10004           # misaligned


def test_validation_errors_without_launch():
    import sparse_attention_decode_indexer_amd as dsa
    E = {v: k for k, v in dsa.STATUS.items()}
    f = lambda *a, **k: dsa.dsa_indexer_scores(*a, stream=0, raise_on_error=False, **k)
    assert f(None, FAKE, FAKE, None, dsa.BF16, 1, 100, 99, FAKE, 100) == E["DSA_ERR_NULL"]
    assert f(FAKE, FAKE, FAKE, None, 7, 1, 100, 99, FAKE, 100) == E["DSA_ERR_DTYPE"]
    assert f(FAKE, FAKE, FAKE, None, dsa.FP8_E4M3, 1, 100, 99, FAKE, 100) == E["DSA_ERR_DTYPE"]
    assert f(FAKE, FAKE, FAKE, FAKE, dsa.BF16, 1, 100, 99, FAKE, 100) == E["DSA_ERR_DTYPE"]
    assert f(FAKE, FAKE, FAKE, None, dsa.BF16, 9, 100, 90, FAKE, 100) == E["DSA_ERR_SHAPE"]
    assert f(FAKE, FAKE, FAKE, None, dsa.BF16, 0, 100, 90, FAKE, 100) == E["DSA_ERR_SHAPE"]
    assert f(FAKE, FAKE, FAKE, None, dsa.BF16, 2, 100, 99, FAKE, 100) == E["DSA_ERR_SHAPE"]   # pos0+T > L
    assert f(FAKE, FAKE, FAKE, None, dsa.BF16, 1, 100, 99, FAKE, 98) == E["DSA_ERR_SHAPE"]    # ld < L
    assert f(FAKE, FAKE, FAKE, None, dsa.BF16, 1, 100, 99, FAKE, 102) == E["DSA_ERR_SHAPE"]   # ld % 4
    assert f(MIS, FAKE, FAKE, None, dsa.BF16, 1, 100, 99, FAKE, 100) == E["DSA_ERR_ALIGN"]
    t = lambda *a: dsa.dsa_topk(*a, stream=0, raise_on_error=False)
    assert t(FAKE, 1, 100, 100, 99, 0, FAKE, None, FAKE, 1 << 30) == E["DSA_ERR_SHAPE"]        # k = 0
    assert t(FAKE, 1, 100, 100, 99, 2049, FAKE, None, FAKE, 1 << 30) == E["DSA_ERR_SHAPE"]
    assert t(FAKE, 1, 100, 100, 99, 16, FAKE, None, FAKE, 16) == E["DSA_ERR_WORKSPACE"]
    assert t(FAKE, 1, 100, 100, 99, 16, None, None, FAKE, 1 << 30) == E["DSA_ERR_NULL"]
    too_long = dsa.dsa_max_context() + 8
    assert t(FAKE, 1, too_long, too_long, too_long - 1, 16, FAKE, None, FAKE, 1 << 40) == E["DSA_ERR_SHAPE"]
    a = lambda *x: dsa.dsa_sparse_attn(*x, stream=0, raise_on_error=False)
    assert a(FAKE, FAKE, FAKE, None, None, dsa.FP8_E4M3, FAKE, 16, 1, 100, 0.1, None, FAKE, dsa.FP32,
             FAKE, 1 << 30) == E["DSA_ERR_DTYPE"]
    assert a(FAKE, FAKE, FAKE, None, None, dsa.BF16, FAKE, 16, 1, 100, 0.1, None, FAKE, 5,
             FAKE, 1 << 30) == E["DSA_ERR_DTYPE"]
    assert a(FAKE, FAKE, FAKE, None, None, dsa.BF16, FAKE, 16, 1, 100, 0.1, None, FAKE, dsa.FP32,
             FAKE, 8) == E["DSA_ERR_WORKSPACE"]
    s = lambda *x: dsa.swa_attn(*x, stream=0, raise_on_error=False)
    assert s(FAKE, FAKE, FAKE, None, None, dsa.BF16, 130, 8, 500, 128, 0.1, None, FAKE, dsa.FP32, FAKE,
             1 << 30) == E["DSA_ERR_SHAPE"]
    assert s(FAKE, FAKE, FAKE, None, None, dsa.BF16, 135, 8, 500, 128, 0.1, None, FAKE, dsa.FP32, None,
             1 << 30) == E["DSA_ERR_WORKSPACE"]
    # e4m3 rings need both row-scale vectors, bf16 rings none
    assert s(FAKE, FAKE, FAKE, None, FAKE, dsa.FP8_E4M3, 135, 8, 500, 128, 0.1, None, FAKE, dsa.FP32, FAKE,
             1 << 30) == E["DSA_ERR_DTYPE"]
    assert s(FAKE, FAKE, FAKE, FAKE, FAKE, dsa.BF16, 135, 8, 500, 128, 0.1, None, FAKE, dsa.FP32, FAKE,
             1 << 30) == E["DSA_ERR_DTYPE"]
    cfg = dsa.layer_config(dsa.LAYER_DSA)
    w = dsa.LayerWeights(FAKE, FAKE, FAKE)
    c = dsa.LayerCache(FAKE, FAKE, FAKE, FAKE, 1000)
    L = lambda **kw: dsa.dsa_layer_step(cfg, w, c, FAKE, FAKE + 0x1000, 8, 100, ws=FAKE, ws_bytes=16,
                                        stream=0, raise_on_error=False, **kw)
    assert L() == E["DSA_ERR_WORKSPACE"]
    c.capacity = 100
    assert L() == E["DSA_ERR_SHAPE"]          # pos0 + T > capacity
    cfg.hidden = 2048
    c.capacity = 1000
    assert L() == E["DSA_ERR_SHAPE"]
    cfg.hidden = 4096
    c.k_idx = None
    assert L() == E["DSA_ERR_NULL"]


def test_w8a8_validation_without_launch():
    import sparse_attention_decode_indexer_amd as dsa
    E = {v: k for k, v in dsa.STATUS.items()}
    cfg = dsa.layer_config(dsa.LAYER_DSA)
    c = dsa.LayerCache(FAKE, FAKE, FAKE, FAKE, 1000)

    def L(w):
        return dsa.dsa_layer_step(cfg, w, c, FAKE, FAKE + 0x1000, 8, 100, ws=FAKE, ws_bytes=1 << 40,
                                  stream=0, raise_on_error=False)
    assert L(dsa.LayerWeights(FAKE, FAKE, FAKE, 7, None, None)) == E["DSA_ERR_DTYPE"]
    # e4m3 weights need both row-scale vectors; bf16 weights take none
    assert L(dsa.LayerWeights(FAKE, FAKE, FAKE, dsa.FP8_E4M3, None, None)) == E["DSA_ERR_DTYPE"]
    assert L(dsa.LayerWeights(FAKE, FAKE, FAKE, dsa.FP8_E4M3, FAKE, None)) == E["DSA_ERR_DTYPE"]
    assert L(dsa.LayerWeights(FAKE, FAKE, FAKE, dsa.BF16, FAKE, FAKE)) == E["DSA_ERR_DTYPE"]


def test_workspace_status_validation_without_device_access():
    """The status call checks its arguments before it synchronises or reads anything."""
    import sparse_attention_decode_indexer_amd as dsa
    E = {v: k for k, v in dsa.STATUS.items()}
    st = lambda *a: dsa.dsa_workspace_status(*a, stream=0, raise_on_error=False)
    assert st(None, 1 << 20) == E["DSA_ERR_NULL"]
    assert st(MIS, 1 << 20) == E["DSA_ERR_ALIGN"]
    assert st(FAKE, 16383) == E["DSA_ERR_WORKSPACE"]        # smaller than the control block


def test_every_workspace_holds_the_control_block():
    import sparse_attention_decode_indexer_amd as dsa
    for kind, k in ((dsa.WS_TOPK, 64), (dsa.WS_INDEX_TOPK, 64), (dsa.WS_SPARSE_ATTN, 64),
                    (dsa.WS_SWA_ATTN, 128), (dsa.WS_LAYER_DSA, 64), (dsa.WS_LAYER_SWA, 128),
                    (dsa.WS_MODULE, 64), (dsa.WS_MODULE, 0)):
        assert dsa.dsa_workspace_bytes(kind, 1, 4096, k) >= 16384, kind


def test_read_ceiling_helper_is_outside_the_library_and_validates():
    """The benchmark's streaming-read helper lives in its own library: libdsa.so does not
    export it, and it rejects bad arguments without launching."""
    import sparse_attention_decode_indexer_amd as dsa
    lib = C.CDLL(dsa.LIB_PATH)
    assert not hasattr(lib, "dsa_stream_read") and not hasattr(lib, "dsa_read_ceiling_stream")
    rc = C.CDLL(os.path.join(os.path.dirname(dsa.LIB_PATH), "libdsa_read_ceiling.so"))
    f = rc.dsa_read_ceiling_stream
    f.argtypes = [C.c_void_p, C.c_size_t, C.c_void_p, C.c_void_p]
    f.restype = C.c_int
    assert f(None, 1024, FAKE, None) == -1
    assert f(FAKE, 1024, None, None) == -1
    assert f(MIS, 1024, FAKE, None) == -1
    assert f(FAKE, 1000, FAKE, None) == -1
    assert f(FAKE, 0, FAKE, None) == -1


def test_static_attention_validation_without_launch():
    """The allocation-free attention call checks its arguments before it looks up its scratch
    or launches anything."""
    import sparse_attention_decode_indexer_amd as dsa
    E = {v: k for k, v in dsa.STATUS.items()}
    a = lambda *x: dsa.dsa_sparse_attn_static(*x, stream=0, raise_on_error=False)
    assert a(None, FAKE, FAKE, None, None, dsa.BF16, FAKE, 16, 1, 100, 0.1, None, FAKE, dsa.FP32) == E["DSA_ERR_NULL"]
    assert a(FAKE, FAKE, FAKE, None, None, dsa.FP8_E4M3, FAKE, 16, 1, 100, 0.1, None, FAKE,
             dsa.FP32) == E["DSA_ERR_DTYPE"]
    assert a(FAKE, FAKE, FAKE, None, None, dsa.BF16, FAKE, 2049, 1, 100, 0.1, None, FAKE, dsa.FP32) == E["DSA_ERR_SHAPE"]
    assert a(FAKE, FAKE, FAKE, None, None, dsa.BF16, FAKE, 16, 9, 100, 0.1, None, FAKE, dsa.FP32) == E["DSA_ERR_SHAPE"]
    assert a(MIS, FAKE, FAKE, None, None, dsa.BF16, FAKE, 16, 1, 100, 0.1, None, FAKE, dsa.FP32) == E["DSA_ERR_ALIGN"]


def test_module_step_validation_without_launch():
    """dsa_module_step checks every layer (the layer step's checks), the layer count, the
    aliasing of x_in and x_out, idx_out without a DSA layer and the workspace before any
    launch; its workspace covers a DSA layer's and grows with top-k."""
    import sparse_attention_decode_indexer_amd as dsa
    E = {v: k for k, v in dsa.STATUS.items()}
    swa = dsa.layer_config(dsa.LAYER_SWA)
    dsa_cfg = dsa.layer_config(dsa.LAYER_DSA)
    w = dsa.LayerWeights(FAKE, FAKE, FAKE)
    ring = dsa.LayerCache(FAKE, FAKE, None, None, 256)
    cache = dsa.LayerCache(FAKE, FAKE, FAKE, FAKE, 1000)
    big = 1 << 40

    def M(cfgs, caches, xo=FAKE + 0x1000, ws_bytes=big, idx=None, T=8, pos0=100):
        return dsa.dsa_module_step(cfgs, [w] * len(cfgs), caches, FAKE, xo, T, pos0, idx_out=idx, ws=FAKE,
                                   ws_bytes=ws_bytes, stream=0, raise_on_error=False)
    assert M([swa], [ring], ws_bytes=16) == E["DSA_ERR_WORKSPACE"]
    assert M([swa], [ring], xo=FAKE) == E["DSA_ERR_SHAPE"]                       # x_out aliases x_in
    assert M([swa] * 65, [ring] * 65) == E["DSA_ERR_SHAPE"]                       # too many layers
    assert M([swa], [ring], idx=FAKE) == E["DSA_ERR_SHAPE"]                       # no DSA layer to report
    assert M([swa, dsa_cfg], [ring, dsa.LayerCache(FAKE, FAKE, None, FAKE, 1000)]) == E["DSA_ERR_NULL"]
    assert M([swa, dsa_cfg], [ring, dsa.LayerCache(FAKE, FAKE, FAKE, FAKE, 100)]) == E["DSA_ERR_SHAPE"]
    assert M([swa], [dsa.LayerCache(FAKE, FAKE, None, None, 100)]) == E["DSA_ERR_SHAPE"]   # ring too small
    assert M([swa, dsa_cfg], [ring, dsa.LayerCache(FAKE, MIS, FAKE, FAKE, 1000)]) == E["DSA_ERR_ALIGN"]
    assert M([swa, dsa_cfg], [ring, cache], T=9) == E["DSA_ERR_SHAPE"]
    assert dsa.dsa_module_step([], [], [], FAKE, FAKE + 0x1000, 8, 100, ws=FAKE, ws_bytes=big, stream=0,
                               raise_on_error=False) == E["DSA_ERR_SHAPE"]
    m0 = dsa.dsa_workspace_bytes(dsa.WS_MODULE, 8, 1 << 20, 0)
    m1 = dsa.dsa_workspace_bytes(dsa.WS_MODULE, 8, 1 << 20, 2048)
    assert m1 > m0 > 0
    assert m1 >= dsa.dsa_workspace_bytes(dsa.WS_LAYER_DSA, 8, 1 << 20, 2048)
    assert M([swa, dsa_cfg], [ring, cache], ws_bytes=m0) == E["DSA_ERR_WORKSPACE"]
