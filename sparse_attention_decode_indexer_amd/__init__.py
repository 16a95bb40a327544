"""Python binding of the MI355X DSA decode/verify library (``libdsa.so``).

Argument marshalling only: every function forwards to the C entry point of the same
name declared in ``include/dsa.h``; all computation runs in the HIP kernels.  Tensor
arguments may be PyTorch tensors (their ``data_ptr()`` is passed) or raw integer
addresses; PyTorch supplies device memory and streams, nothing else.  Importing the
package fails loudly if the library has not been built.
"""
from __future__ import annotations

import ctypes as C
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdsa.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python sparse_attention_decode_indexer_amd/build.py` "
        "(or __graft_entry__.build()); there is no fallback implementation.")

_lib = C.CDLL(LIB_PATH)

# dtypes / kinds (include/dsa.h)
BF16, FP8_E4M3, FP32 = 0, 1, 2
WS_TOPK, WS_INDEX_TOPK, WS_SPARSE_ATTN, WS_SWA_ATTN, WS_LAYER_DSA, WS_LAYER_SWA, WS_MODULE = 1, 2, 3, 4, 5, 6, 7
MAX_MODULE_LAYERS = 64
LAYER_DSA, LAYER_SWA = 0, 1
STATUS = {0: "DSA_OK", 1: "DSA_ERR_NULL", 2: "DSA_ERR_SHAPE", 3: "DSA_ERR_DTYPE", 4: "DSA_ERR_ALIGN",
          5: "DSA_ERR_WORKSPACE", 6: "DSA_ERR_LAUNCH", 7: "DSA_ERR_HIP"}

EXPORTS = ("dsa_indexer_scores", "dsa_topk", "dsa_index_topk", "dsa_sparse_attn", "dsa_sparse_attn_static", "swa_attn",
           "dsa_layer_step", "dsa_module_step", "dsa_workspace_bytes", "dsa_workspace_init", "dsa_workspace_status",
           "dsa_max_context", "dsa_status_string", "dsa_last_error")


class DSAError(RuntimeError):
    def __init__(self, fn: str, status: int):
        msg = _lib.dsa_status_string(status).decode()
        extra = _lib.dsa_last_error().decode()
        super().__init__(f"{fn}: {STATUS.get(status, status)} ({msg}){' -- ' + extra if extra else ''}")
        self.status = status


class LayerConfig(C.Structure):
    _fields_ = [("kind", C.c_int), ("hidden", C.c_int), ("top_k", C.c_int), ("window", C.c_int),
                ("rms_eps", C.c_float), ("rope_theta", C.c_float), ("sm_scale", C.c_float),
                ("sink", C.c_void_p)]


class LayerWeights(C.Structure):
    """rms_gamma, w_qkvi, w_o (+ w_dtype, w_qkvi_scale, w_o_scale for W8A8); unset
    trailing fields are 0 / NULL, i.e. bf16 weights."""
    _fields_ = [("rms_gamma", C.c_void_p), ("w_qkvi", C.c_void_p), ("w_o", C.c_void_p),
                ("w_dtype", C.c_int), ("w_qkvi_scale", C.c_void_p), ("w_o_scale", C.c_void_p)]


class LayerCache(C.Structure):
    _fields_ = [("k", C.c_void_p), ("v", C.c_void_p), ("k_idx", C.c_void_p),
                ("k_idx_scale", C.c_void_p), ("capacity", C.c_int64)]


_P, _I, _L, _F, _S = C.c_void_p, C.c_int, C.c_int64, C.c_float, C.c_size_t
_sig = {
    "dsa_indexer_scores": [_P, _P, _P, _P, _I, _I, _L, _L, _P, _L, _P],
    "dsa_topk": [_P, _I, _L, _L, _L, _I, _P, _P, _P, _S, _P],
    "dsa_index_topk": [_P, _P, _P, _P, _I, _I, _L, _L, _I, _P, _P, _P, _S, _P],
    "dsa_sparse_attn": [_P, _P, _P, _P, _P, _I, _P, _I, _I, _L, _F, _P, _P, _I, _P, _S, _P],
    "dsa_sparse_attn_static": [_P, _P, _P, _P, _P, _I, _P, _I, _I, _L, _F, _P, _P, _I, _P],
    "swa_attn": [_P, _P, _P, _P, _P, _I, _L, _I, _L, _I, _F, _P, _P, _I, _P, _S, _P],
    "dsa_layer_step": [C.POINTER(LayerConfig), C.POINTER(LayerWeights), C.POINTER(LayerCache),
                       _P, _P, _I, _L, _P, _P, _P, _S, _P],
    "dsa_module_step": [_I, C.POINTER(LayerConfig), C.POINTER(LayerWeights), C.POINTER(LayerCache),
                        _P, _P, _I, _L, _P, _P, _S, _P],
    "dsa_workspace_init": [_P, _S, _P],
    "dsa_workspace_status": [_P, _S, _P],
}
for _name, _args in _sig.items():
    getattr(_lib, _name).argtypes = _args
    getattr(_lib, _name).restype = C.c_int
_lib.dsa_workspace_bytes.argtypes = [_I, _I, _L, _I]
_lib.dsa_workspace_bytes.restype = C.c_size_t
_lib.dsa_max_context.argtypes = []
_lib.dsa_max_context.restype = C.c_int64
_lib.dsa_status_string.argtypes = [C.c_int]
_lib.dsa_status_string.restype = C.c_char_p
_lib.dsa_last_error.argtypes = []
_lib.dsa_last_error.restype = C.c_char_p


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _nbytes(x):
    if isinstance(x, int) or x is None:
        return 0
    return x.numel() * x.element_size()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(fn, status, raise_on_error):
    if status != 0 and raise_on_error:
        raise DSAError(fn, status)
    return status


# ----------------------------------------------------------------------------- entry points

def dsa_indexer_scores(q_idx, w_idx, k_idx, k_idx_scale, k_dtype, T, L, pos0, scores, ld,
                       stream=None, raise_on_error=True):
    st = _lib.dsa_indexer_scores(_ptr(q_idx), _ptr(w_idx), _ptr(k_idx), _ptr(k_idx_scale), k_dtype,
                                 T, L, pos0, _ptr(scores), ld, _stream(stream))
    return _check("dsa_indexer_scores", st, raise_on_error)


def dsa_topk(scores, T, L, ld, pos0, k, idx, count, ws, ws_bytes=None, stream=None,
             raise_on_error=True):
    st = _lib.dsa_topk(_ptr(scores), T, L, ld, pos0, k, _ptr(idx), _ptr(count), _ptr(ws),
                       _nbytes(ws) if ws_bytes is None else ws_bytes, _stream(stream))
    return _check("dsa_topk", st, raise_on_error)


def dsa_index_topk(q_idx, w_idx, k_idx, k_idx_scale, k_dtype, T, L, pos0, k, idx, count, ws,
                   ws_bytes=None, stream=None, raise_on_error=True):
    st = _lib.dsa_index_topk(_ptr(q_idx), _ptr(w_idx), _ptr(k_idx), _ptr(k_idx_scale), k_dtype, T, L,
                             pos0, k, _ptr(idx), _ptr(count), _ptr(ws),
                             _nbytes(ws) if ws_bytes is None else ws_bytes, _stream(stream))
    return _check("dsa_index_topk", st, raise_on_error)


def dsa_sparse_attn(q, k_cache, v_cache, k_scale, v_scale, kv_dtype, idx, k, T, L, sm_scale, sink,
                    out, out_dtype, ws, ws_bytes=None, stream=None, raise_on_error=True):
    st = _lib.dsa_sparse_attn(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale),
                              kv_dtype, _ptr(idx), k, T, L, sm_scale, _ptr(sink), _ptr(out), out_dtype,
                              _ptr(ws), _nbytes(ws) if ws_bytes is None else ws_bytes, _stream(stream))
    return _check("dsa_sparse_attn", st, raise_on_error)


def dsa_sparse_attn_static(q, k_cache, v_cache, k_scale, v_scale, kv_dtype, idx, k, T, L, sm_scale, sink,
                           out, out_dtype, stream=None, raise_on_error=True):
    st = _lib.dsa_sparse_attn_static(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale),
                                     kv_dtype, _ptr(idx), k, T, L, sm_scale, _ptr(sink), _ptr(out), out_dtype,
                                     _stream(stream))
    return _check("dsa_sparse_attn_static", st, raise_on_error)


def swa_attn(q, k_ring, v_ring, k_scale, v_scale, kv_dtype, ring_cap, T, pos0, window, sm_scale, sink,
             out, out_dtype, ws, ws_bytes=None, stream=None, raise_on_error=True):
    st = _lib.swa_attn(_ptr(q), _ptr(k_ring), _ptr(v_ring), _ptr(k_scale), _ptr(v_scale), kv_dtype, ring_cap,
                       T, pos0, window, sm_scale, _ptr(sink), _ptr(out), out_dtype, _ptr(ws),
                       _nbytes(ws) if ws_bytes is None else ws_bytes, _stream(stream))
    return _check("swa_attn", st, raise_on_error)


def dsa_layer_step(cfg: LayerConfig, weights: LayerWeights, cache: LayerCache, x_in, x_out, T, pos0,
                   idx_out=None, qkv_out=None, ws=None, ws_bytes=None, stream=None,
                   raise_on_error=True):
    st = _lib.dsa_layer_step(C.byref(cfg), C.byref(weights), C.byref(cache), _ptr(x_in), _ptr(x_out),
                             T, pos0, _ptr(idx_out), _ptr(qkv_out), _ptr(ws),
                             _nbytes(ws) if ws_bytes is None else ws_bytes, _stream(stream))
    return _check("dsa_layer_step", st, raise_on_error)


def dsa_module_step(cfgs, weights, caches, x_in, x_out, T, pos0, idx_out=None, ws=None, ws_bytes=None,
                    stream=None, raise_on_error=True):
    """Layers cfgs[i], weights[i], caches[i] applied in order to the block (one call)."""
    n = len(cfgs)
    if len(weights) != n or len(caches) != n:
        raise ValueError("dsa_module_step: one config, weight set and cache per layer")
    ca = (LayerConfig * n)(*cfgs)
    wa = (LayerWeights * n)(*weights)
    ka = (LayerCache * n)(*caches)
    st = _lib.dsa_module_step(n, ca, wa, ka, _ptr(x_in), _ptr(x_out), T, pos0, _ptr(idx_out), _ptr(ws),
                              _nbytes(ws) if ws_bytes is None else ws_bytes, _stream(stream))
    return _check("dsa_module_step", st, raise_on_error)


def dsa_workspace_bytes(kind, T, L, k):
    return _lib.dsa_workspace_bytes(kind, T, L, k)


def dsa_workspace_init(ws, ws_bytes=None, stream=None):
    st = _lib.dsa_workspace_init(_ptr(ws), _nbytes(ws) if ws_bytes is None else ws_bytes, _stream(stream))
    return _check("dsa_workspace_init", st, True)


def dsa_workspace_status(ws, ws_bytes=None, stream=None, raise_on_error=True):
    """Blocking: synchronises the stream and reports the workspace's sticky error word."""
    st = _lib.dsa_workspace_status(_ptr(ws), _nbytes(ws) if ws_bytes is None else ws_bytes, _stream(stream))
    return _check("dsa_workspace_status", st, raise_on_error)


def dsa_max_context():
    return _lib.dsa_max_context()


def dsa_status_string(status):
    return _lib.dsa_status_string(status).decode()


def dsa_last_error():
    return _lib.dsa_last_error().decode()


# ----------------------------------------------------------------------------- conveniences

def workspace(kind, T, L, k, device="cuda"):
    """A zero-filled workspace tensor of the size the library asks for."""
    import torch
    n = dsa_workspace_bytes(kind, T, L, k)
    n = (n + 255) // 256 * 256
    return torch.zeros(n, dtype=torch.uint8, device=device)


def layer_config(kind, top_k=2048, window=128, rms_eps=1e-6, rope_theta=1e6, sm_scale=None, sink=None):
    import math
    return LayerConfig(kind, 4096, top_k, window, rms_eps, rope_theta,
                       1.0 / math.sqrt(128) if sm_scale is None else sm_scale, _ptr(sink))
