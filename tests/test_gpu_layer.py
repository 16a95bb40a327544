"""dsa_layer_step on the GPU against the oracle's layer step.

Stage checks are teacher-forced: the oracle consumes the GPU's own rotated projection
(qkv_out) and selected indices, so each stage is compared on identical inputs:
* projection + RoPE: within one bf16 ulp of the fp64 result (fp32 accumulation);
* cache append: K/V rows equal the exported rotated rows bit for bit; the e4m3 indexer
  rows and scales equal the oracle's quantisation of the exported k_I bit for bit;
* selection: within the 2^-16 * S rounding band of the fp64 indexer scores;
* DSA layer output: the standalone sparse attention on the step's own rotated queries,
  cache and indices reproduces the layer's attention output bit for bit; the oracle's
  output projection of it must match to one bf16 ulp plus the fp32 accumulation bound
  2^-16 * sum |terms| (and the free-running oracle to 2e-2 * max(1, |ref|));
* SWA layer output: two bf16 ulps of the teacher-forced oracle.
"""
import math

import numpy as np
import pytest
import torch

import synth
from oracle import dsa_oracle as O
from tests.gpu_util import DEV, up, down, bf16_bits, tie_band_ok, check_oproj

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dsa():
    import sparse_attention_decode_indexer_amd as m
    return m


def _within_ulp(g, r, kind="dsa"):
    """Projection outputs: one bf16 ulp of the value for plain columns; for rotated
    columns the inputs of the rotation carry one-ulp differences each, so the bound is
    two ulps of the rotation pair's norm (which the rotation preserves)."""
    scale = np.abs(r).copy()
    segs = [(0, 1024, 128), (1024, 128, 128)]
    if kind == "dsa":
        segs += [(1280, 1024, 64), (2304, 64, 64)]
    for off, n, d in segs:
        blk = r[:, off:off + n].reshape(r.shape[0], -1, d)
        a, b = blk[..., : d // 2], blk[..., d // 2:]
        nrm = np.sqrt(a * a + b * b)
        scale[:, off:off + n] = np.concatenate([nrm, nrm], axis=-1).reshape(r.shape[0], n) * 2.0
    tol = 2.0 ** -7 * np.maximum(scale, 2.0 ** -30)
    return np.abs(g - r) <= tol


def _run_layer(dsa, kind, lay, x_bits, T, pos0, top_k=2048, window=128, sink=None, eps=1e-6, gamma=None,
               w8=None):
    """One dsa_layer_step; w8 = (w_qkvi codes, scales, w_o codes, scales) selects W8A8."""
    n_proj = synth.N_PROJ_DSA if kind == "dsa" else synth.N_PROJ_SWA
    cfg = dsa.layer_config(dsa.LAYER_DSA if kind == "dsa" else dsa.LAYER_SWA, top_k=top_k, window=window,
                           sink=sink, rms_eps=eps)
    g_gamma = up(lay.gamma if gamma is None else gamma)
    if w8 is None:
        g_w, g_wo = up(lay.w_qkvi), up(lay.w_o)
    else:
        g_w, g_sq, g_wo, g_so = (up(a) for a in w8)
    kc, vc = up(lay.k), up(lay.v)
    ki = up(lay.k_idx) if kind == "dsa" else None
    ks = up(lay.k_idx_scale) if kind == "dsa" else None
    cache = dsa.LayerCache(kc.data_ptr(), vc.data_ptr(), ki.data_ptr() if ki is not None else None,
                           ks.data_ptr() if ks is not None else None, lay.capacity)
    if w8 is None:
        w = dsa.LayerWeights(g_gamma.data_ptr(), g_w.data_ptr(), g_wo.data_ptr())
    else:
        w = dsa.LayerWeights(g_gamma.data_ptr(), g_w.data_ptr(), g_wo.data_ptr(), dsa.FP8_E4M3,
                             g_sq.data_ptr(), g_so.data_ptr())
    x = up(x_bits)
    xo = torch.zeros_like(x)
    qkv = torch.zeros((T, n_proj), dtype=torch.int16, device=DEV)
    idx = torch.full((T, top_k), -7, dtype=torch.int32, device=DEV) if kind == "dsa" else None
    ws = dsa.workspace(dsa.WS_LAYER_DSA if kind == "dsa" else dsa.WS_LAYER_SWA, T, pos0 + T,
                       top_k if kind == "dsa" else window)
    dsa.dsa_layer_step(cfg, w, cache, x, xo, T, pos0, idx_out=idx, qkv_out=qkv, ws=ws)
    torch.cuda.synchronize()
    out = {"x_out": bf16_bits(xo), "qkv": bf16_bits(qkv), "k": bf16_bits(kc), "v": bf16_bits(vc),
           "dev": {"qkv": qkv, "k": kc, "v": vc, "idx": idx}}
    if kind == "dsa":
        out["idx"] = down(idx)
        out["k_idx"] = down(ki)
        out["k_idx_scale"] = down(ks)
    return out


def _gpu_attention(dsa, g, T, L, top_k, sink=None):
    """The layer's attention output as the standalone call computes it on the step's own
    rotated queries, cache and indices (bf16 bits [T][1024])."""
    d = g["dev"]
    att = torch.zeros((T, 1024), dtype=torch.int16, device=DEV)
    ws = dsa.workspace(dsa.WS_SPARSE_ATTN, T, L, top_k)
    dsa.dsa_sparse_attn(d["qkv"][:, :1024].contiguous(), d["k"], d["v"], None, None, dsa.BF16, d["idx"], top_k, T,
                        L, 1 / math.sqrt(128), sink, att, dsa.BF16, ws)
    torch.cuda.synchronize()
    return bf16_bits(att)


def _check_dsa_output(dsa, g, lay, x, T, pos0, top_k, sink=None, w8=None):
    """Tight check of the DSA layer's output: teacher-forced oracle fed the GPU's rotated
    projection, indices and attention output; one bf16 ulp + 2^-16 * sum |terms|."""
    L = pos0 + T
    att = _gpu_attention(dsa, g, T, L, top_k, sink)
    cache = {"k": lay.k.copy(), "v": lay.v.copy(), "k_idx": lay.k_idx.copy(), "k_idx_scale": lay.k_idx_scale.copy()}
    kw = dict(top_k=top_k)
    wq, wo = lay.w_qkvi, lay.w_o
    if w8 is not None:
        wq, wo = w8[0], w8[2]
        kw.update(w_qkvi_scale=w8[1], w_o_scale=w8[3])
        wo_deq = O.decode_e4m3(w8[2]) * np.asarray(w8[3], np.float64)[:, None]
    else:
        wo_deq = O.decode_bf16(lay.w_o)
    tf = O.layer_step("dsa", x, lay.gamma, wq, wo, cache, pos0, teacher={"qkv": g["qkv"], "idx": g["idx"], "attn": att},
                      **kw)
    check_oproj(O.decode_bf16(g["x_out"]), tf["x_out_f64"], O.decode_bf16(att), wo_deq, O.decode_bf16(x))
    return tf


# one decoded token over a short context (4096 and 1500 keys): one selection workgroup
@pytest.mark.parametrize("L,T,top_k", [(3000, 8, 2048), (40000, 8, 2048), (777, 3, 64), (4096, 1, 2048),
                                       (1500, 1, 512)])
def test_dsa_layer_step_stages(dsa, L, T, top_k):
    pos0 = L - T
    lay = synth.layer_inputs("dsa", 0, L, T, seed=L)
    x = synth.module_x(L, T)
    g = _run_layer(dsa, "dsa", lay, x, T, pos0, top_k=top_k)
    # free-running oracle for the projection
    cache0 = {"k": lay.k.copy(), "v": lay.v.copy(), "k_idx": lay.k_idx.copy(), "k_idx_scale": lay.k_idx_scale.copy()}
    free = O.layer_step("dsa", x, lay.gamma, lay.w_qkvi, lay.w_o, cache0, pos0, top_k=top_k)
    gq = O.decode_bf16(g["qkv"])
    ok = _within_ulp(gq, free["qkv"])
    assert ok.mean() == 1.0, f"{(~ok).sum()} projection values beyond one bf16 ulp"
    # teacher-forced oracle
    cache = {"k": lay.k.copy(), "v": lay.v.copy(), "k_idx": lay.k_idx.copy(), "k_idx_scale": lay.k_idx_scale.copy()}
    tf = O.layer_step("dsa", x, lay.gamma, lay.w_qkvi, lay.w_o, cache, pos0, top_k=top_k,
                      teacher={"qkv": g["qkv"], "idx": g["idx"]})
    # appended rows
    assert np.array_equal(g["k"][pos0:L], g["qkv"][:, 1024:1152])
    assert np.array_equal(g["v"][pos0:L], g["qkv"][:, 1152:1280])
    assert np.array_equal(g["k_idx"][pos0:L], cache["k_idx"][pos0:L])
    assert np.array_equal(g["k_idx_scale"][pos0:L], cache["k_idx_scale"][pos0:L])
    # untouched rows stay untouched
    assert np.array_equal(g["k"][:pos0], lay.k[:pos0]) and np.array_equal(g["k_idx"][:pos0], lay.k_idx[:pos0])
    # selection vs the fp64 scores of the same rotated queries and cache
    krows = O.dequant_rows(cache["k_idx"][:L], "fp8", cache["k_idx_scale"][:L])
    qi = O.decode_bf16(g["qkv"][:, 1280:2304]).reshape(T, 16, 64)
    wi = O.decode_bf16(g["qkv"][:, 2368:2384])
    r, S = O.indexer_scores(qi, wi, krows, pos0, with_abs=True)
    ridx, _ = O.topk_indices(r, pos0, top_k)
    okb, nd = tie_band_ok(g["idx"], ridx, r, S, pos0, top_k)
    assert okb, nd
    # layer output: tight against the teacher-forced oracle on the GPU's attention output,
    # loose against the free-running oracle (whose selection may differ inside the band)
    _check_dsa_output(dsa, g, lay, x, T, pos0, top_k)
    gx = O.decode_bf16(g["x_out"])
    for ref in (tf["x_out"], free["x_out"]):
        assert np.all(np.abs(gx - ref) <= 2e-2 * np.maximum(1.0, np.abs(ref)))


# windows up to 153 run attention inside the output projection (W + T - 1 <= 160 rows);
# 200 takes the separate attention launch
@pytest.mark.parametrize("pos0,T,window", [(5000, 8, 128), (100, 8, 128), (0, 1, 128), (3, 5, 128),
                                           (5000, 8, 153), (5000, 8, 200), (20, 8, 200), ((1 << 20) - 8, 8, 128)])
def test_swa_layer_step_stages(dsa, pos0, T, window):
    cap = 256
    L = pos0 + T
    lay = synth.layer_inputs("swa", 1, L, T, seed=7, ring_cap=cap)
    x = synth.module_x(7, T)
    g = _run_layer(dsa, "swa", lay, x, T, pos0, window=window)
    c0 = {"k": lay.k.copy(), "v": lay.v.copy(), "ring_cap": cap}
    free = O.layer_step("swa", x, lay.gamma, lay.w_qkvi, lay.w_o, c0, pos0, window=window)
    assert _within_ulp(O.decode_bf16(g["qkv"]), free["qkv"], "swa").all()
    c1 = {"k": lay.k.copy(), "v": lay.v.copy(), "ring_cap": cap}
    tf = O.layer_step("swa", x, lay.gamma, lay.w_qkvi, lay.w_o, c1, pos0, window=window,
                      teacher={"qkv": g["qkv"]})
    for t in range(T):
        assert np.array_equal(g["k"][(pos0 + t) % cap], g["qkv"][t, 1024:1152])
    gx = O.decode_bf16(g["x_out"])
    for ref in (tf["x_out"], free["x_out"]):
        assert np.all(np.abs(gx - ref) <= 2e-2 * np.maximum(1.0, np.abs(ref)))
    # teacher-forced: the oracle's attention (fp64, rounded to bf16) and projection on the
    # GPU's own rotated q/k/v; the GPU differs by fp32 accumulation and rare bf16 rounding
    # flips of the attention output: two bf16 ulps of the result
    assert np.all(np.abs(gx - tf["x_out"]) <= 2.0 ** -7 * np.maximum(np.abs(tf["x_out"]), 1 / 16))


def test_swa_layer_step_with_sink_matches_oracle_attention(dsa):
    """Sink logits through the fused window attention: the oracle's window attention with
    the sink on the GPU's rotated q/k/v, rounded to bf16, projected, plus the residual."""
    pos0, T, window, cap = 3000, 8, 128, 256
    L = pos0 + T
    lay = synth.layer_inputs("swa", 1, L, T, seed=17, ring_cap=cap)
    x = synth.module_x(17, T)
    sink = synth.sink_logits(17, std=2.0)
    g = _run_layer(dsa, "swa", lay, x, T, pos0, window=window, sink=up(sink))
    q = O.decode_bf16(g["qkv"][:, :1024]).reshape(T, 8, 128)
    attn = O.swa_attention(q, O.decode_bf16(g["k"]), O.decode_bf16(g["v"]), cap, pos0, window,
                           1 / math.sqrt(128), sink.astype(np.float64))
    attn = O.bf16_round_trip(attn.reshape(T, 1024))
    ref = O.bf16_round_trip(O.project(attn, O.decode_bf16(lay.w_o)) + O.decode_bf16(x))
    gx = O.decode_bf16(g["x_out"])
    assert np.all(np.abs(gx - ref) <= 2.0 ** -7 * np.maximum(np.abs(ref), 1 / 16))


def test_layer_step_run_to_run_bitwise(dsa):
    L, T = 20000, 8
    lay = synth.layer_inputs("dsa", 0, L, T, seed=11)
    x = synth.module_x(11, T)
    a = _run_layer(dsa, "dsa", lay, x, T, L - T)
    for _ in range(2):
        b = _run_layer(dsa, "dsa", lay, x, T, L - T)
        for key in a:
            if key != "dev":
                assert np.array_equal(a[key], b[key]), key


def test_layer_step_with_sink_matches_oracle_attention(dsa):
    """Sink logits through the layer: compare against the oracle fed the GPU's
    rotated projection and indices, attention recomputed with the sink."""
    L, T = 5000, 4
    lay = synth.layer_inputs("dsa", 0, L, T, seed=13)
    x = synth.module_x(13, T)
    sink = up(synth.sink_logits(13, std=2.0))
    g = _run_layer(dsa, "dsa", lay, x, T, L - T, sink=sink)
    q = O.decode_bf16(g["qkv"][:, :1024]).reshape(T, 8, 128)
    Kc = O.decode_bf16(g["k"][:L]); Vc = O.decode_bf16(g["v"][:L])
    attn = O.sparse_attention(q, Kc, Vc, g["idx"], 1 / math.sqrt(128), down(sink).astype(np.float64))
    attn = O.bf16_round_trip(attn.reshape(T, 1024))
    ref = O.project(attn, O.decode_bf16(lay.w_o)) + O.decode_bf16(x)
    gx = O.decode_bf16(g["x_out"])
    assert np.all(np.abs(gx - ref) <= 2e-2 * np.maximum(1.0, np.abs(ref)))
    # the GPU's own attention output with the sink (the standalone call on the step's
    # inputs): the oracle's attention with the sink within the attention tolerance, and
    # the output projection of it within one ulp + the accumulation bound
    att = _gpu_attention(dsa, g, T, L, 2048, sink)
    assert np.max(np.abs(O.decode_bf16(att) - attn)) <= 2e-2
    ref_t = O.project(O.decode_bf16(att), O.decode_bf16(lay.w_o)) + O.decode_bf16(x)
    check_oproj(gx, ref_t, O.decode_bf16(att), O.decode_bf16(lay.w_o), O.decode_bf16(x))


@pytest.mark.parametrize("kind,L,T", [("dsa", 40000, 8), ("swa", 3000, 8), ("dsa", 777, 3)])
def test_layer_step_graph_replays_match_direct_launch(dsa, kind, L, T):
    """The layer step captured in a HIP graph: every replay, with the program's own eager
    work and synchronisations between replays, reproduces the direct launch bit for bit."""
    top_k = 2048 if L > 2048 else 64
    lay = synth.layer_inputs(kind, 0, L, T, seed=17)
    x_bits = synth.module_x(17, T)
    pos0 = L - T
    ref = _run_layer(dsa, kind, lay, x_bits, T, pos0, top_k=top_k)

    n_proj = synth.N_PROJ_DSA if kind == "dsa" else synth.N_PROJ_SWA
    cfg = dsa.layer_config(dsa.LAYER_DSA if kind == "dsa" else dsa.LAYER_SWA, top_k=top_k, window=128)
    g_gamma, g_w, g_wo = up(lay.gamma), up(lay.w_qkvi), up(lay.w_o)
    kc, vc = up(lay.k), up(lay.v)
    ki = up(lay.k_idx) if kind == "dsa" else None
    ks = up(lay.k_idx_scale) if kind == "dsa" else None
    cache = dsa.LayerCache(kc.data_ptr(), vc.data_ptr(), ki.data_ptr() if ki is not None else None,
                           ks.data_ptr() if ks is not None else None, lay.capacity)
    w = dsa.LayerWeights(g_gamma.data_ptr(), g_w.data_ptr(), g_wo.data_ptr())
    x = up(x_bits)
    xo = torch.zeros_like(x)
    qkv = torch.zeros((T, n_proj), dtype=torch.int16, device=DEV)
    idx = torch.full((T, top_k), -7, dtype=torch.int32, device=DEV) if kind == "dsa" else None
    ws = dsa.workspace(dsa.WS_LAYER_DSA if kind == "dsa" else dsa.WS_LAYER_SWA, T, L,
                       top_k if kind == "dsa" else 128)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(g, stream=side):
        dsa.dsa_layer_step(cfg, w, cache, x, xo, T, pos0, idx_out=idx, qkv_out=qkv, ws=ws,
                           stream=torch.cuda.current_stream())
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for rep in range(3):
        # eager work between replays: clear the outputs and run an unrelated reduction
        xo.zero_()
        qkv.zero_()
        if idx is not None:
            idx.fill_(-7)
        _ = (x.float() * 1.5).sum().item()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = {"x_out": bf16_bits(xo), "qkv": bf16_bits(qkv), "k": bf16_bits(kc), "v": bf16_bits(vc)}
        if kind == "dsa":
            got["idx"] = down(idx)
            got["k_idx"] = down(ki)
            got["k_idx_scale"] = down(ks)
        for key in got:
            assert np.array_equal(got[key], ref[key]), (rep, key)


@pytest.mark.parametrize("w8a8", [False, True])
def test_dsa_layer_step_full_context(dsa, w8a8):
    """The DSA layer step at the benchmark's size (L = 2^20, T = 8, top-2048): the projection
    and RoPE at positions 2^20 - 8 .. 2^20 - 1 against the free-running oracle, appended rows
    bitwise, the selection within the score band of the fp64 scores of the GPU's own rotated
    queries over the updated cache, and the output against the teacher-forced oracle fed the
    GPU's own attention output (one ulp + the accumulation bound)."""
    L, T, top_k = 1 << 20, 8, 2048
    pos0 = L - T
    lay = synth.layer_inputs("dsa", 5, L, T, seed=21)
    x = synth.module_x(21, T)
    w8 = synth.w8a8_weights(lay) if w8a8 else None
    g = _run_layer(dsa, "dsa", lay, x, T, pos0, top_k=top_k, w8=w8)
    kw = dict(top_k=top_k)
    wq, wo = lay.w_qkvi, lay.w_o
    if w8a8:
        wq, wo = w8[0], w8[2]
        kw.update(w_qkvi_scale=w8[1], w_o_scale=w8[3])
    cache = {"k": lay.k.copy(), "v": lay.v.copy(), "k_idx": lay.k_idx.copy(), "k_idx_scale": lay.k_idx_scale.copy()}
    tf = O.layer_step("dsa", x, lay.gamma, wq, wo, cache, pos0, teacher={"qkv": g["qkv"], "idx": g["idx"]}, **kw)
    # tf["qkv"] is the oracle's own (free-running) projection + RoPE at these positions
    if w8a8:
        from tests.test_gpu_w8a8 import _proj_ok
        _proj_ok(O.decode_bf16(g["qkv"]), tf["qkv"], tf["normed"], w8[0], w8[1], "dsa")
    else:
        okq = _within_ulp(O.decode_bf16(g["qkv"]), tf["qkv"])
        assert okq.all(), f"{(~okq).sum()} projection values beyond tolerance at 1M positions"
    assert np.array_equal(g["k"][pos0:L], g["qkv"][:, 1024:1152])
    assert np.array_equal(g["v"][pos0:L], g["qkv"][:, 1152:1280])
    assert np.array_equal(g["k_idx"][pos0:L], cache["k_idx"][pos0:L])
    assert np.array_equal(g["k_idx_scale"][pos0:L], cache["k_idx_scale"][pos0:L])
    krows = O.dequant_rows(cache["k_idx"][:L], "fp8", cache["k_idx_scale"][:L])
    qi = O.decode_bf16(g["qkv"][:, 1280:2304]).reshape(T, 16, 64)
    wi = O.decode_bf16(g["qkv"][:, 2368:2384])
    r, S = O.indexer_scores(qi, wi, krows, pos0, with_abs=True)
    ridx, _ = O.topk_indices(r, pos0, top_k)
    okb, nd = tie_band_ok(g["idx"], ridx, r, S, pos0, top_k)
    assert okb, nd
    gx = O.decode_bf16(g["x_out"])
    assert np.all(np.abs(gx - tf["x_out"]) <= 2e-2 * np.maximum(1.0, np.abs(tf["x_out"])))
    _check_dsa_output(dsa, g, lay, x, T, pos0, top_k, w8=w8)


@pytest.mark.parametrize("L,T,top_k,w8a8,sink", [(3000, 8, 2048, False, False), (40000, 8, 2048, True, False),
                                                 (777, 3, 64, False, True), (20000, 1, 2048, False, False),
                                                 (5000, 5, 300, True, True), (9000, 8, 2048, False, True),
                                                 (1 << 20, 8, 2048, False, True), (1 << 20, 8, 2048, True, False),
                                                 (2500, 1, 1024, False, True)])
def test_persistent_tail_equals_five_launch_composition(dsa, monkeypatch, L, T, top_k, w8a8, sink):
    """The DSA layer with one persistent launch after the selection (attention, split
    merge, output projection; DSA_LAYER_PERSISTENT_TAIL=1) equals the five-launch chain bit
    for bit: outputs, indices, the exported projection and every cache row."""
    lay = synth.layer_inputs("dsa", 0, L, T, seed=L + T)
    x = synth.module_x(L + T, T)
    w8 = synth.w8a8_weights(lay) if w8a8 else None
    sk = up(synth.sink_logits(L, std=2.0)) if sink else None
    monkeypatch.setenv("DSA_LAYER_PERSISTENT_TAIL", "1")
    a = _run_layer(dsa, "dsa", lay, x, T, L - T, top_k=top_k, sink=sk, w8=w8)
    monkeypatch.delenv("DSA_LAYER_PERSISTENT_TAIL")
    b = _run_layer(dsa, "dsa", lay, x, T, L - T, top_k=top_k, sink=sk, w8=w8)
    for key in ("x_out", "qkv", "idx", "k", "v", "k_idx", "k_idx_scale"):
        assert np.array_equal(a[key], b[key]), key
    assert np.all((a["idx"] >= 0).sum(axis=1) == np.minimum(top_k, np.arange(L - T + 1, L + 1)))
