"""dsa_module_step on the GPU: a run of decoder layers in one call.

* Against the same layers called one dsa_layer_step at a time: the module's x_out, the
  last DSA layer's selection and every layer's cache or ring after the step are equal bit
  for bit, both for the default path (the layer steps enqueued back to back) and with
  DSA_MODULE_CHAIN=1 (runs of SWA layers through the persistent multi-layer launch; a run
  longer than eight layers split over launches; DSA and W8A8 layers take the layer step).
* Against the oracle's free-running composition of the layers (module_step): the module
  output within 2e-2 * max(1, |ref|) per element and 1e-2 relative in norm -- each layer
  adds fp32-accumulation and bf16-rounding differences that the next layer carries on.
* Two calls in a row on one workspace (the launch counter advances), the co-residency
  fallback (the same bits), and the workspace status.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import dsa_oracle as O
from tests.gpu_util import DEV, up, bf16_bits, down

pytestmark = pytest.mark.gpu

CAP = 256


@pytest.fixture(scope="module")
def dsa():
    import sparse_attention_decode_indexer_amd as m
    return m


@pytest.fixture
def chain(monkeypatch):
    """The persistent multi-layer SWA launch for the module calls of the test."""
    monkeypatch.setenv("DSA_MODULE_CHAIN", "1")


def _host_layers(kinds, L, T, seed, w8a8=()):
    lays = []
    for i, kind in enumerate(kinds):
        lay = synth.layer_inputs(kind, i, L, T, seed=seed, ring_cap=CAP)
        lays.append((lay, synth.w8a8_weights(lay) if i in w8a8 else None))
    return lays


class _Dev:
    """Device copies of the layers (fresh caches on every construction)."""

    def __init__(self, dsa, kinds, host, top_k, window, sinks=None):
        self.keep, self.cfgs, self.ws, self.caches, self.tensors = [], [], [], [], []
        for i, (kind, (lay, w8)) in enumerate(zip(kinds, host)):
            sink = None if sinks is None or sinks[i] is None else up(sinks[i])
            cfg = dsa.layer_config(dsa.LAYER_DSA if kind == "dsa" else dsa.LAYER_SWA, top_k=top_k, window=window,
                                   sink=sink)
            g = up(lay.gamma)
            if w8 is None:
                wq, wo = up(lay.w_qkvi), up(lay.w_o)
                w = dsa.LayerWeights(g.data_ptr(), wq.data_ptr(), wo.data_ptr())
                extra = (wq, wo)
            else:
                wq, sq, wo, so = (up(a) for a in w8)
                w = dsa.LayerWeights(g.data_ptr(), wq.data_ptr(), wo.data_ptr(), dsa.FP8_E4M3, sq.data_ptr(),
                                     so.data_ptr())
                extra = (wq, sq, wo, so)
            kc, vc = up(lay.k), up(lay.v)
            ki = up(lay.k_idx) if kind == "dsa" else None
            ks = up(lay.k_idx_scale) if kind == "dsa" else None
            c = dsa.LayerCache(kc.data_ptr(), vc.data_ptr(), ki.data_ptr() if ki is not None else None,
                               ks.data_ptr() if ks is not None else None, lay.capacity)
            self.keep += [sink, g, kc, vc, ki, ks, *extra]
            self.cfgs.append(cfg)
            self.ws.append(w)
            self.caches.append(c)
            self.tensors.append((kc, vc, ki, ks))

    def cache_bits(self):
        out = []
        for kc, vc, ki, ks in self.tensors:
            out.append([bf16_bits(kc), bf16_bits(vc)] + ([down(ki), down(ks)] if ki is not None else []))
        return out


def _module(dsa, kinds, host, x_bits, T, pos0, top_k, window, sinks=None, per_layer=False, ws=None):
    d = _Dev(dsa, kinds, host, top_k, window, sinks)
    x = up(x_bits)
    xo = torch.zeros_like(x)
    has_dsa = "dsa" in kinds
    idx = torch.full((T, top_k), -7, dtype=torch.int32, device=DEV) if has_dsa else None
    L = pos0 + T
    if per_layer:
        xin = x
        last = max(i for i, k in enumerate(kinds) if k == "dsa") if has_dsa else -1
        for i, kind in enumerate(kinds):
            out = xo if i == len(kinds) - 1 else torch.zeros_like(x)
            lws = dsa.workspace(dsa.WS_LAYER_DSA if kind == "dsa" else dsa.WS_LAYER_SWA, T, L,
                                top_k if kind == "dsa" else window)
            dsa.dsa_layer_step(d.cfgs[i], d.ws[i], d.caches[i], xin, out, T, pos0,
                               idx_out=idx if i == last else None, ws=lws)
            xin = out
    else:
        if ws is None:
            ws = dsa.workspace(dsa.WS_MODULE, T, L, top_k if has_dsa else 0)
        dsa.dsa_module_step(d.cfgs, d.ws, d.caches, x, xo, T, pos0, idx_out=idx, ws=ws)
        assert dsa.dsa_workspace_status(ws) == 0
    torch.cuda.synchronize()
    return {"x_out": bf16_bits(xo), "idx": down(idx) if has_dsa else None, "caches": d.cache_bits()}


def _assert_same(a, b):
    assert np.array_equal(a["x_out"], b["x_out"])
    if a["idx"] is not None:
        assert np.array_equal(a["idx"], b["idx"])
    for ca, cb in zip(a["caches"], b["caches"]):
        for u, v in zip(ca, cb):
            assert np.array_equal(u, v)


MODULE = ("swa",) * 5 + ("dsa",)


@pytest.mark.parametrize("kinds,L,T,top_k,window", [
    (MODULE, 3000, 8, 2048, 128),                          # the module's layer mix
    (MODULE, 40000, 3, 64, 128),
    (("swa",) * 9, 500, 8, 2048, 128),                     # split over two launches (8 + 1)
    (("swa",), 1, 1, 2048, 128),                           # first token of the context
    (("swa", "swa"), 6, 5, 2048, 128),                     # window reaching before position 0
    (("swa", "dsa", "swa", "swa"), 2000, 8, 256, 128),     # runs of 1 and 2 around a DSA layer
    (("swa",) * 3, 1000, 8, 2048, 153),                    # the widest window one workgroup holds
    (("swa",) * 2, (1 << 20), 8, 2048, 128),               # positions near 2^20, ring wrap
    (("swa",) * 3, 700, 4, 2048, 60),
])
def test_module_equals_layer_by_layer(dsa, chain, kinds, L, T, top_k, window):
    pos0 = L - T
    host = _host_layers(kinds, L, T, seed=L + T)
    x = synth.module_x(L + 3, T)
    a = _module(dsa, kinds, host, x, T, pos0, top_k, window)
    b = _module(dsa, kinds, host, x, T, pos0, top_k, window, per_layer=True)
    _assert_same(a, b)


def test_module_with_sinks_and_w8a8_equals_layer_by_layer(dsa, chain):
    """Per-layer sinks (and none) through the chain; a W8A8 SWA layer breaks the run."""
    kinds = ("swa", "swa", "swa", "swa", "dsa")
    L, T = 2500, 8
    host = _host_layers(kinds, L, T, seed=31, w8a8=(2,))
    sinks = [synth.sink_logits(1, 2.0), None, synth.sink_logits(3, 1.0), None, synth.sink_logits(5, 1.0)]
    x = synth.module_x(31, T)
    a = _module(dsa, kinds, host, x, T, L - T, 2048, 128, sinks=sinks)
    b = _module(dsa, kinds, host, x, T, L - T, 2048, 128, sinks=sinks, per_layer=True)
    _assert_same(a, b)


def test_module_two_calls_on_one_workspace(dsa, chain):
    """The second call (new launch counter, same workspace, a smaller block) is again equal
    to the layer-by-layer result."""
    kinds = ("swa",) * 4
    ws = dsa.workspace(dsa.WS_MODULE, 8, 5000, 0)
    for T, L, seed in ((8, 5000, 1), (3, 4000, 2), (8, 4500, 3)):
        host = _host_layers(kinds, L, T, seed=seed)
        x = synth.module_x(seed, T)
        a = _module(dsa, kinds, host, x, T, L - T, 2048, 128, ws=ws)
        b = _module(dsa, kinds, host, x, T, L - T, 2048, 128, per_layer=True)
        _assert_same(a, b)


def test_module_without_co_residency_runs_layer_by_layer(dsa, chain, monkeypatch):
    """With fewer resident workgroups than the chain needs (the DSA_RESIDENT_LIMIT hook),
    the SWA layers run one layer step at a time: the same bits."""
    kinds = ("swa",) * 3
    L, T = 900, 8
    host = _host_layers(kinds, L, T, seed=41)
    x = synth.module_x(41, T)
    b = _module(dsa, kinds, host, x, T, L - T, 2048, 128, per_layer=True)
    monkeypatch.setenv("DSA_RESIDENT_LIMIT", "100")
    a = _module(dsa, kinds, host, x, T, L - T, 2048, 128)
    _assert_same(a, b)


@pytest.mark.parametrize("persistent", [False, True])
def test_default_module_equals_layer_by_layer(dsa, monkeypatch, persistent):
    """The default path (layer steps enqueued back to back, outputs ping-ponged in the
    workspace) on the module's layer mix; the persistent variant on the same inputs."""
    if persistent:
        monkeypatch.setenv("DSA_MODULE_CHAIN", "1")
    L, T = 5000, 8
    host = _host_layers(MODULE, L, T, seed=51)
    x = synth.module_x(51, T)
    a = _module(dsa, MODULE, host, x, T, L - T, 2048, 128)
    b = _module(dsa, MODULE, host, x, T, L - T, 2048, 128, per_layer=True)
    _assert_same(a, b)


@pytest.mark.parametrize("L,T,persistent", [(2000, 8, True), (300, 5, True), (2000, 8, False)])
def test_module_matches_oracle_composition(dsa, monkeypatch, L, T, persistent):
    """The module against the oracle's free-running composition of its six layers (top-k
    2048 >= L: the DSA layer attends its whole context, so its selection is unique)."""
    if persistent:
        monkeypatch.setenv("DSA_MODULE_CHAIN", "1")
    pos0 = L - T
    host = _host_layers(MODULE, L, T, seed=L)
    x = synth.module_x(L, T)
    g = _module(dsa, MODULE, host, x, T, pos0, 2048, 128)
    layers = []
    for kind, (lay, _) in zip(MODULE, host):
        cache = ({"k": lay.k.copy(), "v": lay.v.copy(), "k_idx": lay.k_idx.copy(),
                  "k_idx_scale": lay.k_idx_scale.copy()} if kind == "dsa"
                 else {"k": lay.k.copy(), "v": lay.v.copy(), "ring_cap": CAP})
        layers.append(dict(kind=kind, gamma=lay.gamma, w_qkvi=lay.w_qkvi, w_o=lay.w_o, cache=cache, top_k=2048))
    ref_bits, _ = O.module_step(layers, x, pos0)
    ref = O.decode_bf16(ref_bits)
    gx = O.decode_bf16(g["x_out"])
    assert np.all(np.abs(gx - ref) <= 2e-2 * np.maximum(1.0, np.abs(ref)))
    assert np.linalg.norm(gx - ref) <= 1e-2 * np.linalg.norm(ref)
    # every token's selection is its whole causal context
    for t in range(T):
        sel = g["idx"][t][g["idx"][t] >= 0]
        assert np.array_equal(np.sort(sel), np.arange(pos0 + t + 1))
