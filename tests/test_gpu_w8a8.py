"""W8A8 dsa_layer_step on the GPU against the oracle's W8A8 layer step.

Inputs: exact-norm residual rows (eps = 0 and a power-of-4 mean square make the RMS
factor an exact power of two), a random RMSNorm gain and the layer's weights stored as
e4m3 codes with per-row scales.  The normalised rows are then identical on both sides,
so the per-token activation codes are identical and the projection differs only by the
fp32 accumulation: one bf16 ulp plus 2^-16 of the sum of absolute products.

Output projection: where the layer runs a separate attention launch (DSA layers, SWA
windows with W + T - 1 > 160) the standalone attention call on the same inputs gives
the GPU's attention output bit for bit, and the oracle's W8A8 output projection of it
must match to one bf16 ulp plus the fp32 accumulation bound.  Where the SWA window
attention is fused into the output projection, the GPU's attention output is not
visible: attention elements whose bf16 rounding the GPU's arithmetic could flip (fp64
value within 2^-14 * sum_j p_j |v_j| of a rounding midpoint) get the full code-flip
allowance, and a token whose largest magnitude is such an element gets it everywhere.
"""
import math

import numpy as np
import pytest
import torch

import synth
from oracle import dsa_oracle as O
from tests.gpu_util import DEV, up, down, bf16_bits, tie_band_ok, check_oproj
from tests.test_gpu_layer import _run_layer, _within_ulp

pytestmark = pytest.mark.gpu
SM = 1.0 / math.sqrt(128)


@pytest.fixture(scope="module")
def dsa():
    import sparse_attention_decode_indexer_amd as m
    return m


def _wdeq(codes, scale):
    return O.decode_e4m3(codes) * np.asarray(scale, np.float64)[:, None]


def _proj_ok(gq, rq, y, w_codes, w_scale, kind):
    """Projection after RoPE: the one-ulp rule of the bf16 test plus the fp32 accumulation
    bound 2^-16 * sum_k |a_k b_k| s_y s_w (rotation pairs: the sum over both inputs)."""
    codes, s = O.quantize_tokens_w8a8(y)
    S = O.project(np.abs(O.decode_e4m3(codes)) * s[:, None].astype(np.float64), np.abs(_wdeq(w_codes, w_scale)))
    segs = [(0, 1024, 128), (1024, 128, 128)] + ([(1280, 1024, 64), (2304, 64, 64)] if kind == "dsa" else [])
    for off, n, d in segs:
        blk = S[:, off:off + n].reshape(S.shape[0], -1, d)
        pair = blk[..., : d // 2] + blk[..., d // 2:]
        S[:, off:off + n] = np.concatenate([pair, pair], axis=-1).reshape(S.shape[0], n)
    ok = _within_ulp(gq, rq, kind) | (np.abs(gq - rq) <= 2.0 ** -7 * np.abs(rq) + 2.0 ** -16 * S)
    if not ok.all():
        t, c = np.argwhere(~ok)[0]
        raise AssertionError(f"{(~ok).sum()} projection values beyond tolerance; first [{t},{c}]: gpu {gq[t, c]!r} "
                             f"oracle {rq[t, c]!r} sum|terms| {S[t, c]!r}")


_check_oproj = check_oproj


@pytest.mark.parametrize("L,T,top_k", [(3000, 8, 2048), (40000, 8, 2048), (777, 3, 64)])
def test_w8a8_dsa_layer_step(dsa, L, T, top_k):
    pos0 = L - T
    lay = synth.layer_inputs("dsa", 0, L, T, seed=L + 1)
    w8 = synth.w8a8_weights(lay)
    x = synth.exact_norm_x(L, T)
    gamma = synth.random_gamma(L)
    g = _run_layer(dsa, "dsa", lay, x, T, pos0, top_k=top_k, eps=0.0, gamma=gamma, w8=w8)
    kw = dict(eps=0.0, top_k=top_k, w_qkvi_scale=w8[1], w_o_scale=w8[3])
    c0 = {"k": lay.k.copy(), "v": lay.v.copy(), "k_idx": lay.k_idx.copy(), "k_idx_scale": lay.k_idx_scale.copy()}
    free = O.layer_step("dsa", x, gamma, w8[0], w8[2], c0, pos0, **kw)
    _proj_ok(O.decode_bf16(g["qkv"]), free["qkv"], free["normed"], w8[0], w8[1], "dsa")
    # the GPU's attention output: the standalone call on the step's own queries, cache and indices
    d = g["dev"]
    att = torch.zeros((T, 1024), dtype=torch.int16, device=DEV)
    ws = dsa.workspace(dsa.WS_SPARSE_ATTN, T, L, top_k)
    dsa.dsa_sparse_attn(d["qkv"][:, :1024].contiguous(), d["k"], d["v"], None, None, dsa.BF16, d["idx"], top_k, T,
                        L, SM, None, att, dsa.BF16, ws)
    torch.cuda.synchronize()
    att_bits = bf16_bits(att)
    c1 = {"k": lay.k.copy(), "v": lay.v.copy(), "k_idx": lay.k_idx.copy(), "k_idx_scale": lay.k_idx_scale.copy()}
    tf = O.layer_step("dsa", x, gamma, w8[0], w8[2], c1, pos0,
                      teacher={"qkv": g["qkv"], "idx": g["idx"], "attn": att_bits}, **kw)
    # appended rows and the indexer-key quantisation of the exported rows
    assert np.array_equal(g["k"][pos0:L], g["qkv"][:, 1024:1152])
    assert np.array_equal(g["k_idx"][pos0:L], c1["k_idx"][pos0:L])
    # selection vs the fp64 scores of the GPU's rotated queries over the updated cache
    krows = O.dequant_rows(c1["k_idx"][:L], "fp8", c1["k_idx_scale"][:L])
    qi = O.decode_bf16(g["qkv"][:, 1280:2304]).reshape(T, 16, 64)
    wi = O.decode_bf16(g["qkv"][:, 2368:2384])
    r, S = O.indexer_scores(qi, wi, krows, pos0, with_abs=True)
    ridx, _ = O.topk_indices(r, pos0, top_k)
    okb, nd = tie_band_ok(g["idx"], ridx, r, S, pos0, top_k)
    assert okb, nd
    _check_oproj(O.decode_bf16(g["x_out"]), tf["x_out_f64"], O.decode_bf16(att_bits), _wdeq(w8[2], w8[3]),
                 O.decode_bf16(x))


def _fused_allowance(q, Kr, Vr, cap, pos0, window, wo_deq):
    """Code-flip allowance [T][4096] for the fused SWA output projection (module doc)."""
    o64 = O.swa_attention(q, Kr, Vr, cap, pos0, window, SM).reshape(q.shape[0], -1)
    pv = O.swa_attention(q, Kr, np.abs(Vr), cap, pos0, window, SM).reshape(q.shape[0], -1)
    delta = 2.0 ** -14 * pv
    lo, hi = O.bf16_round_trip(o64 - delta), O.bf16_round_trip(o64 + delta)
    amb = lo != hi
    mag_hi = np.maximum(np.abs(lo), np.abs(hi))
    mag_lo = np.minimum(np.abs(lo), np.abs(hi))
    am_hi = mag_hi.max(axis=1)
    am_lo = np.where(amb, mag_lo, mag_hi).max(axis=1)
    amb_tok = am_hi != am_lo
    s = am_hi / 448.0
    term = np.abs(hi - lo) + 2.0 * ((2.0 ** -4 + 2.0 ** -22) * mag_hi + 2.0 ** -10 * s[:, None])
    mask = np.where(amb_tok[:, None], True, amb)
    return O.project(np.where(mask, term, 0.0), np.abs(wo_deq)), int(amb.sum()), int(amb_tok.sum())


@pytest.mark.parametrize("pos0,T,window", [(5000, 8, 128), (3, 5, 128), (0, 1, 128), (5000, 8, 200), (20, 8, 200)])
def test_w8a8_swa_layer_step(dsa, pos0, T, window):
    cap = 256
    L = pos0 + T
    lay = synth.layer_inputs("swa", 1, L, T, seed=9, ring_cap=cap)
    w8 = synth.w8a8_weights(lay)
    x = synth.exact_norm_x(pos0 + 11, T)
    gamma = synth.random_gamma(pos0 + 11)
    g = _run_layer(dsa, "swa", lay, x, T, pos0, window=window, eps=0.0, gamma=gamma, w8=w8)
    kw = dict(eps=0.0, window=window, w_qkvi_scale=w8[1], w_o_scale=w8[3])
    free = O.layer_step("swa", x, gamma, w8[0], w8[2], {"k": lay.k.copy(), "v": lay.v.copy(), "ring_cap": cap},
                        pos0, **kw)
    _proj_ok(O.decode_bf16(g["qkv"]), free["qkv"], free["normed"], w8[0], w8[1], "swa")
    for t in range(T):
        assert np.array_equal(g["k"][(pos0 + t) % cap], g["qkv"][t, 1024:1152])
    wo_deq = _wdeq(w8[2], w8[3])
    c1 = {"k": lay.k.copy(), "v": lay.v.copy(), "ring_cap": cap}
    if window + T - 1 > 160:
        # separate attention launch: the standalone call reproduces its output
        d = g["dev"]
        att = torch.zeros((T, 1024), dtype=torch.int16, device=DEV)
        ws = dsa.workspace(dsa.WS_SWA_ATTN, T, L, window)
        dsa.swa_attn(d["qkv"][:, :1024].contiguous(), d["k"], d["v"], None, None, dsa.BF16, cap, T, pos0, window,
                     SM, None, att, dsa.BF16, ws)
        torch.cuda.synchronize()
        att_bits = bf16_bits(att)
        tf = O.layer_step("swa", x, gamma, w8[0], w8[2], c1, pos0, teacher={"qkv": g["qkv"], "attn": att_bits}, **kw)
        _check_oproj(O.decode_bf16(g["x_out"]), tf["x_out_f64"], O.decode_bf16(att_bits), wo_deq, O.decode_bf16(x))
    else:
        tf = O.layer_step("swa", x, gamma, w8[0], w8[2], c1, pos0, teacher={"qkv": g["qkv"]}, **kw)
        q = O.decode_bf16(g["qkv"][:, :1024]).reshape(T, 8, 128)
        allow, n_amb, n_tok = _fused_allowance(q, O.decode_bf16(c1["k"]), O.decode_bf16(c1["v"]), cap, pos0, window,
                                               wo_deq)
        print(f"ambiguous attention elements {n_amb}, tokens with an ambiguous maximum {n_tok}")
        _check_oproj(O.decode_bf16(g["x_out"]), tf["x_out_f64"], tf["attn"], wo_deq, O.decode_bf16(x), allow)


def test_w8a8_layer_step_run_to_run_bitwise(dsa):
    L, T = 20000, 8
    lay = synth.layer_inputs("dsa", 0, L, T, seed=12)
    w8 = synth.w8a8_weights(lay)
    x = synth.module_x(12, T)
    a = _run_layer(dsa, "dsa", lay, x, T, L - T, w8=w8)
    for _ in range(2):
        b = _run_layer(dsa, "dsa", lay, x, T, L - T, w8=w8)
        for key in ("x_out", "qkv", "idx", "k_idx"):
            assert np.array_equal(a[key], b[key]), key


def test_w8a8_free_running_module_inputs_within_quantiser_bound(dsa):
    """The module's own inputs (gamma = 1, eps = 1e-6, x ~ N(0,1)): the GPU's normalised
    rows may differ from the oracle's in the last bf16 bit, so codes may differ; the
    projection must still lie within the quantiser's error bound of the exact product."""
    L, T = 5000, 8
    pos0 = L - T
    lay = synth.layer_inputs("dsa", 0, L, T, seed=13)
    w8 = synth.w8a8_weights(lay)
    x = synth.module_x(13, T)
    g = _run_layer(dsa, "dsa", lay, x, T, pos0, top_k=2048, w8=w8)
    c0 = {"k": lay.k.copy(), "v": lay.v.copy(), "k_idx": lay.k_idx.copy(), "k_idx_scale": lay.k_idx_scale.copy()}
    free = O.layer_step("dsa", x, lay.gamma, w8[0], w8[2], c0, pos0, w_qkvi_scale=w8[1], w_o_scale=w8[3])
    # pre-RoPE bound on |P_gpu - P_oracle|: both are within the quantiser bound of y . W
    y = free["normed"]
    wq = _wdeq(w8[0], w8[1])
    _, s = O.quantize_tokens_w8a8(y)
    qb = O.project((2.0 ** -4 + 2.0 ** -22) * np.abs(y) + 2.0 ** -10 * s[:, None].astype(np.float64), np.abs(wq))
    ynb = O.project(2.0 ** -8 * np.abs(y), np.abs(wq))          # one-ulp differences of y
    gq, rq = O.decode_bf16(g["qkv"]), free["qkv"]
    # rotated columns mix pairs: bound by the pair's combined bound
    bound = 2.0 * qb + ynb
    for off, n, d in [(0, 1024, 128), (1024, 128, 128), (1280, 1024, 64), (2304, 64, 64)]:
        blk = bound[:, off:off + n].reshape(T, -1, d)
        pair = blk[..., : d // 2] + blk[..., d // 2:]
        bound[:, off:off + n] = np.concatenate([pair, pair], axis=-1).reshape(T, n)
    tol = bound + 2.0 ** -7 * np.abs(rq) + 2.0 ** -7 * np.abs(gq)
    assert np.all(np.abs(gq - rq) <= tol)
