"""Pins of the CPU oracle against facts that do not come from the oracle itself:
hand-derived examples, exact integer arithmetic, library routines (PyTorch's
float8/bf16 casts, scaled_dot_product_attention, rms_norm), closed forms and
invariants.  CPU only."""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import dsa_oracle as O
import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------- formats

def test_e4m3_decode_all_codes_vs_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = O.decode_e4m3(codes)
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan], got[~nan])
    assert O.decode_e4m3(np.array([0x7E], np.uint8))[0] == 448.0
    assert O.decode_e4m3(np.array([0x01], np.uint8))[0] == 2.0 ** -9


def test_e4m3_encode_vs_torch_sweep_and_midpoints():
    g = np.random.default_rng(7)
    x = np.concatenate([
        g.standard_normal(20000).astype(np.float32) * 30,
        g.uniform(-448, 448, 20000).astype(np.float32),
        (g.standard_normal(5000) * 1e-3).astype(np.float32),
    ])
    mags = O.decode_e4m3(np.arange(127, dtype=np.uint8))
    mids = ((mags[:-1] + mags[1:]) / 2).astype(np.float32)    # exact in fp32
    x = np.concatenate([x, mids, -mids, mags.astype(np.float32)])
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = O.encode_e4m3(x)
    # torch maps -0.0 to 0x80 as well; compare everything
    assert np.array_equal(ref, got)


def test_e4m3_encode_saturates():
    x = np.array([448.0, 460.0, 1e4, 3e38, -500.0, -1e9], np.float32)
    got = O.encode_e4m3(x)
    assert list(got) == [0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE]


def test_bf16_decode_and_round_vs_torch():
    g = np.random.default_rng(3)
    x = (g.standard_normal(4000) * np.exp2(g.integers(-130, 100, 4000))).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(O.round_to_bf16(x.astype(np.float64)), ref)
    back = torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(O.decode_bf16(ref), back)


def test_bf16_round_is_single_rounding_from_fp64():
    # 1 + 2^-8 + 2^-30 lies above the midpoint between 1 and 1+2^-7; rounding
    # through fp32 first would land exactly on the midpoint and go to 1.0.
    v = 1.0 + 2.0 ** -8 + 2.0 ** -30
    assert O.round_to_bf16(np.array([v]))[0] == 0x3F81
    assert O.round_to_bf16(np.array([1.0 + 2.0 ** -8]))[0] == 0x3F80   # tie -> even
    assert O.round_to_bf16(np.array([-0.0]))[0] == 0x8000


# ----------------------------------------------------------------------------- indexer

def test_indexer_hand_example():
    g = json.load(open(os.path.join(GOLD, "indexer_topk_tiny.json")))
    s = O.indexer_scores(np.array(g["q"], float), np.array(g["w"], float),
                         np.array(g["k"], float), g["pos0"])
    assert np.array_equal(s, np.array(g["scores"]))
    idx, cnt = O.topk_indices(s, g["pos0"], 2)
    assert idx.tolist() == g["top2"] and cnt.tolist() == [2]
    idx, _ = O.topk_indices(s, g["pos0"], 3)
    assert idx.tolist() == g["top3"]


def test_indexer_integer_config_is_exact():
    """Integer q/k and w on a 1/256 grid: 256*I is an integer computed exactly in int64."""
    inp = synth.dsa_config("tiny", seed=1, L=512)
    q = O.decode_bf16(inp.q_idx)
    k = O.decode_bf16(inp.k_idx)
    w = inp.w_idx.astype(np.float64)
    s = O.indexer_scores(q, w, k, inp.pos0)
    qi = q.astype(np.int64)
    ki = k.astype(np.int64)
    wi = np.rint(w * 256).astype(np.int64)
    assert np.array_equal(wi, w * 256)
    d = np.einsum("thd,sd->ths", qi, ki)
    exact = np.einsum("th,ths->ts", wi, np.maximum(d, 0))
    assert np.array_equal(s * 256, exact.astype(np.float64))


def test_indexer_causal_mask_and_fp8_scale():
    T, L = 3, 40
    g = np.random.default_rng(5)
    q = g.standard_normal((T, 16, 64))
    w = g.random((T, 16))
    kf = g.standard_normal((L, 64)).astype(np.float32)
    codes, scale = synth.to_e4m3_rows(kf)
    rows = O.dequant_rows(codes, "fp8", scale)
    s = O.indexer_scores(q, w, rows, L - T)
    for t in range(T):
        assert np.all(np.isneginf(s[t, L - T + t + 1:]))
        assert np.all(np.isfinite(s[t, :L - T + t + 1]))
    # scaled rows: scale * (q . code) == q . (scale * code); a positive scale commutes with relu
    unscaled = O.indexer_scores(q, w, O.decode_e4m3(codes), L - T)
    vis = np.isfinite(s)
    np.testing.assert_allclose(s[vis], (unscaled * scale[None, :])[vis], rtol=1e-12)


def test_indexer_magnitude_hand_example():
    """The band magnitude S[t,s] = sum_h |w| sum_d |q k|, worked out by hand in the fixture."""
    g = json.load(open(os.path.join(GOLD, "indexer_topk_tiny.json")))
    s, S = O.indexer_scores(np.array(g["q"], float), np.array(g["w"], float),
                            np.array(g["k"], float), g["pos0"], with_abs=True)
    assert np.array_equal(S, np.array(g["magnitude"]))
    assert np.array_equal(s, np.array(g["scores"]))


def test_indexer_magnitude_invariants():
    """S ignores every sign (q, k, w, per head or per element), equals the score when every
    input is non-negative (relu and |.| are then the identity), bounds |I|, scales with |w|,
    and is 0 beyond the causal limit."""
    g = np.random.default_rng(31)
    T, H, D, L = 3, 16, 64, 50
    q = g.standard_normal((T, H, D))
    k = g.standard_normal((L, D))
    w = g.standard_normal((T, H))
    pos0 = L - T
    s, S = O.indexer_scores(q, w, k, pos0, with_abs=True)
    flips = np.where(g.random((T, H, D)) < 0.5, -1.0, 1.0)
    kflips = np.where(g.random((L, D)) < 0.5, -1.0, 1.0)
    for q2, k2, w2 in ((-q, k, w), (q * flips, k, w), (q, -k, w), (q, k * kflips, w), (q, k, -w),
                       (q * flips, k * kflips, -w)):
        _, S2 = O.indexer_scores(q2, w2, k2, pos0, with_abs=True)
        np.testing.assert_allclose(S2, S, rtol=1e-13, atol=0)
    vis = np.isfinite(s)
    assert np.all(np.abs(s[vis]) <= S[vis] * (1 + 1e-13))
    assert np.all(S[~vis] == 0)
    sp, Sp = O.indexer_scores(np.abs(q), np.abs(w), np.abs(k), pos0, with_abs=True)
    np.testing.assert_allclose(sp[vis], Sp[vis], rtol=1e-13)
    _, S3 = O.indexer_scores(q, 3.0 * w, k, pos0, with_abs=True)
    np.testing.assert_allclose(S3, 3.0 * S, rtol=1e-13)
    # per-head weights: S is linear in |w| head by head
    e = np.zeros((T, H)); e[:, 5] = 1.0
    _, S5 = O.indexer_scores(q, e, k, pos0, with_abs=True)
    ref5 = np.abs(q[:, 5, :]) @ np.abs(k).T
    np.testing.assert_allclose(S5[vis], ref5[vis], rtol=1e-13)


# ----------------------------------------------------------------------------- the indexer leg of the layer step

_LEG_T, _LEG_A, _LEG_SHIFT = 4, 3, 65539


def _zero_prefix_dsa(pos0, T, seed=41):
    """A DSA layer whose cache rows before pos0 are zero (indexer codes 0, scale 1)."""
    L = pos0 + T
    lay = synth.layer_inputs("dsa", 0, 64, T, seed=seed)          # weights only (they do not depend on L)
    cache = {"k": np.zeros((L, 128), np.uint16), "v": np.zeros((L, 128), np.uint16),
             "k_idx": np.zeros((L, 64), np.uint8), "k_idx_scale": np.ones(L, np.float32)}
    return lay, cache


@pytest.fixture(scope="module")
def indexer_leg():
    """The same block (inputs and weights) stepped at pos0 = A and at pos0 = A + shift over
    all-zero prefix caches."""
    T = _LEG_T
    x = synth.module_x(41, T)
    out = {}
    for pos0 in (_LEG_A, _LEG_A + _LEG_SHIFT):
        lay, cache = _zero_prefix_dsa(pos0, T)
        r = O.layer_step("dsa", x, lay.gamma, lay.w_qkvi, lay.w_o, cache, pos0, top_k=64)
        out[pos0] = (r, cache)
    return out


def _pairs(seg, d):
    """[T][n] -> complex [T][n/d][d/2]: rotate-half pairs (i, i + d/2) as a + ib."""
    b = seg.reshape(seg.shape[0], -1, d)
    return b[..., : d // 2] + 1j * b[..., d // 2:]


def test_layer_step_rotates_indexer_queries_and_keys_by_position(indexer_leg):
    """Rotate-half RoPE by absolute position on q_I and k_I (and Q, K): moving the block by
    `shift` positions multiplies every pair by exp(i * shift * theta^(-2j/d)) (within the
    bf16 roundings of both results); the indexer head weights w_I are not rotated (bit-equal
    at both positions); V is not rotated.  Fails if q_I or k_I is left unrotated, rotated by
    the in-block offset only, or if w_I is rotated."""
    A, B = _LEG_A, _LEG_A + _LEG_SHIFT
    ra, rb = indexer_leg[A][0], indexer_leg[B][0]
    lay = O.proj_layout("dsa")
    for name, d in (("q_idx", 64), ("k_idx", 64), ("q", 128), ("k", 128)):
        o, n = lay[name]
        za, zb = _pairs(ra["qkv"][:, o:o + n], d), _pairs(rb["qkv"][:, o:o + n], d)
        j = np.arange(d // 2)
        rot = np.exp(1j * _LEG_SHIFT * 1e6 ** (-2.0 * j / d))
        err = np.abs(zb - za * rot)
        tol = 2.0 ** -7 * (np.abs(za) + np.abs(zb)) + 1e-30
        assert np.all(err <= tol), name
        # the rotation does act: a pair keeps its place only if it is (near) zero
        moved = np.abs(zb - za) > 4 * tol
        assert moved.mean() > 0.9, name
    for name in ("w_idx", "v"):
        o, n = lay[name]
        assert np.array_equal(ra["qkv"][:, o:o + n], rb["qkv"][:, o:o + n]), name


def test_layer_step_rotation_is_identity_at_position_zero():
    """Token 0 of a block at pos0 = 0 sits at position 0, where RoPE is the identity: its
    rotated q_I / k_I / Q / K equal the bf16 projection of the normalised row."""
    T = 2
    lay, cache = _zero_prefix_dsa(0, T)
    x = synth.module_x(43, T)
    r = O.layer_step("dsa", x, lay.gamma, lay.w_qkvi, lay.w_o, cache, 0, top_k=64)
    pre = O.bf16_round_trip(O.project(r["normed"], O.decode_bf16(lay.w_qkvi)))
    assert np.array_equal(r["qkv"][0], pre[0])
    assert not np.array_equal(r["qkv"][1], pre[1])      # token 1 is at position 1


def test_layer_step_indexer_reads_back_quantised_rows(indexer_leg):
    """The indexer of the layer step scores the cache as stored: the block's own k_I rows
    quantised to e4m3 (codes and scales equal the row quantiser of the rotated k_I), the
    rotated q_I and the unrotated w_I; an all-zero prefix scores exactly 0."""
    lay = O.proj_layout("dsa")
    for pos0, (r, cache) in indexer_leg.items():
        T = _LEG_T
        L = pos0 + T
        o, n = lay["k_idx"]
        codes, sc = O.quantize_rows_e4m3(r["qkv"][:, o:o + n])
        assert np.array_equal(cache["k_idx"][pos0:L], codes)
        assert np.array_equal(cache["k_idx_scale"][pos0:L], sc)
        o, n = lay["q_idx"]
        qi = r["qkv"][:, o:o + n].reshape(T, 16, 64)
        o, n = lay["w_idx"]
        wi = r["qkv"][:, o:o + n]
        kt = O.decode_e4m3(codes) * sc.astype(np.float64)[:, None]
        d = np.einsum("thd,sd->ths", qi, kt)
        ref = np.einsum("th,ths->ts", wi, np.maximum(d, 0.0))
        mag = np.einsum("th,ths->ts", np.abs(wi), np.einsum("thd,sd->ths", np.abs(qi), np.abs(kt)))
        for t in range(T):
            assert np.all(r["scores"][t, :pos0] == 0.0)
            got = r["scores"][t, pos0:pos0 + t + 1]
            assert np.all(np.abs(got - ref[t, : t + 1]) <= 1e-13 * mag[t, : t + 1])
            assert np.all(np.isneginf(r["scores"][t, pos0 + t + 1:]))


def test_layer_step_block_scores_shift_invariant_within_quantiser_bound(indexer_leg):
    """q_I(p) . k_I(p') depends only on p' - p, so the block's own indexer scores at pos0 = A
    and at A + shift agree within the rounding of each side: bf16 rotated rows (half an ulp,
    2^-8 relative), e4m3 keys (2^-4 relative, 2^-10 of the row scale below the normal
    range) and fp32 cos/sin (2^-22 of the pair norm, with slack)."""
    lay = O.proj_layout("dsa")
    T = _LEG_T
    scores, bounds = [], []
    for pos0, (r, cache) in indexer_leg.items():
        o, n = lay["q_idx"]
        q = r["qkv"][:, o:o + n].reshape(T, 16, 64)
        o, n = lay["k_idx"]
        k = r["qkv"][:, o:o + n]
        o, n = lay["w_idx"]
        w = r["qkv"][:, o:o + n]
        s = cache["k_idx_scale"][pos0:pos0 + T].astype(np.float64)
        nq = np.abs(_pairs(q.reshape(T, -1), 64)).reshape(T, 16, 32)
        nq = np.concatenate([nq, nq], axis=-1)
        nk = np.abs(_pairs(k, 64)).reshape(T, 32)
        nk = np.concatenate([nk, nk], axis=-1)
        ek = (2.0 ** -4 + 2.0 ** -7) * np.abs(k) + 2.0 ** -10 * s[:, None] + 2.0 ** -20 * nk
        eq = 2.0 ** -7 * np.abs(q) + 2.0 ** -20 * nq
        e = (np.einsum("thd,sd->ths", np.abs(q), ek) + np.einsum("thd,sd->ths", eq, np.abs(k) + ek))
        bounds.append(np.einsum("th,ths->ts", np.abs(w), e))
        scores.append(r["scores"][:, pos0:pos0 + T])
    for t in range(T):
        a, b = scores[0][t, : t + 1], scores[1][t, : t + 1]
        assert np.all(np.abs(a - b) <= bounds[0][t, : t + 1] + bounds[1][t, : t + 1])


# ----------------------------------------------------------------------------- top-k

def _brute_topk(scores, pos0, k):
    T = scores.shape[0]
    out = []
    for t in range(T):
        vis = pos0 + t + 1
        ranked = sorted(range(vis), key=lambda s: (-float(scores[t, s]), s))
        sel = sorted(ranked[:min(k, vis)])
        out.append(sel + [-1] * (k - len(sel)))
    return np.array(out, np.int32)


@pytest.mark.parametrize("seed", range(6))
def test_topk_vs_brute_force_with_ties(seed):
    g = np.random.default_rng(seed)
    T, L, k = 4, 48, 9
    scores = g.integers(0, 6, size=(T, L)).astype(np.float64)   # many ties
    scores[:, ::7] *= -1
    idx, cnt = O.topk_indices(scores, L - T, k)
    assert np.array_equal(idx, _brute_topk(scores, L - T, k))
    assert list(cnt) == [k] * T


def test_topk_golden_tie_case_and_all_equal():
    g = json.load(open(os.path.join(GOLD, "indexer_topk_tiny.json")))["tie_case"]
    s = np.array(g["scores"], float)
    assert O.topk_indices(s, g["pos0"], 2)[0].tolist() == g["top2"]
    assert O.topk_indices(s, g["pos0"], 4)[0].tolist() == g["top4"]
    eq = np.full((2, 100), 3.25)
    idx, _ = O.topk_indices(eq, 98, 10)
    assert idx.tolist() == [list(range(10))] * 2


def test_topk_negative_zero_ties_positive_zero():
    s = np.array([[0.0, -0.0, 0.0, -1.0]])
    idx, _ = O.topk_indices(s, 3, 2)
    assert idx.tolist() == [[0, 1]]


def test_topk_visible_at_most_k_selects_all():
    g = np.random.default_rng(1)
    T, L, k = 3, 10, 16
    s = g.standard_normal((T, L))
    idx, cnt = O.topk_indices(s, L - T, k)
    for t in range(T):
        vis = L - T + t + 1
        assert cnt[t] == vis
        assert idx[t, :vis].tolist() == list(range(vis))
        assert np.all(idx[t, vis:] == -1)


def test_topk_permutation_invariance_tie_free():
    g = np.random.default_rng(2)
    L, k = 300, 37
    s = g.standard_normal((1, L))           # continuous: no ties
    perm = g.permutation(L)
    idx, _ = O.topk_indices(s, L - 1, k)
    idx_p, _ = O.topk_indices(s[:, perm], L - 1, k)
    assert sorted(perm[idx_p[0]].tolist()) == idx[0].tolist()


# ----------------------------------------------------------------------------- attention

def _sdpa_causal(q, K, V, pos0, sm_scale):
    """Dense causal attention via torch's library routine (fp64, CPU)."""
    T, H, D = q.shape
    L = K.shape[0]
    qt = torch.from_numpy(q).permute(1, 0, 2)[None]              # [1,H,T,D]
    kt = torch.from_numpy(K)[None, None].expand(1, H, L, D)
    vt = torch.from_numpy(V)[None, None].expand(1, H, L, D)
    mask = torch.zeros(T, L, dtype=torch.bool)
    for t in range(T):
        mask[t, :pos0 + t + 1] = True
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=sm_scale)
    return o[0].permute(1, 0, 2).numpy()


def test_attention_hand_example():
    g = json.load(open(os.path.join(GOLD, "indexer_topk_tiny.json")))["attention_case"]
    out = O.attend_rows(np.array(g["q"]), np.array(g["K"]), np.array(g["V"]), 1.0)
    np.testing.assert_allclose(out, np.array(g["out"]), rtol=1e-14)


def test_sparse_attention_equals_dense_when_visible_le_k():
    g = np.random.default_rng(4)
    T, H, D, L, k = 4, 8, 128, 60, 2048
    q = g.standard_normal((T, H, D))
    K = g.standard_normal((L, D))
    V = g.standard_normal((L, D))
    scores = g.standard_normal((T, L))
    idx, _ = O.topk_indices(scores, L - T, k)
    got = O.sparse_attention(q, K, V, idx, 1 / math.sqrt(D))
    ref = _sdpa_causal(q, K, V, L - T, 1 / math.sqrt(D))
    np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-12)


def test_attention_closed_forms():
    g = np.random.default_rng(6)
    H, D = 8, 128
    q = g.standard_normal((H, D))
    K = g.standard_normal((5, D))
    V = g.standard_normal((5, D))
    one = O.attend_rows(q, K[:1], V[:1], 0.1)
    np.testing.assert_allclose(one, np.broadcast_to(V[0], (H, D)), rtol=1e-14)
    Vc = np.broadcast_to(V[2], (5, D))
    np.testing.assert_allclose(O.attend_rows(q, K, Vc, 0.1), np.broadcast_to(V[2], (H, D)), rtol=1e-13)
    # sink: constant V scaled by 1 - p_sink
    sink = g.standard_normal(H)
    z = 0.1 * q @ K.T
    p_sink = np.exp(sink) / (np.exp(z).sum(axis=1) + np.exp(sink))
    got = O.attend_rows(q, K, Vc, 0.1, sink)
    np.testing.assert_allclose(got, (1 - p_sink)[:, None] * V[2][None, :], rtol=1e-12)
    # sink of -inf is no sink
    np.testing.assert_allclose(O.attend_rows(q, K, V, 0.1, np.full(H, -np.inf)),
                               O.attend_rows(q, K, V, 0.1), rtol=0, atol=0)
    # order of the index list does not matter (up to fp64 rounding)
    idx = np.array([[3, 0, 4, 1]])
    a = O.sparse_attention(q[None], K, V, idx, 0.1)
    b = O.sparse_attention(q[None], K, V, idx[:, ::-1], 0.1)
    assert np.max(np.abs(a - b)) <= 1e-12
    # skipped entries and an empty list
    c = O.sparse_attention(q[None], K, V, np.array([[3, -1, 0, 99, 4, 1]]), 0.1)
    np.testing.assert_array_equal(a, c)
    assert np.all(O.sparse_attention(q[None], K, V, np.array([[-1, -1]]), 0.1) == 0)


def test_swa_equals_dense_when_window_covers_context_and_w1_is_self():
    g = np.random.default_rng(8)
    T, H, D, L = 5, 8, 128, 40
    q = g.standard_normal((T, H, D))
    K = g.standard_normal((L, D))
    V = g.standard_normal((L, D))
    cap = 64
    Kr = np.zeros((cap, D)); Vr = np.zeros((cap, D))
    for p in range(L):
        Kr[p % cap] = K[p]; Vr[p % cap] = V[p]
    got = O.swa_attention(q, Kr, Vr, cap, L - T, 128, 1 / math.sqrt(D))
    ref = _sdpa_causal(q, K, V, L - T, 1 / math.sqrt(D))
    np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-12)
    w1 = O.swa_attention(q, Kr, Vr, cap, L - T, 1, 1 / math.sqrt(D))
    for t in range(T):
        np.testing.assert_allclose(w1[t], np.broadcast_to(V[L - T + t], (H, D)), rtol=1e-14)


# ----------------------------------------------------------------------------- layer stages

def test_rmsnorm_vs_torch_and_constant():
    g = np.random.default_rng(9)
    x = g.standard_normal((8, 4096))
    gam = g.standard_normal(4096)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (4096,), torch.from_numpy(gam), eps=1e-6)
    np.testing.assert_allclose(O.rmsnorm(x, gam, 1e-6), ref.numpy(), rtol=1e-13)
    c = 0.37
    y = O.rmsnorm(np.full((1, 16), c), np.ones(16), 1e-6)
    np.testing.assert_allclose(y, c / math.sqrt(c * c + 1e-6), rtol=1e-14)


def test_rope_closed_forms_and_invariants():
    d = 128
    theta = 1e6
    # pos 0 is the identity
    g = np.random.default_rng(10)
    x = g.standard_normal((1, 3, d))
    assert np.array_equal(O.rope(x, [0], theta), x)
    # unit vector e_i rotates in the (i, i + d/2) plane by pos * theta^(-2i/d)
    for i in (0, 5, 63):
        e = np.zeros((1, 1, d)); e[0, 0, i] = 1.0
        p = 1000003
        out = O.rope(e, [p], theta)[0, 0]
        ang = p * theta ** (-2.0 * i / d)
        assert abs(out[i] - math.cos(ang)) < 1e-7
        assert abs(out[i + d // 2] - math.sin(ang)) < 1e-7
        assert np.count_nonzero(out) <= 2
    # complex formulation: (a + ib) * exp(i*angle)
    pos = np.array([3, 77, 1048575])
    x = g.standard_normal((3, 2, d))
    c, s = O.rope_cos_sin(pos, d, theta)
    z = (x[..., :d // 2] + 1j * x[..., d // 2:]) * (c + 1j * s)[:, None, :]
    ref = np.concatenate([z.real, z.imag], axis=-1)
    np.testing.assert_allclose(O.rope(x, pos, theta), ref, rtol=1e-13, atol=1e-13)
    # norm and relative position (cos/sin are fp32-rounded, so 1e-6)
    y = O.rope(x, pos, theta)
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-6)
    qv = g.standard_normal((1, 1, d)); kv = g.standard_normal((1, 1, d))
    a = np.sum(O.rope(qv, [500], theta) * O.rope(kv, [200], theta))
    b = np.sum(O.rope(qv, [900500], theta) * O.rope(kv, [900200], theta))
    assert abs(a - b) <= 1e-5 * (np.linalg.norm(qv) * np.linalg.norm(kv))


def test_quantize_rows_vs_torch_cast_and_bounds():
    g = np.random.default_rng(11)
    rows = O.bf16_round_trip(g.standard_normal((64, 64)) * 3)
    rows[5] = 0.0
    codes, scale = O.quantize_rows_e4m3(rows)
    assert scale[5] == 1.0 and np.all(codes[5] & 0x7F == 0)
    amax = np.max(np.abs(rows), axis=1)
    np.testing.assert_array_equal(scale[amax > 0], (amax[amax > 0] / 448.0).astype(np.float32))
    # the division and cast done by the library give the same codes
    xs = (torch.from_numpy(rows.astype(np.float32)) / torch.from_numpy(scale)[:, None])
    ref = xs.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(codes, ref)
    # the largest magnitude of each nonzero row maps to +-448
    deq = O.dequant_rows(codes, "fp8", scale)
    nz = amax > 0
    assert np.all(np.max(np.abs(O.decode_e4m3(codes[nz])), axis=1) == 448.0)
    # relative error of normal codes <= 2^-4
    big = np.abs(rows) >= (2.0 ** -6) * scale[:, None]
    assert np.all(np.abs(deq - rows)[big] <= 2.0 ** -4 * np.abs(rows)[big])


def test_project_with_permutation_weights_is_exact_selection():
    g = np.random.default_rng(12)
    y = O.bf16_round_trip(g.standard_normal((8, 32)))
    perm = g.permutation(32)[:20]
    W = np.zeros((20, 32)); W[np.arange(20), perm] = 1.0
    assert np.array_equal(O.project(y, W), y[:, perm])


# ----------------------------------------------------------------------------- layer step

def _small_dsa_layer(seed, L, T, w_std=0.02, top_k=2048):
    lay = synth.layer_inputs("dsa", 0, L, T, seed=seed, w_std=w_std)
    cache = {"k": lay.k.copy(), "v": lay.v.copy(), "k_idx": lay.k_idx.copy(),
             "k_idx_scale": lay.k_idx_scale.copy()}
    return lay, cache


def test_layer_step_zero_output_projection_is_residual():
    T, L = 2, 64
    lay, cache = _small_dsa_layer(0, L, T)
    x = synth.module_x(0, T)
    w_o = np.zeros_like(lay.w_o)
    r = O.layer_step("dsa", x, lay.gamma, lay.w_qkvi, w_o, cache, L - T, top_k=16)
    np.testing.assert_array_equal(r["x_out"], O.decode_bf16(x))


def test_layer_step_zero_query_projection_averages_selected_values():
    """Q weights 0 => every logit 0 => each head's output is the plain mean of
    the selected V rows (rounded to bf16)."""
    T, L, k = 3, 200, 32
    lay, cache = _small_dsa_layer(1, L, T)
    w = lay.w_qkvi.copy()
    w[:1024] = 0
    x = synth.module_x(1, T)
    r = O.layer_step("dsa", x, lay.gamma, w, lay.w_o, cache, L - T, top_k=k)
    V = O.decode_bf16(cache["v"])
    for t in range(T):
        sel = r["idx"][t][r["idx"][t] >= 0]
        assert len(sel) == k
        mean = V[sel].mean(axis=0)
        ref = O.bf16_round_trip(np.tile(mean, 8))
        np.testing.assert_array_equal(r["attn"][t], ref)


def test_layer_step_dsa_with_short_context_is_dense_attention():
    T, L = 4, 50
    lay, cache = _small_dsa_layer(2, L, T)
    x = synth.module_x(2, T)
    r = O.layer_step("dsa", x, lay.gamma, lay.w_qkvi, lay.w_o, cache, L - T, top_k=2048)
    q = r["qkv"][:, :1024].reshape(T, 8, 128)
    K = O.decode_bf16(cache["k"][:L]); V = O.decode_bf16(cache["v"][:L])
    dense = _sdpa_causal(q, K, V, L - T, 1 / math.sqrt(128)).reshape(T, 1024)
    np.testing.assert_array_equal(r["attn"], O.bf16_round_trip(dense))
    # the new rows were appended before attention and quantised indexer keys written
    assert np.array_equal(cache["k"][L - T:L], O.round_to_bf16(r["qkv"][:, 1024:1152]))
    assert np.array_equal(cache["k_idx"][L - T:L], r["k_idx_codes"])


def test_layer_step_swa_small_context_is_dense():
    T, L = 3, 20
    lay = synth.layer_inputs("swa", 0, L, T, seed=3, ring_cap=160)
    cache = {"k": lay.k.copy(), "v": lay.v.copy(), "ring_cap": 160}
    x = synth.module_x(3, T)
    r = O.layer_step("swa", x, lay.gamma, lay.w_qkvi, lay.w_o, cache, L - T)
    q = r["qkv"][:, :1024].reshape(T, 8, 128)
    K = O.decode_bf16(cache["k"][:L]); V = O.decode_bf16(cache["v"][:L])
    dense = _sdpa_causal(q, K, V, L - T, 1 / math.sqrt(128)).reshape(T, 1024)
    np.testing.assert_array_equal(r["attn"], O.bf16_round_trip(dense))


# ----------------------------------------------------------------------------- W8A8

def _grid_rows(g, T, K, j):
    """Rows of e4m3 values times 2^j[t]; each row's largest magnitude is 448 * 2^j[t]."""
    codes = (g.integers(0, 127, size=(T, K)) | (g.integers(0, 2, size=(T, K)) << 7)).astype(np.uint8)
    codes[:, 0] = 126                                     # +448
    return O.decode_e4m3(codes) * np.exp2(np.asarray(j, np.float64))[:, None]


def test_w8a8_quantiser_is_lossless_on_scaled_e4m3_rows():
    g = np.random.default_rng(21)
    j = np.array([-3, 0, 2, -7])
    rows = _grid_rows(g, 4, 96, j)
    codes, s = O.quantize_tokens_w8a8(rows)
    np.testing.assert_array_equal(s, np.exp2(j).astype(np.float32))       # amax / 448 = 2^j exactly
    np.testing.assert_array_equal(O.decode_e4m3(codes) * s[:, None].astype(np.float64), rows)


def test_w8a8_quantiser_zero_rows_scaling_and_bounds():
    g = np.random.default_rng(22)
    rows = O.bf16_round_trip(g.standard_normal((32, 256)) * 2.5)
    rows[3] = 0.0
    codes, s = O.quantize_tokens_w8a8(rows)
    assert s[3] == 1.0 and np.all(codes[3] & 0x7F == 0)
    # a power-of-two rescaling of a row changes only its scale
    c4, s4 = O.quantize_tokens_w8a8(rows * 4.0)
    np.testing.assert_array_equal(c4, codes)
    nz = np.arange(32) != 3                                 # (the zero row keeps scale 1)
    np.testing.assert_array_equal(s4[nz], s[nz] * np.float32(4.0))
    # each row's largest magnitude lands on +-448
    assert np.all(np.max(np.abs(O.decode_e4m3(codes[nz])), axis=1) == 448.0)
    # error bound: half an e4m3 ulp (2^-4 relative; 2^-10 * scale in the subnormal range)
    # plus the fp32 roundings of the product and of the scale
    deq = O.decode_e4m3(codes) * s[:, None].astype(np.float64)
    bound = (2.0 ** -4 + 2.0 ** -22) * np.abs(rows) + 2.0 ** -10 * s[:, None]
    assert np.all(np.abs(deq - rows) <= bound)


def test_w8a8_quantiser_vs_torch_fp32_ops_and_cast():
    """The same steps done by the library in fp32: 448 / amax, y * inv, cast to e4m3fn."""
    g = np.random.default_rng(23)
    rows = O.bf16_round_trip(g.standard_normal((48, 512)) * np.exp2(g.integers(-6, 6, size=(48, 1))))
    codes, s = O.quantize_tokens_w8a8(rows)
    t = torch.from_numpy(rows.astype(np.float32))
    amax = t.abs().amax(dim=1)
    inv = torch.tensor(448.0, dtype=torch.float32) / amax
    ref = (t * inv[:, None]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(codes, ref)
    np.testing.assert_array_equal(s, (amax / torch.tensor(448.0, dtype=torch.float32)).numpy())


def test_w8a8_projection_lossless_rows_equal_dequantised_product():
    """Rows the quantiser represents exactly: the W8A8 product is the plain product with
    the dequantised weights (non-square shapes and distinct per-token / per-row scales
    catch a transposed operand or a swapped scale)."""
    g = np.random.default_rng(24)
    T, K, N = 3, 64, 5
    y = _grid_rows(g, T, K, [1, -2, 0])
    wc = (g.integers(0, 127, size=(N, K)) | (g.integers(0, 2, size=(N, K)) << 7)).astype(np.uint8)
    ws = (g.uniform(0.5, 2.0, size=N) * 1e-3).astype(np.float32)
    got = O.project_w8a8(y, wc, ws)
    wdeq = O.decode_e4m3(wc) * ws[:, None].astype(np.float64)
    ref = O.project(y, wdeq)
    mag = O.project(np.abs(y), np.abs(wdeq))
    assert np.all(np.abs(got - ref) <= 1e-14 * mag)
    # one nonzero weight per row selects one scaled input column
    wc1 = np.zeros((N, K), np.uint8)
    cols = g.permutation(K)[:N]
    wc1[np.arange(N), cols] = 0x38                        # 1.0
    got1 = O.project_w8a8(y, wc1, ws)
    np.testing.assert_array_equal(got1, y[:, cols] * ws[None, :].astype(np.float64))


def test_w8a8_projection_error_bound_on_general_rows():
    g = np.random.default_rng(25)
    T, K, N = 4, 1024, 7
    y = O.bf16_round_trip(g.standard_normal((T, K)))
    wc, ws = synth.to_e4m3_rows(g.standard_normal((N, K)).astype(np.float32) * 0.02)
    _, s = O.quantize_tokens_w8a8(y)
    wdeq = O.decode_e4m3(wc) * ws[:, None].astype(np.float64)
    err = np.abs(O.project_w8a8(y, wc, ws) - O.project(y, wdeq))
    bound = O.project((2.0 ** -4 + 2.0 ** -22) * np.abs(y) + 2.0 ** -10 * s[:, None].astype(np.float64),
                      np.abs(wdeq))
    assert np.all(err <= bound)
    assert np.max(err) > 0                                  # the quantiser does act here


def test_layer_step_w8a8_equals_bf16_step_when_lossless():
    """gamma = 112 and exact-norm inputs make every normalised value 0, +-112, +-224 or
    +-448 with 448 in every row (scale 1, lossless codes), and power-of-two weight row
    scales make the dequantised weights exact bf16 values: the W8A8 step then equals the
    bf16 step on those weights exactly up to the output projection, whose input (the
    attention output) is quantised with the bounded error of the quantiser."""
    T, L = 3, 300
    g = np.random.default_rng(26)
    lay, cache_a = _small_dsa_layer(4, L, T)
    cache_b = {k: v.copy() for k, v in cache_a.items()}
    x = synth.exact_norm_x(5, T, groups=((1,) * 16, (2, 2, 2, 2), (4,)))
    gamma = synth.to_bf16_bits(np.full(4096, 112.0, np.float32))
    wq = (g.integers(0, 127, size=lay.w_qkvi.shape) | (g.integers(0, 2, size=lay.w_qkvi.shape) << 7)).astype(np.uint8)
    wo = (g.integers(0, 127, size=lay.w_o.shape) | (g.integers(0, 2, size=lay.w_o.shape) << 7)).astype(np.uint8)
    sq = np.exp2(g.integers(-16, -12, size=wq.shape[0])).astype(np.float32)
    so = np.exp2(g.integers(-16, -12, size=wo.shape[0])).astype(np.float32)
    wq_bf = synth.to_bf16_bits((O.decode_e4m3(wq) * sq[:, None]).astype(np.float32))
    wo_bf = synth.to_bf16_bits((O.decode_e4m3(wo) * so[:, None]).astype(np.float32))
    assert np.array_equal(O.decode_bf16(wq_bf), O.decode_e4m3(wq) * sq[:, None])   # exact bf16 values
    a = O.layer_step("dsa", x, gamma, wq, wo, cache_a, L - T, eps=0.0, top_k=64,
                     w_qkvi_scale=sq, w_o_scale=so)
    b = O.layer_step("dsa", x, gamma, wq_bf, wo_bf, cache_b, L - T, eps=0.0, top_k=64)
    assert set(np.unique(np.abs(a["normed"]))) <= {0.0, 112.0, 224.0, 448.0}
    for key in ("qkv", "idx", "attn"):
        np.testing.assert_array_equal(a[key], b[key])
    codes, s = O.quantize_tokens_w8a8(a["attn"])
    wod = O.decode_bf16(wo_bf)
    bound = O.project((2.0 ** -4 + 2.0 ** -22) * np.abs(a["attn"]) + 2.0 ** -10 * s[:, None].astype(np.float64),
                      np.abs(wod))
    assert np.all(np.abs(a["x_out_f64"] - b["x_out_f64"]) <= bound)
    assert not np.array_equal(a["x_out_f64"], b["x_out_f64"])


# ----------------------------------------------------------------------------- module step

def _swa_stack(n, pos0, T, seed, zero_wo=()):
    """n SWA layers of the module workload; layers in zero_wo get W_o = 0, which makes
    them the identity on x (the output is the residual alone)."""
    out = []
    for i in range(n):
        lay = synth.layer_inputs("swa", i, pos0 + T, T, seed=seed, ring_cap=256)
        w_o = lay.w_o.copy()
        if i in zero_wo:
            w_o[:] = 0
        out.append(dict(kind="swa", gamma=lay.gamma, w_qkvi=lay.w_qkvi, w_o=w_o,
                        cache={"k": lay.k.copy(), "v": lay.v.copy(), "ring_cap": 256}))
    return out


def test_module_step_hands_each_layer_the_previous_output():
    """Identity layers pin the chaining: with layer 0 the identity the module is layer 1
    alone on x; with layer 1 the identity it is layer 0 alone (a chain that fed x_in to
    every layer, or returned the first layer's output, fails one of the two)."""
    pos0, T = 300, 4
    x = synth.module_x(5, T)
    got, _ = O.module_step(_swa_stack(2, pos0, T, 9, zero_wo={0}), x, pos0)
    l1 = _swa_stack(2, pos0, T, 9)[1]
    ref = O.layer_step("swa", x, l1["gamma"], l1["w_qkvi"], l1["w_o"], l1["cache"], pos0)
    assert np.array_equal(got, O.round_to_bf16(ref["x_out_f64"]))
    assert not np.array_equal(got, x)
    got, _ = O.module_step(_swa_stack(2, pos0, T, 9, zero_wo={1}), x, pos0)
    l0 = _swa_stack(2, pos0, T, 9)[0]
    ref = O.layer_step("swa", x, l0["gamma"], l0["w_qkvi"], l0["w_o"], l0["cache"], pos0)
    assert np.array_equal(got, O.round_to_bf16(ref["x_out_f64"]))


def test_module_step_of_identity_layers_keeps_x_and_fills_every_cache():
    pos0, T = 1000, 3
    x = synth.module_x(6, T)
    layers = _swa_stack(3, pos0, T, 4, zero_wo={0, 1, 2})
    got, res = O.module_step(layers, x, pos0)
    assert np.array_equal(got, x)
    for lay, r in zip(layers, res):
        for t in range(T):
            slot = (pos0 + t) % 256
            assert np.array_equal(lay["cache"]["k"][slot], O.round_to_bf16(r["qkv"][t, 1024:1152]))
            assert np.array_equal(lay["cache"]["v"][slot], O.round_to_bf16(r["qkv"][t, 1152:1280]))
    # the layers' own weights differ, so their new rows do too
    assert not np.array_equal(layers[0]["cache"]["k"][pos0 % 256], layers[1]["cache"]["k"][pos0 % 256])
