"""GPU parity of every entry point against the CPU oracle (through the C ABI).

Tolerances (derived from the arithmetic):
* indexer scores: products of bf16 operands are exact in fp32; the 64-term dot, the
  16-term weighted head sum and the scale multiply each add at most n*2^-24 relative
  error of the absolute sum S = sum_h |w| sum_d |q k|, so |gpu - exact| <= 2^-16 * S.
  Integer-valued inputs are exact in fp32 under any order: bit-exact there.
* top-k on given scores: bit-exact (integer radix on order-preserving keys).
* fused scan + top-k: bit-identical to top-k of the materialised GPU scores; against
  the fp64 scores the index sets may differ only inside the 2^-16 * S rounding band.
* attention: fp32 output ||g - r||_inf <= 1e-5 ||r||_inf per (token, head) row;
  bf16 output max-abs <= 2e-2.
"""
import math

import numpy as np
import pytest
import torch

import synth
from oracle import dsa_oracle as O
from tests.gpu_util import DEV, up, down, bf16_bits, tie_band_ok

pytestmark = pytest.mark.gpu

SM = 1.0 / math.sqrt(128)


@pytest.fixture(scope="module")
def dsa():
    import sparse_attention_decode_indexer_amd as m
    assert torch.cuda.is_available()
    return m


def _kdt(dsa, inp):
    return dsa.BF16 if inp.k_idx_dtype == "bf16" else dsa.FP8_E4M3


def _gpu_scores(dsa, inp, T=None, L=None, pos0=None):
    T = T or inp.T
    L = L or inp.L
    pos0 = inp.pos0 if pos0 is None else pos0
    ld = (L + 3) // 4 * 4
    sc = torch.full((T, ld), float("nan"), dtype=torch.float32, device=DEV)
    kscale = up(inp.k_idx_scale) if inp.k_idx_scale is not None else None
    dsa.dsa_indexer_scores(up(inp.q_idx), up(inp.w_idx), up(inp.k_idx), kscale, _kdt(dsa, inp), T, L,
                           pos0, sc, ld)
    torch.cuda.synchronize()
    return down(sc)[:, :L]


def _oracle_scores(inp, with_abs=True):
    krows = O.dequant_rows(inp.k_idx, inp.k_idx_dtype, inp.k_idx_scale)
    return O.indexer_scores(O.decode_bf16(inp.q_idx), inp.w_idx, krows, inp.pos0, with_abs=with_abs)


# ----------------------------------------------------------------------------- indexer

@pytest.mark.parametrize("tie", [False, True])
def test_indexer_scores_integer_config_bit_exact(dsa, tie):
    inp = synth.dsa_config("tiny", seed=0, tie_stress=tie)
    g = _gpu_scores(dsa, inp)
    r = _oracle_scores(inp, with_abs=False)
    assert np.array_equal(g.astype(np.float64), r)


@pytest.mark.parametrize("name,L,T", [("verify64k", 5000, 8), ("verify64k", 4099, 5),
                                      ("verify256k_fp8", 9001, 8), ("verify256k_fp8", 300, 3),
                                      ("verify1m", 20000, 8)])
def test_indexer_scores_within_rounding_band(dsa, name, L, T):
    inp = synth.dsa_config(name, seed=1, L=L, T=T)
    g = _gpu_scores(dsa, inp)
    r, S = _oracle_scores(inp)
    vis = np.isfinite(r)
    assert np.array_equal(vis, np.isfinite(g)), "causal mask differs"
    assert np.all(np.isneginf(g[~vis]))
    err = np.abs(g[vis] - r[vis])
    assert np.all(err <= 2.0 ** -16 * S[vis] + 1e-30), float(np.max(err / (S[vis] + 1e-30)))


def test_indexer_fp8_decode_all_codes(dsa):
    """Each key row holds one e4m3 code in dim 0; q = +-e_0 on head 0 with weight 1
    recovers relu(+-value * scale) exactly for all 256 codes (NaN codes skipped)."""
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    L = len(codes)
    k = np.zeros((L, 64), np.uint8)
    k[:, 0] = codes
    scale = np.full(L, 0.5, np.float32)
    vals = O.decode_e4m3(codes) * 0.5
    for sign in (1.0, -1.0):
        q = np.zeros((1, 16, 64), np.float32)
        q[0, 0, 0] = sign
        w = np.zeros((1, 16), np.float32)
        w[0, 0] = 1.0
        sc = torch.zeros((1, L + (-L) % 4), dtype=torch.float32, device=DEV)
        dsa.dsa_indexer_scores(up(synth.to_bf16_bits(q)), up(w), up(k), up(scale), dsa.FP8_E4M3, 1, L,
                               L - 1, sc, sc.shape[1])
        torch.cuda.synchronize()
        g = down(sc)[0, :L].astype(np.float64)
        assert np.array_equal(g, np.maximum(sign * vals, 0.0))


def test_indexer_full_context_sampled(dsa):
    """1M-position workload at its full size: GPU scores checked on sampled columns."""
    inp = synth.dsa_config("verify1m", seed=0)
    g = _gpu_scores(dsa, inp)
    rng = np.random.default_rng(0)
    cols = np.unique(np.concatenate([rng.choice(inp.L, 4000, replace=False),
                                     np.arange(inp.L - 64, inp.L), inp.planted[:500]]))
    krows = O.dequant_rows(inp.k_idx[cols], "fp8", inp.k_idx_scale[cols])
    # the oracle over the sampled rows only, every row visible to every token; the causal
    # limit is then applied by the rows' own positions
    r, S = O.indexer_scores(O.decode_bf16(inp.q_idx), inp.w_idx, krows, len(cols) - 1, with_abs=True)
    for t in range(inp.T):
        vis = cols <= inp.pos0 + t
        assert np.all(np.abs(g[t, cols[vis]] - r[t, vis]) <= 2.0 ** -16 * S[t, vis] + 1e-30)
        assert np.all(np.isneginf(g[t, cols[~vis]]))


# ----------------------------------------------------------------------------- top-k

def _gpu_topk(dsa, scores, pos0, k):
    T, L = scores.shape
    ld = (L + 3) // 4 * 4
    s = np.full((T, ld), -np.inf, np.float32)
    s[:, :L] = scores
    idx = torch.full((T, k), -7, dtype=torch.int32, device=DEV)
    cnt = torch.full((T,), -7, dtype=torch.int32, device=DEV)
    ws = dsa.workspace(dsa.WS_TOPK, T, L, k)
    dsa.dsa_topk(up(s), T, L, ld, pos0, k, idx, cnt, ws)
    torch.cuda.synchronize()
    return down(idx), down(cnt)


TOPK_CASES = [
    # (name, T, L, k, generator)
    ("ints-ties", 8, 5000, 2048, lambda g, T, L: g.integers(-3, 30, (T, L)).astype(np.float32)),
    ("all-equal", 3, 3000, 100, lambda g, T, L: np.full((T, L), 1.5, np.float32)),
    ("neg-zero", 2, 600, 37, lambda g, T, L: np.where(g.random((T, L)) < 0.5, -0.0, 0.0).astype(np.float32)),
    ("normal", 8, 70000, 2048, lambda g, T, L: g.standard_normal((T, L)).astype(np.float32)),
    ("vis-le-k", 8, 1000, 2048, lambda g, T, L: g.standard_normal((T, L)).astype(np.float32)),
    ("small-k", 5, 9999, 7, lambda g, T, L: g.standard_normal((T, L)).astype(np.float32)),
    ("k1", 1, 130, 1, lambda g, T, L: g.integers(0, 3, (T, L)).astype(np.float32)),
    ("tiny-L", 8, 8, 4, lambda g, T, L: g.integers(0, 3, (T, L)).astype(np.float32)),
    ("negatives", 4, 20000, 512, lambda g, T, L: -np.abs(g.standard_normal((T, L))).astype(np.float32)),
    # candidate counts around the register-resident limit of the selection tail (8192)
    ("reg-edge", 3, 8194, 2048, lambda g, T, L: g.standard_normal((T, L)).astype(np.float32)),
    ("mid-nc", 2, 12000, 2048, lambda g, T, L: g.standard_normal((T, L)).astype(np.float32)),
    ("sparse-big", 8, 262144, 2048,
     lambda g, T, L: np.where(g.random((T, L)) < 0.003, 100 + g.random((T, L)), g.random((T, L))).astype(np.float32)),
    # ties at the cut inside a small boundary bin of the first radix digit (the bin's keys
    # are resolved by one wave), taken whole or in part
    ("cut-ties", 8, 70000, 2048, lambda g, T, L: _with_cut_ties(g, g.standard_normal((T, L)), 2048, 6)),
    ("cut-ties-many", 4, 40000, 1000, lambda g, T, L: _with_cut_ties(g, g.random((T, L)), 1000, 40)),
    # runs of high scores: some workgroups then hold 33-64 and hundreds of candidates
    ("clustered", 4, 70000, 2048,
     lambda g, T, L: _with_runs(g, g.standard_normal((T, L)), [(1000, 300), (20000, 30), (40100, 60)])),
]


def _with_runs(g, s, runs):
    """Scores 5 + U(0,1) over each (start, length) run of positions."""
    s = s.astype(np.float32)
    for a, n in runs:
        s[:, a:a + n] = (5 + g.random((s.shape[0], n))).astype(np.float32)
    return s


def _with_cut_ties(g, s, k, n):
    """Copies of each row's k-th largest early score written at n random early positions."""
    s = s.astype(np.float32)
    T, L = s.shape
    for t in range(T):
        v = np.sort(s[t, : L - T])[-k]
        s[t, g.choice(L - T, n, replace=False)] = v
    return s


@pytest.mark.parametrize("case", TOPK_CASES, ids=[c[0] for c in TOPK_CASES])
def test_topk_bit_exact_on_given_scores(dsa, case):
    name, T, L, k, gen = case
    g = np.random.default_rng(3)
    s = gen(g, T, L)
    pos0 = L - T
    idx, cnt = _gpu_topk(dsa, s, pos0, k)
    ridx, rcnt = O.topk_indices(s.astype(np.float64), pos0, k)
    assert np.array_equal(cnt, rcnt)
    assert np.array_equal(idx, ridx)


def test_topk_full_context(dsa):
    T, L, k = 8, 1 << 20, 2048
    g = np.random.default_rng(5)
    s = g.standard_normal((T, L)).astype(np.float32)
    s[:, g.choice(L - T, 20000, replace=False)] = 7.0    # a large tie block across the boundary
    idx, cnt = _gpu_topk(dsa, s, L - T, k)
    ridx, rcnt = O.topk_indices(s.astype(np.float64), L - T, k)
    assert np.array_equal(cnt, rcnt) and np.array_equal(idx, ridx)


# ----------------------------------------------------------------------------- fused scan + top-k

@pytest.mark.parametrize("name,L,T,seed,tie", [("tiny", None, None, 0, False), ("tiny", None, None, 0, True),
                                               ("tiny", None, 8, 1, True), ("verify64k", 65536, 8, 0, False),
                                               ("verify256k_fp8", 40000, 8, 1, False),
                                               ("verify256k_fp8", None, None, 0, False),
                                               ("verify1m", 100000, 7, 2, False), ("verify1m", None, None, 3, False)])
def test_index_topk_matches_materialised_path_and_oracle(dsa, name, L, T, seed, tie):
    """Fused scan + top-k equals top-k of the GPU's own materialised scores bit for bit, and
    the oracle's selection within the rounding band; on the integer configs (plain and
    tie-stress, where most keys tie at the cut) it equals the oracle's bit for bit."""
    inp = synth.dsa_config(name, seed=seed, L=L, T=T, tie_stress=tie)
    T, L, k = inp.T, inp.L, inp.top_k
    idx = torch.full((T, k), -7, dtype=torch.int32, device=DEV)
    cnt = torch.zeros(T, dtype=torch.int32, device=DEV)
    ws = dsa.workspace(dsa.WS_INDEX_TOPK, T, L, k)
    kscale = up(inp.k_idx_scale) if inp.k_idx_scale is not None else None
    dsa.dsa_index_topk(up(inp.q_idx), up(inp.w_idx), up(inp.k_idx), kscale, _kdt(dsa, inp), T, L, inp.pos0,
                       k, idx, cnt, ws)
    torch.cuda.synchronize()
    fused = down(idx)
    g = _gpu_scores(dsa, inp)
    ridx_same, rcnt = O.topk_indices(g.astype(np.float64), inp.pos0, k)
    assert np.array_equal(fused, ridx_same), "fused selection differs from top-k of the GPU scores"
    assert np.array_equal(down(cnt), rcnt)
    r, S = _oracle_scores(inp)
    ridx, _ = O.topk_indices(r, inp.pos0, k)
    ok, ndiff = tie_band_ok(fused, ridx, r, S, inp.pos0, k)
    assert ok, f"selection differs outside the rounding band ({ndiff})"
    if name == "tiny":
        assert np.array_equal(fused, ridx)


# One token whose context fits one workgroup's chunk (L <= 4096) is selected by a single
# workgroup without any hand-off; L = 4097 is the first length over several workgroups.
SINGLE_L = [1, 2, 33, 511, 512, 513, 2047, 2048, 2049, 3000, 4095, 4096, 4097]


@pytest.mark.parametrize("L", SINGLE_L)
@pytest.mark.parametrize("k,gen", [(2048, "normal"), (7, "ints"), (300, "ties"), (1, "equal")])
def test_topk_single_token_short_context(dsa, L, k, gen):
    g = np.random.default_rng(L * 31 + k)
    if gen == "normal":
        s = g.standard_normal((1, L)).astype(np.float32)
    elif gen == "ints":
        s = g.integers(-2, 3, (1, L)).astype(np.float32)
    elif gen == "ties":
        s = _with_cut_ties(g, g.random((1, L)), min(k, max(1, L - 1)), min(9, max(0, L - 1))) if L > 1 else \
            np.zeros((1, 1), np.float32)
    else:
        s = np.where(g.random((1, L)) < 0.5, -0.0, 0.0).astype(np.float32)
    idx, cnt = _gpu_topk(dsa, s, L - 1, k)
    ridx, rcnt = O.topk_indices(s.astype(np.float64), L - 1, k)
    assert np.array_equal(cnt, rcnt)
    assert np.array_equal(idx, ridx)


@pytest.mark.parametrize("L", SINGLE_L)
@pytest.mark.parametrize("k,tie", [(2048, False), (2048, True), (100, False), (1, True)])
def test_index_topk_single_token_short_context(dsa, L, k, tie):
    """Integer-valued bf16 indexer inputs (exact scores): the fused selection of one token
    equals the oracle's bit for bit, tie order included (one workgroup up to 4096 keys,
    several beyond)."""
    inp = synth.dsa_config("tiny", seed=L, L=L, T=1, tie_stress=tie)
    idx = torch.full((1, k), -7, dtype=torch.int32, device=DEV)
    cnt = torch.full((1,), -7, dtype=torch.int32, device=DEV)
    ws = dsa.workspace(dsa.WS_INDEX_TOPK, 1, L, k)
    dsa.dsa_index_topk(up(inp.q_idx), up(inp.w_idx), up(inp.k_idx), None, dsa.BF16, 1, L, inp.pos0, k, idx, cnt,
                       ws)
    torch.cuda.synchronize()
    r, _ = _oracle_scores(inp)
    ridx, rcnt = O.topk_indices(r, inp.pos0, k)
    assert np.array_equal(down(cnt), rcnt)
    assert np.array_equal(down(idx), ridx)
    assert dsa.dsa_workspace_status(ws) == 0


@pytest.mark.parametrize("L", SINGLE_L)
@pytest.mark.parametrize("k", [2048, 64])
def test_index_topk_single_token_short_context_fp8(dsa, L, k):
    """e4m3 indexer keys (one workgroup up to 4096 keys): the fused selection equals top-k
    of the GPU's own materialised scores bit for bit and the oracle's within the rounding
    band."""
    inp = synth.dsa_config("verify256k_fp8", seed=L, L=L, T=1)
    idx = torch.full((1, k), -7, dtype=torch.int32, device=DEV)
    cnt = torch.full((1,), -7, dtype=torch.int32, device=DEV)
    ws = dsa.workspace(dsa.WS_INDEX_TOPK, 1, L, k)
    dsa.dsa_index_topk(up(inp.q_idx), up(inp.w_idx), up(inp.k_idx), up(inp.k_idx_scale), dsa.FP8_E4M3, 1, L,
                       inp.pos0, k, idx, cnt, ws)
    torch.cuda.synchronize()
    fused = down(idx)
    g = _gpu_scores(dsa, inp)
    ridx_same, rcnt = O.topk_indices(g.astype(np.float64), inp.pos0, k)
    assert np.array_equal(fused, ridx_same)
    assert np.array_equal(down(cnt), rcnt)
    r, S = _oracle_scores(inp)
    ridx, _ = O.topk_indices(r, inp.pos0, k)
    ok, ndiff = tie_band_ok(fused, ridx, r, S, inp.pos0, k)
    assert ok, f"selection differs outside the rounding band ({ndiff})"


def test_index_topk_full_context_planted(dsa):
    inp = synth.dsa_config("verify1m", seed=0)
    T, L, k = inp.T, inp.L, inp.top_k
    idx = torch.full((T, k), -7, dtype=torch.int32, device=DEV)
    ws = dsa.workspace(dsa.WS_INDEX_TOPK, T, L, k)
    dsa.dsa_index_topk(up(inp.q_idx), up(inp.w_idx), up(inp.k_idx), up(inp.k_idx_scale), dsa.FP8_E4M3, T, L,
                       inp.pos0, k, idx, None, ws)
    torch.cuda.synchronize()
    fused = down(idx)
    g = _gpu_scores(dsa, inp)
    ridx_same, _ = O.topk_indices(g.astype(np.float64), inp.pos0, k)
    assert np.array_equal(fused, ridx_same)
    r, S = _oracle_scores(inp)
    ridx, _ = O.topk_indices(r, inp.pos0, k)
    ok, ndiff = tie_band_ok(fused, ridx, r, S, inp.pos0, k)
    assert ok, ndiff
    # planted rows dominate the selection
    assert np.isin(fused[0], inp.planted).mean() > 0.99
    # run-to-run bitwise
    idx2 = torch.full((T, k), -9, dtype=torch.int32, device=DEV)
    dsa.dsa_index_topk(up(inp.q_idx), up(inp.w_idx), up(inp.k_idx), up(inp.k_idx_scale), dsa.FP8_E4M3, T, L,
                       inp.pos0, k, idx2, None, ws)
    torch.cuda.synchronize()
    assert np.array_equal(down(idx2), fused)


# ----------------------------------------------------------------------------- attention

def _attn_inputs(inp):
    if inp.kv_dtype == "bf16":
        return O.decode_bf16(inp.k), O.decode_bf16(inp.v)
    return O.dequant_rows(inp.k, "fp8", inp.k_scale), O.dequant_rows(inp.v, "fp8", inp.v_scale)


def _run_sparse(dsa, inp, idx, k, out_dtype, sink=None):
    T, L = inp.T, inp.L
    f32 = out_dtype == "f32"
    out = torch.full((T, 8, 128), float("nan"), dtype=torch.float32 if f32 else torch.bfloat16, device=DEV)
    ws = dsa.workspace(dsa.WS_SPARSE_ATTN, T, L, k)
    fp8 = inp.kv_dtype == "fp8"
    dsa.dsa_sparse_attn(up(inp.q), up(inp.k), up(inp.v), up(inp.k_scale) if fp8 else None,
                        up(inp.v_scale) if fp8 else None, dsa.FP8_E4M3 if fp8 else dsa.BF16, up(idx), k, T, L,
                        SM, None if sink is None else up(sink), out, dsa.FP32 if f32 else dsa.BF16, ws)
    torch.cuda.synchronize()
    if f32:
        return down(out).astype(np.float64)
    return O.decode_bf16(bf16_bits(out))


def _check_attn(got, ref, out_dtype):
    if out_dtype == "f32":
        T, H, _ = ref.shape
        for t in range(T):
            for h in range(H):
                den = max(np.max(np.abs(ref[t, h])), 1e-30)
                assert np.max(np.abs(got[t, h] - ref[t, h])) / den <= 1e-5, (t, h)
    else:
        assert np.max(np.abs(got - ref)) <= 2e-2


@pytest.mark.parametrize("name,L,out_dtype,with_sink", [
    ("tiny", None, "f32", False), ("verify64k", 20000, "f32", False), ("verify64k", 20000, "bf16", False),
    ("verify256k_fp8", 30000, "f32", False), ("verify256k_fp8", 30000, "bf16", True),
    ("verify64k", 3000, "f32", True)])
def test_sparse_attention_vs_oracle(dsa, name, L, out_dtype, with_sink):
    inp = synth.dsa_config(name, seed=2, L=L)
    k = inp.top_k
    g = np.random.default_rng(9)
    idx = np.full((inp.T, k), -1, np.int32)
    for t in range(inp.T):
        vis = inp.pos0 + t + 1
        n = min(k, vis)
        idx[t, :n] = np.sort(g.choice(vis, n, replace=False))
    sink = synth.sink_logits(2) if with_sink else None
    got = _run_sparse(dsa, inp, idx, k, out_dtype, sink)
    K, V = _attn_inputs(inp)
    ref = O.sparse_attention(O.decode_bf16(inp.q), K, V, idx, SM, sink)
    _check_attn(got, ref, out_dtype)


def test_sparse_attention_fp8_cache_full_256k(dsa):
    """The 256K verify config at its stated size: e4m3 indexer keys and e4m3 K/V with row
    scales; attention over the fused selection's own indices against the oracle."""
    inp = synth.dsa_config("verify256k_fp8", seed=0)
    T, L, k = inp.T, inp.L, inp.top_k
    idx = torch.full((T, k), -7, dtype=torch.int32, device=DEV)
    ws = dsa.workspace(dsa.WS_INDEX_TOPK, T, L, k)
    dsa.dsa_index_topk(up(inp.q_idx), up(inp.w_idx), up(inp.k_idx), up(inp.k_idx_scale), dsa.FP8_E4M3, T, L,
                       inp.pos0, k, idx, None, ws)
    torch.cuda.synchronize()
    gi = down(idx)
    assert np.all((gi >= 0).sum(axis=1) == k)
    K, V = _attn_inputs(inp)
    ref = O.sparse_attention(O.decode_bf16(inp.q), K, V, gi, SM)
    for out_dtype in ("f32", "bf16"):
        _check_attn(_run_sparse(dsa, inp, gi, k, out_dtype), ref, out_dtype)


def test_sparse_attention_ragged_lists(dsa):
    """Skipped entries (-1, >= L), duplicates, a short list, an empty token row."""
    inp = synth.dsa_config("verify64k", seed=4, L=2000, T=4)
    k = 150
    g = np.random.default_rng(1)
    idx = g.integers(0, inp.L, (inp.T, k)).astype(np.int32)
    idx[0, ::3] = -1
    idx[1, ::5] = inp.L + 7
    idx[2, :] = 11                        # one row repeated
    idx[3, :] = -1                        # nothing to attend
    got = _run_sparse(dsa, inp, idx, k, "f32")
    K, V = _attn_inputs(inp)
    ref = O.sparse_attention(O.decode_bf16(inp.q), K, V, idx, SM)
    np.testing.assert_allclose(got[3], 0.0)
    _check_attn(got[:3], ref[:3], "f32")
    # a -inf sink is no sink
    got2 = _run_sparse(dsa, inp, idx, k, "f32", np.full(8, -np.inf, np.float32))
    assert np.array_equal(got, got2)


def test_sparse_attention_fp8_values_all_codes(dsa):
    """A single selected row: the output is that row's decoded V exactly (fp32)."""
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    rows = (len(codes) + 127) // 128
    L = rows
    V = np.zeros((L, 128), np.uint8)
    V.reshape(-1)[:len(codes)] = codes
    K = np.zeros((L, 128), np.uint8)
    vs = np.full(L, 0.25, np.float32)
    ks = np.ones(L, np.float32)
    q = synth.to_bf16_bits(np.ones((L, 8, 128), np.float32))
    idx = np.arange(L, dtype=np.int32)[:, None].repeat(1, axis=1)
    out = torch.zeros((L, 8, 128), dtype=torch.float32, device=DEV)
    ws = dsa.workspace(dsa.WS_SPARSE_ATTN, L, L, 1)
    dsa.dsa_sparse_attn(up(q), up(K), up(V), up(ks), up(vs), dsa.FP8_E4M3, up(idx), 1, L, L, SM, None, out,
                        dsa.FP32, ws)
    torch.cuda.synchronize()
    got = down(out)
    want = O.decode_e4m3(V) * 0.25
    for t in range(L):
        for h in range(8):
            assert np.array_equal(got[t, h].astype(np.float64), want[t])


@pytest.mark.parametrize("pos0,T,window,cap,kv", [(5000, 8, 128, 135, "bf16"), (3, 4, 128, 140, "bf16"),
                                                  (1000, 1, 1, 8, "bf16"), (70, 8, 128, 256, "bf16"),
                                                  (5000, 8, 300, 320, "bf16"), (200, 3, 129, 140, "bf16"),
                                                  (5000, 8, 128, 135, "fp8"), (1048568, 8, 128, 256, "fp8"),
                                                  (40, 5, 300, 320, "fp8")])
def test_swa_vs_oracle(dsa, pos0, T, window, cap, kv):
    g = np.random.default_rng(pos0)
    Kf = g.standard_normal((cap, 128)).astype(np.float32)
    Vf = g.standard_normal((cap, 128)).astype(np.float32)
    if kv == "bf16":
        Kr, Vr, ks, vs = synth.to_bf16_bits(Kf), synth.to_bf16_bits(Vf), None, None
        K64, V64 = O.decode_bf16(Kr), O.decode_bf16(Vr)
    else:
        (Kr, ks), (Vr, vs) = synth.to_e4m3_rows(Kf), synth.to_e4m3_rows(Vf)
        K64, V64 = O.dequant_rows(Kr, "fp8", ks), O.dequant_rows(Vr, "fp8", vs)
    q = synth.to_bf16_bits(g.standard_normal((T, 8, 128)).astype(np.float32))
    for sink in (None, synth.sink_logits(5)):
        out = torch.full((T, 8, 128), float("nan"), dtype=torch.float32, device=DEV)
        ws = dsa.workspace(dsa.WS_SWA_ATTN, T, pos0 + T, window)
        dsa.swa_attn(up(q), up(Kr), up(Vr), None if ks is None else up(ks), None if vs is None else up(vs),
                     dsa.BF16 if kv == "bf16" else dsa.FP8_E4M3, cap, T, pos0, window, SM,
                     None if sink is None else up(sink), out, dsa.FP32, ws)
        torch.cuda.synchronize()
        ref = O.swa_attention(O.decode_bf16(q), K64, V64, cap, pos0, window, SM, sink)
        _check_attn(down(out).astype(np.float64), ref, "f32")


def test_attention_run_to_run_bitwise(dsa):
    inp = synth.dsa_config("verify64k", seed=6, L=30000)
    k = inp.top_k
    g = np.random.default_rng(2)
    idx = np.sort(np.stack([g.choice(inp.pos0 + 1, k, replace=False) for _ in range(inp.T)]), axis=1)
    a = _run_sparse(dsa, inp, idx.astype(np.int32), k, "f32")
    for _ in range(3):
        b = _run_sparse(dsa, inp, idx.astype(np.int32), k, "f32")
        assert np.array_equal(a, b)


@pytest.mark.parametrize("nbytes", [16, 4096 + 48, (1 << 20) + 16 * 777, 64 << 20])
def test_read_ceiling_stream_folds_every_word(dsa, nbytes):
    """The benchmark's bandwidth helper (its own library) reads every 16-byte word exactly
    once: the xor of the per-workgroup folds equals the host's xor of all 32-bit words."""
    import ctypes as C
    import os
    lib = C.CDLL(os.path.join(os.path.dirname(dsa.LIB_PATH), "libdsa_read_ceiling.so"))
    fn = lib.dsa_read_ceiling_stream
    fn.argtypes = [C.c_void_p, C.c_size_t, C.c_void_p, C.c_void_p]
    fn.restype = C.c_int
    g = np.random.default_rng(nbytes)
    words = g.integers(0, 2 ** 32, size=nbytes // 4, dtype=np.uint64).astype(np.uint32)
    src = up(words.view(np.int32))
    sink = torch.zeros(1024, dtype=torch.int32, device=DEV)
    assert fn(src.data_ptr(), nbytes, sink.data_ptr(), torch.cuda.current_stream().cuda_stream) == 0
    torch.cuda.synchronize()
    fold = np.bitwise_xor.reduce(down(sink).view(np.uint32))
    assert fold == np.bitwise_xor.reduce(words)


# ----------------------------------------------------------------------------- failure reporting

def test_workspace_status_reports_a_set_error_word_and_poisons_the_workspace(dsa):
    """The error word is set from the host (standing in for a launch that gave up): the
    status call reports DSA_ERR_LAUNCH, selection calls on the workspace write empty
    selections, and after dsa_workspace_init the workspace selects correctly again."""
    inp = synth.dsa_config("tiny", seed=0)
    T, L, k = inp.T, inp.L, inp.top_k
    ws = dsa.workspace(dsa.WS_INDEX_TOPK, T, L, k)
    assert dsa.dsa_workspace_status(ws) == 0
    ws.view(torch.int32)[769] = 1                      # the sticky error word
    E = {v: kk for kk, v in dsa.STATUS.items()}
    assert dsa.dsa_workspace_status(ws, raise_on_error=False) == E["DSA_ERR_LAUNCH"]
    assert "not valid" in dsa.dsa_last_error()
    idx = torch.full((T, k), -7, dtype=torch.int32, device=DEV)
    cnt = torch.full((T,), -7, dtype=torch.int32, device=DEV)
    args = (up(inp.q_idx), up(inp.w_idx), up(inp.k_idx), None, dsa.BF16, T, L, inp.pos0, k, idx, cnt, ws)
    dsa.dsa_index_topk(*args)
    torch.cuda.synchronize()
    assert np.all(down(idx) == -1) and np.all(down(cnt) == 0)
    assert dsa.dsa_workspace_status(ws, raise_on_error=False) == E["DSA_ERR_LAUNCH"]
    dsa.dsa_workspace_init(ws)
    assert dsa.dsa_workspace_status(ws) == 0
    dsa.dsa_index_topk(*args)
    torch.cuda.synchronize()
    s_ref = O.indexer_scores(O.decode_bf16(inp.q_idx), inp.w_idx, O.decode_bf16(inp.k_idx), inp.pos0)
    ridx, rcnt = O.topk_indices(s_ref, inp.pos0, k)
    assert np.array_equal(down(idx), ridx) and np.array_equal(down(cnt), rcnt)
    assert dsa.dsa_workspace_status(ws) == 0


def test_resident_limit_hook_refuses_before_launching(dsa, monkeypatch):
    """With fewer resident workgroups than the selection needs, the selection calls and the
    DSA layer step return DSA_ERR_LAUNCH before writing anything (outputs and cache rows
    keep their values)."""
    E = {v: kk for kk, v in dsa.STATUS.items()}
    inp = synth.dsa_config("verify1m", seed=1, L=200000, T=8)
    T, L, k = inp.T, inp.L, inp.top_k
    ws = dsa.workspace(dsa.WS_INDEX_TOPK, T, L, k)
    idx = torch.full((T, k), -7, dtype=torch.int32, device=DEV)
    monkeypatch.setenv("DSA_RESIDENT_LIMIT", "3")
    st = dsa.dsa_index_topk(up(inp.q_idx), up(inp.w_idx), up(inp.k_idx), up(inp.k_idx_scale), dsa.FP8_E4M3, T, L,
                            inp.pos0, k, idx, None, ws, raise_on_error=False)
    assert st == E["DSA_ERR_LAUNCH"]
    sc = up(np.zeros((T, L), np.float32))
    st = dsa.dsa_topk(sc, T, L, L, inp.pos0, k, idx, None, dsa.workspace(dsa.WS_TOPK, T, L, k),
                      raise_on_error=False)
    assert st == E["DSA_ERR_LAUNCH"]
    torch.cuda.synchronize()
    assert np.all(down(idx) == -7)
    lay = synth.layer_inputs("dsa", 0, 20000, T, seed=3)
    kc, vc, ki, ks = up(lay.k), up(lay.v), up(lay.k_idx), up(lay.k_idx_scale)
    cache = dsa.LayerCache(kc.data_ptr(), vc.data_ptr(), ki.data_ptr(), ks.data_ptr(), lay.capacity)
    g_gamma, g_w, g_wo = up(lay.gamma), up(lay.w_qkvi), up(lay.w_o)
    w = dsa.LayerWeights(g_gamma.data_ptr(), g_w.data_ptr(), g_wo.data_ptr())
    x = up(synth.module_x(3, T))
    xo = torch.zeros_like(x)
    wsl = dsa.workspace(dsa.WS_LAYER_DSA, T, 20000, k)
    st = dsa.dsa_layer_step(dsa.layer_config(dsa.LAYER_DSA), w, cache, x, xo, T, 20000 - T, ws=wsl,
                            raise_on_error=False)
    assert st == E["DSA_ERR_LAUNCH"]
    torch.cuda.synchronize()
    assert np.array_equal(bf16_bits(kc), lay.k) and np.array_equal(down(ki), lay.k_idx)
    assert np.all(down(xo) == 0)
    monkeypatch.delenv("DSA_RESIDENT_LIMIT")
    dsa.dsa_layer_step(dsa.layer_config(dsa.LAYER_DSA), w, cache, x, xo, T, 20000 - T, ws=wsl)
    torch.cuda.synchronize()
    assert not np.array_equal(bf16_bits(kc), lay.k)
