"""Contexts longer than 4096 keys per CU: the fused selection keeps the first 4096 scores
of each workgroup's chunk in LDS and the rest in the workspace (materialised scores are
read again from the input).  The selection is defined by the exact top-k, so it must not
depend on the chunking: checked against the oracle, against the top-k of the GPU's own
materialised scores, and bit for bit against the same call cut into chunks that fit LDS.

Small contexts reach the long-chunk path through the DSA_NUM_CU test hook (the geometry
is cut for that many CUs, so L = 40000 on 4 CUs gives 10240-key chunks); one case runs
past 4096 x CUs on the whole device.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import dsa_oracle as O
from tests.gpu_util import DEV, up, down, bf16_bits, tie_band_ok

pytestmark = pytest.mark.gpu

LDS_CHUNK = 4096


@pytest.fixture(scope="module")
def dsa():
    import sparse_attention_decode_indexer_amd as m
    assert torch.cuda.is_available()
    return m


def _chunk(L, ncu):
    per = -(-L // ncu)
    return max(512, -(-per // 512) * 512)


def _kdt(dsa, inp):
    return dsa.BF16 if inp.k_idx_dtype == "bf16" else dsa.FP8_E4M3


def _index_topk(dsa, inp, T, L, pos0, k):
    idx = torch.full((T, k), -7, dtype=torch.int32, device=DEV)
    cnt = torch.full((T,), -7, dtype=torch.int32, device=DEV)
    ws = dsa.workspace(dsa.WS_INDEX_TOPK, T, L, k)
    kscale = up(inp.k_idx_scale) if inp.k_idx_scale is not None else None
    dsa.dsa_index_topk(up(inp.q_idx), up(inp.w_idx), up(inp.k_idx), kscale, _kdt(dsa, inp), T, L, pos0, k, idx, cnt,
                       ws)
    torch.cuda.synchronize()
    assert dsa.dsa_workspace_status(ws) == 0
    return down(idx), down(cnt)


def _gpu_scores(dsa, inp, T, L, pos0):
    ld = (L + 3) // 4 * 4
    sc = torch.full((T, ld), float("nan"), dtype=torch.float32, device=DEV)
    kscale = up(inp.k_idx_scale) if inp.k_idx_scale is not None else None
    dsa.dsa_indexer_scores(up(inp.q_idx), up(inp.w_idx), up(inp.k_idx), kscale, _kdt(dsa, inp), T, L, pos0, sc, ld)
    torch.cuda.synchronize()
    return down(sc)[:, :L]


def _gpu_topk(dsa, s, pos0, k):
    T, L = s.shape
    ld = (L + 3) // 4 * 4
    buf = np.full((T, ld), -np.inf, np.float32)
    buf[:, :L] = s
    idx = torch.full((T, k), -7, dtype=torch.int32, device=DEV)
    cnt = torch.full((T,), -7, dtype=torch.int32, device=DEV)
    ws = dsa.workspace(dsa.WS_TOPK, T, L, k)
    dsa.dsa_topk(up(buf), T, L, ld, pos0, k, idx, cnt, ws)
    torch.cuda.synchronize()
    return down(idx), down(cnt)


# (config, L, T, seed, tie-stress, CUs the geometry is cut for, pos0: "end" = L - T, "mid" = L // 2)
CASES = [
    ("tiny", 40000, 8, 0, False, 4, "end"),
    ("tiny", 40000, 8, 1, True, 4, "end"),
    ("tiny", 50001, 3, 2, False, 3, "mid"),
    ("tiny", 20000, 1, 3, False, 1, "end"),
    ("verify64k", 30000, 5, 0, False, 2, "end"),
    ("verify256k_fp8", 50000, 8, 1, False, 4, "end"),
    ("verify1m", 70000, 8, 3, False, 4, "mid"),
    # edges: one key past the LDS part (4608-key chunk, 511 masked spill slots); the longest
    # chunk (65536 keys) with an empty second workgroup; a T = 1 longest chunk on e4m3 keys;
    # a ragged context whose tokens outnumber the chunks (five empty workgroups, no bound)
    ("tiny", 4097, 1, 4, False, 1, "end"),
    ("tiny", 65536, 2, 5, True, 1, "end"),
    ("verify256k_fp8", 65536, 1, 7, False, 1, "end"),
    ("verify64k", 12345, 7, 6, False, 2, "mid"),
]


@pytest.mark.parametrize("name,L,T,seed,tie,ncu,where", CASES)
def test_index_topk_long_chunks(dsa, monkeypatch, name, L, T, seed, tie, ncu, where):
    """Fused scan + top-k over chunks longer than 4096 keys: equal to the selection over
    LDS-sized chunks bit for bit, to top-k of the GPU's materialised scores bit for bit,
    and to the oracle's (bit for bit on integer-valued inputs, else within the rounding
    band)."""
    assert _chunk(L, ncu) > LDS_CHUNK            # the long-chunk path is the one under test
    inp = synth.dsa_config(name, seed=seed, L=L, T=T, tie_stress=tie)
    k = inp.top_k
    pos0 = L - T if where == "end" else L // 2
    monkeypatch.delenv("DSA_NUM_CU", raising=False)
    ref_idx, ref_cnt = _index_topk(dsa, inp, T, L, pos0, k)             # chunks that fit LDS
    assert _chunk(L, 256) <= LDS_CHUNK
    monkeypatch.setenv("DSA_NUM_CU", str(ncu))
    idx, cnt = _index_topk(dsa, inp, T, L, pos0, k)
    assert np.array_equal(idx, ref_idx) and np.array_equal(cnt, ref_cnt), "selection depends on the chunking"
    g = _gpu_scores(dsa, inp, T, L, pos0)
    gi, gc = O.topk_indices(g.astype(np.float64), pos0, k)
    assert np.array_equal(idx, gi) and np.array_equal(cnt, gc), "differs from top-k of the GPU scores"
    krows = O.dequant_rows(inp.k_idx, inp.k_idx_dtype, inp.k_idx_scale)
    r, S = O.indexer_scores(O.decode_bf16(inp.q_idx), inp.w_idx, krows, pos0, with_abs=True)
    ridx, rcnt = O.topk_indices(r, pos0, k)
    assert np.array_equal(cnt, rcnt)
    if name == "tiny":
        assert np.array_equal(idx, ridx)
    else:
        ok, ndiff = tie_band_ok(idx, ridx, r, S, pos0, k)
        assert ok, f"selection differs outside the rounding band ({ndiff})"


def _cut_ties(g, s, k, n):
    s = s.astype(np.float32)
    T, L = s.shape
    for t in range(T):
        v = np.sort(s[t, : L - T])[-k]
        s[t, g.choice(L - T, n, replace=False)] = v
    return s


TOPK_CASES = [
    ("normal", 8, 20000, 2048, "end", lambda g, T, L: g.standard_normal((T, L)).astype(np.float32)),
    ("cut-ties", 8, 30000, 2048, "end", lambda g, T, L: _cut_ties(g, g.standard_normal((T, L)), 2048, 9)),
    ("ints", 4, 25000, 1000, "mid", lambda g, T, L: g.integers(-3, 30, (T, L)).astype(np.float32)),
    ("late-runs", 3, 33333, 2048, "end",
     lambda g, T, L: np.where(np.arange(L) > 9000, 5 + g.random((T, L)), g.random((T, L))).astype(np.float32)),
    # one position past the LDS part of the first chunk (4608-key chunks)
    ("edge-8193", 1, 8193, 2048, "end", lambda g, T, L: g.standard_normal((T, L)).astype(np.float32)),
    # the longest chunks (65536 positions) at the context limit of two CUs, six empty workgroups
    ("longest", 8, 131072, 2048, "end", lambda g, T, L: g.standard_normal((T, L)).astype(np.float32)),
]


@pytest.mark.parametrize("case", TOPK_CASES, ids=[c[0] for c in TOPK_CASES])
def test_topk_long_chunks_on_given_scores(dsa, monkeypatch, case):
    """Top-k of given scores over chunks longer than 4096 positions (the positions past the
    first 4096 of each chunk are read again from the score rows): bit-exact against the
    oracle, ties by lower position included."""
    name, T, L, k, where, gen = case
    monkeypatch.setenv("DSA_NUM_CU", "2")
    assert _chunk(L, 2) > LDS_CHUNK
    s = gen(np.random.default_rng(11), T, L)
    pos0 = L - T if where == "end" else L // 3
    idx, cnt = _gpu_topk(dsa, s, pos0, k)
    ridx, rcnt = O.topk_indices(s.astype(np.float64), pos0, k)
    assert np.array_equal(cnt, rcnt)
    assert np.array_equal(idx, ridx)


def test_dsa_layer_step_long_chunks_equals_lds_chunks(dsa, monkeypatch):
    """A whole DSA layer step whose selection runs over 10240-key chunks produces the same
    bits (layer output, projections, cache rows, indices) as over LDS-sized chunks."""
    from tests.test_gpu_layer import _run_layer
    T, L = 8, 40000
    pos0 = L - T
    lay = synth.layer_inputs("dsa", 5, L, T, seed=7)
    x = synth.module_x(7, T)
    monkeypatch.delenv("DSA_NUM_CU", raising=False)
    a = _run_layer(dsa, "dsa", lay, x, T, pos0)
    monkeypatch.setenv("DSA_NUM_CU", "4")
    b = _run_layer(dsa, "dsa", lay, x, T, pos0)
    for key in ("x_out", "qkv", "k", "v", "idx", "k_idx", "k_idx_scale"):
        assert np.array_equal(a[key], b[key]), key


def test_index_topk_past_lds_context_whole_device(dsa, monkeypatch):
    """Twice the context the LDS holds on this device (8192-key chunks on 256 CUs), integer
    bf16 indexer inputs (exact scores): the fused selection equals the oracle's top-k of
    the materialised scores bit for bit, and those scores equal the oracle's on sampled
    columns."""
    monkeypatch.delenv("DSA_NUM_CU", raising=False)
    L = 2 * int(dsa.dsa_max_context() // 16) + 3000    # 2 x 4096 x CUs + a ragged tail
    T = 8
    inp = synth.dsa_config("tiny", seed=5, L=L, T=T)
    pos0 = L - T
    idx, cnt = _index_topk(dsa, inp, T, L, pos0, inp.top_k)
    g = _gpu_scores(dsa, inp, T, L, pos0)
    gi, gc = O.topk_indices(g.astype(np.float64), pos0, inp.top_k)
    assert np.array_equal(idx, gi) and np.array_equal(cnt, gc)
    rng = np.random.default_rng(5)
    cols = np.unique(np.concatenate([rng.choice(L, 3000, replace=False), np.arange(L - 64, L),
                                     idx[idx >= 0][:2000]]))
    krows = O.decode_bf16(inp.k_idx[cols])
    r = O.indexer_scores(O.decode_bf16(inp.q_idx), inp.w_idx, krows, len(cols) - 1)
    for t in range(T):
        vis = cols <= pos0 + t
        assert np.array_equal(g[t, cols[vis]].astype(np.float64), r[t, vis])
        assert np.all(np.isneginf(g[t, cols[~vis]]))
