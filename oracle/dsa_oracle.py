"""Plain fp64 CPU oracle for one decode/verify step of a DSA layer.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  The
library's product path never touches it, and it shares no code, table or
helper with the HIP kernels.

What it computes follows NaiveAI research page on Naive-N0.5-Flash (naive.ai/en/research):

* §Model Architecture: a lightweight indexer scores the whole history; the
  backbone attends only a selected subset of positions.
* §Hybrid SWA-DSA Architecture: DSA keeps the top 2,048 positions, SWA uses a
  128-token window, the indexer has 16 query heads, attention is GQA.
* §A DSA layer: from 29 kernels to one: the per-step stage list (input
  RMSNorm, Q/K/V projections, RoPE, KV-cache writes, indexer GEMM, top-k,
  sparse gather, attention, output projection).
* §GPU Memory Optimization: positional-encoding precision at 1M context, so
  rotary angles are formed in fp64 here.

The pages give no scoring formula; the oracle uses
``I[t,s] = sum_h w[t,h] * relu(scale_s * (q_I[t,h] . k_I[s]))`` with the top-k
ranking (score descending, position ascending).  Every reading of a point the
pages leave open is listed in the repository's design notes.

All arithmetic is fp64 on exactly decoded inputs.  Library primitives used as
steps: ``numpy.matmul`` (dot products), ``numpy.lexsort`` (the sort that *is*
the top-k definition), ``numpy.exp``/``cos``/``sin``.

Parity status: every function here is pinned by ``tests/test_oracle_pins.py``
(closed forms, brute force, library routines, invariants), including the band
magnitude S of ``indexer_scores`` (hand-derived example, sign invariance, equality
with the score on non-negative inputs).  Within the composed layer step the DSA
indexer leg is pinned on its own: q_I and k_I rotated by absolute position (a shift
of the block multiplies every pair by the shift's rotation), w_I not rotated, the
block's own keys read back quantised, and the block's scores invariant under a shift
within the quantiser bound.  Beyond the pinned stages and special cases with closed
forms, the end-to-end layer step is unpinned (the pages print no worked example).
``module_step`` (layers in order) is pinned by layers made the identity (zero output
projection): the chain must hand each layer the previous layer's output.
"""
from __future__ import annotations

import math
import numpy as np

# ----------------------------------------------------------------------------
# number formats


def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact fp64 values."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def decode_e4m3(codes: np.ndarray) -> np.ndarray:
    """OCP FP8 e4m3fn codes (uint8) -> exact fp64 values.

    Layout S.EEEE.MMM, exponent bias 7, no infinities, S.1111.111 is NaN,
    E=0 encodes subnormals m/8 * 2^-6, largest finite 448.
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    sub = (m / 8.0) * 2.0 ** -6
    val = np.where(e == 0, sub, normal)
    val = np.where((e == 15) & ((c & 7) == 7), np.nan, val)
    return sign * val


# the 127 non-negative finite e4m3 magnitudes, by code
_E4M3_MAG = decode_e4m3(np.arange(127, dtype=np.uint8))


def encode_e4m3(x: np.ndarray) -> np.ndarray:
    """fp32 values -> e4m3fn codes, round to nearest (ties to even code), saturating at 448.

    Written from the format definition: pick the nearest representable
    magnitude; on an exact tie take the code whose last mantissa bit is 0.
    Magnitudes above 448 become 448.  Inputs must be finite.
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), 448.0)
    hi = np.searchsorted(_E4M3_MAG, a, side="left")     # first magnitude >= a
    hi = np.minimum(hi, 126)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _E4M3_MAG[lo]
    d_hi = _E4M3_MAG[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(_E4M3_MAG[hi] == a, hi, code)
    sign = (np.signbit(x)).astype(np.int64) << 7
    return (code | sign).astype(np.uint8)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """fp64 -> bf16 bit patterns, one rounding (nearest, ties to even). Finite inputs."""
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros(x.shape, dtype=np.uint16)
    flat = x.reshape(-1)
    o = out.reshape(-1)
    for i, v in enumerate(flat):
        if v == 0.0:
            o[i] = 0x8000 if math.copysign(1.0, v) < 0 else 0
            continue
        m, e = math.frexp(abs(v))          # v = m * 2^e, m in [0.5, 1)
        # bf16 normal: 8 significant bits -> quantum 2^(e-8); below 2^-126 subnormal quantum 2^-133
        q_exp = max(e - 8, -133)
        q = math.ldexp(1.0, q_exp)
        r = abs(v) / q                       # exact (power-of-two scaling)
        f = math.floor(r)
        rem = r - f
        if rem > 0.5 or (rem == 0.5 and (int(f) & 1)):
            f += 1
        mag = np.float32(f * q)              # exactly representable in bf16
        bits = int(np.array(mag, dtype=np.float32).view(np.uint32)) >> 16
        if v < 0:
            bits |= 0x8000
        o[i] = bits
    return out


def bf16_round_trip(x: np.ndarray) -> np.ndarray:
    """fp64 -> nearest bf16 -> fp64."""
    return decode_bf16(round_to_bf16(x))


def f32(x) -> np.ndarray:
    """fp64 -> fp32 (nearest, ties to even) -> fp64."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


# ----------------------------------------------------------------------------
# indexer (§Model Architecture; §Hybrid SWA-DSA Architecture: 16 indexer heads)


def dequant_rows(values: np.ndarray, dtype: str, scale: np.ndarray | None) -> np.ndarray:
    """Cache rows in storage format -> fp64 rows (row scale applied for e4m3)."""
    if dtype == "bf16":
        return decode_bf16(values)
    if dtype == "fp8":
        return decode_e4m3(values) * np.asarray(scale, np.float64)[:, None]
    raise ValueError(dtype)


def indexer_scores(q_idx, w_idx, k_rows, pos0: int, with_abs: bool = False):
    """I[t,s] = sum_h w[t,h] * relu(q_I[t,h] . k_I[s]) for s <= pos0 + t, else -inf.

    q_idx: [T][H][D] fp64, w_idx: [T][H] fp64, k_rows: [L][D] fp64 (already
    multiplied by the row scale).  With ``with_abs`` also returns
    S[t,s] = sum_h |w| * sum_d |q * k|, the magnitude that bounds the rounding
    error of any summation order.
    """
    q_idx = np.asarray(q_idx, np.float64)
    w_idx = np.asarray(w_idx, np.float64)
    k_rows = np.asarray(k_rows, np.float64)
    T = q_idx.shape[0]
    L = k_rows.shape[0]
    out = np.full((T, L), -np.inf)
    mag = np.zeros((T, L)) if with_abs else None
    for t in range(T):
        vis = pos0 + t + 1
        d = q_idx[t] @ k_rows[:vis].T                 # [H, vis]
        out[t, :vis] = w_idx[t] @ np.maximum(d, 0.0)
        if with_abs:
            mag[t, :vis] = np.abs(w_idx[t]) @ (np.abs(q_idx[t]) @ np.abs(k_rows[:vis]).T)
    return (out, mag) if with_abs else out


# ----------------------------------------------------------------------------
# top-k (§Hybrid SWA-DSA Architecture: top 2,048; §GPU Memory Optimization:
# indices are an explicit, retained result)


def topk_indices(scores: np.ndarray, pos0: int, k: int):
    """Per token, the min(k, pos0+t+1) visible positions ranked first by
    (score descending, position ascending), listed by ascending position and
    padded with -1.  Returns (idx [T][k] int32, count [T] int32).

    Equal scores compare equal (so -0 ties +0); the sort is the plain
    definition of the selection.
    """
    scores = np.asarray(scores)
    T = scores.shape[0]
    idx = np.full((T, k), -1, np.int32)
    cnt = np.zeros(T, np.int32)
    for t in range(T):
        vis = pos0 + t + 1
        s = scores[t, :vis].astype(np.float64) + 0.0      # -0 -> +0
        pos = np.arange(vis)
        order = np.lexsort((pos, -s))                     # primary: -score, then position
        n = min(k, vis)
        sel = np.sort(order[:n])
        idx[t, :n] = sel
        cnt[t] = n
    return idx, cnt


# ----------------------------------------------------------------------------
# attention (§Hybrid SWA-DSA Architecture: GQA, sink bias; §Model Architecture:
# attention over the selected subset only)


def _softmax_rows(z: np.ndarray, sink: np.ndarray | None):
    """Row softmax in fp64; a sink logit joins the denominator and carries no value."""
    m = np.max(z, axis=-1) if z.shape[-1] else np.full(z.shape[:-1], -np.inf)
    if sink is not None:
        m = np.maximum(m, sink)
    m = np.where(np.isfinite(m), m, 0.0)
    e = np.exp(z - m[..., None])
    den = e.sum(axis=-1)
    if sink is not None:
        den = den + np.exp(sink - m)
    return e, den


def attend_rows(q, K_rows, V_rows, sm_scale: float, sink=None):
    """One token: q [H][D], K_rows/V_rows [n][D] (fp64) -> [H][D].

    out_h = sum_j exp(z_hj - m) V_j / (sum_j exp(z_hj - m) [+ exp(sink_h - m)]),
    z_hj = sm_scale * q_h . K_j.  No rows (and no sink) gives 0.
    """
    q = np.asarray(q, np.float64)
    H, D = q.shape
    if K_rows.shape[0] == 0:
        return np.zeros((H, D))
    z = sm_scale * (q @ np.asarray(K_rows, np.float64).T)        # [H, n]
    e, den = _softmax_rows(z, None if sink is None else np.asarray(sink, np.float64))
    num = e @ np.asarray(V_rows, np.float64)                      # [H, D]
    return num / den[:, None]


def _rows(src, j):
    """Rows j of a row source: an fp64 array, or a callable returning fp64 rows."""
    return src(j) if callable(src) else np.asarray(src, np.float64)[j]


def sparse_attention(q, K, V, idx, sm_scale: float, sink=None, L: int | None = None):
    """q [T][H][D] fp64; K/V row sources of length L (fp64 [L][D] arrays or
    callables mapping an index array to fp64 rows); idx [T][k] int, entries
    outside [0, L) skipped."""
    q = np.asarray(q, np.float64)
    T = q.shape[0]
    if L is None:
        L = K.shape[0]
    out = np.zeros(q.shape)
    for t in range(T):
        j = np.asarray(idx[t])
        j = np.sort(j[(j >= 0) & (j < L)])
        out[t] = attend_rows(q[t], _rows(K, j), _rows(V, j), sm_scale, sink)
    return out


def swa_attention(q, K_ring, V_ring, ring_cap: int, pos0: int, window: int,
                  sm_scale: float, sink=None):
    """Sliding window: token t at p = pos0+t attends positions [max(0, p-window+1), p];
    position p lives in ring slot p % ring_cap."""
    q = np.asarray(q, np.float64)
    out = np.zeros(q.shape)
    for t in range(q.shape[0]):
        p = pos0 + t
        pos = np.arange(max(0, p - window + 1), p + 1)
        slots = pos % ring_cap
        out[t] = attend_rows(q[t], K_ring[slots], V_ring[slots], sm_scale, sink)
    return out


# ----------------------------------------------------------------------------
# layer stages (§A DSA layer: from 29 kernels to one)


def rmsnorm(x, gamma, eps: float):
    """y = x / sqrt(mean(x^2) + eps) * gamma, row-wise, fp64."""
    x = np.asarray(x, np.float64)
    r = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    return x * r * np.asarray(gamma, np.float64)


def rope_cos_sin(positions, dim: int, theta: float):
    """Rotate-half tables: inv_freq_i = theta^(-2i/dim), angle = pos * inv_freq
    formed in fp64, cos/sin evaluated in fp64 then rounded to fp32.
    Returns (cos, sin) fp64 arrays [len(positions)][dim/2] holding fp32 values."""
    pos = np.asarray(positions, np.float64)
    i = np.arange(dim // 2, dtype=np.float64)
    inv = theta ** (-2.0 * i / dim)
    ang = pos[:, None] * inv[None, :]
    return f32(np.cos(ang)), f32(np.sin(ang))


def rope(x, positions, theta: float):
    """Rotate-half RoPE on the last dim of x [T][nh][d] fp64: pairs (i, i+d/2)."""
    x = np.asarray(x, np.float64)
    d = x.shape[-1]
    c, s = rope_cos_sin(positions, d, theta)
    c = c[:, None, :]
    s = s[:, None, :]
    a, b = x[..., : d // 2], x[..., d // 2:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def quantize_rows_e4m3(rows):
    """Per-row e4m3 quantisation of fp64 rows holding bf16 values:
    scale = fp32(amax / 448) (1 if amax == 0), code = e4m3(fp32(x / scale)).
    Returns (codes uint8, scale fp32)."""
    rows = np.asarray(rows, np.float64)
    amax = np.max(np.abs(rows), axis=-1)
    scale = np.where(amax > 0, f32(amax / 448.0), 1.0)
    qv = f32(rows / scale[:, None])
    return encode_e4m3(qv), scale.astype(np.float32)


def project(y, W):
    """y [T][K] fp64 times W [N][K] (out-features major) -> [T][N] fp64."""
    return np.asarray(y, np.float64) @ np.asarray(W, np.float64).T


# W8A8 projections (§How it was built: W8A8 kernels; §Get NaiveRT: W8A8 checkpoint).
# The pages fix no granularity; the reading here is one fp32 scale per weight row and
# one per token of the projection input, formed from the token's largest magnitude.


def quantize_tokens_w8a8(rows):
    """Per-token e4m3 quantisation of a projection input (fp64 rows holding bf16 values):
    amax = max |y|; scale = fp32(amax / 448); inv = fp32(448 / amax) (both 1 when
    amax = 0); code = e4m3(fp32(y * inv)), nearest even, saturating.
    Returns (codes uint8 [T][K], scale fp32 [T]); y ~ decode(code) * scale."""
    rows = np.asarray(rows, np.float64)
    amax = np.max(np.abs(rows), axis=-1)
    nz = amax > 0
    safe = np.where(nz, amax, 1.0)
    scale = np.where(nz, f32(safe / 448.0), 1.0)
    inv = np.where(nz, f32(448.0 / safe), 1.0)
    return encode_e4m3(f32(rows * inv[:, None])), scale.astype(np.float32)


def project_w8a8(y, w_codes, w_scale):
    """W8A8 product: y [T][K] (bf16 values) quantised per token, W as e4m3 codes [N][K]
    with row scales [N].  Returns fp64 [T][N] = s_y[t] * s_w[n] * sum_k a[t,k] * b[n,k]
    with a, b the decoded codes.  Every product of two e4m3 values is exact in fp64 and
    all of them lie within 2^48 of each other, so the fp64 sum is exact in any order."""
    codes, s_y = quantize_tokens_w8a8(y)
    acc = decode_e4m3(codes) @ decode_e4m3(w_codes).T
    return acc * np.asarray(s_y, np.float64)[:, None] * np.asarray(w_scale, np.float64)[None, :]


# column layout of the fused projection output (per layer)
def proj_layout(kind: str, H_q=8, D=128, H_I=16, D_I=64):
    lay = {"q": (0, H_q * D), "k": (H_q * D, D), "v": (H_q * D + D, D)}
    if kind == "dsa":
        o = H_q * D + 2 * D
        lay["q_idx"] = (o, H_I * D_I)
        lay["k_idx"] = (o + H_I * D_I, D_I)
        lay["w_idx"] = (o + H_I * D_I + D_I, H_I)
    return lay


def layer_step(kind: str, x_bits, gamma_bits, w_qkvi_bits, w_o_bits, cache: dict,
               pos0: int, *, eps=1e-6, theta=1e6, top_k=2048, window=128,
               H_q=8, D=128, H_I=16, D_I=64, sm_scale=None, teacher=None,
               w_qkvi_scale=None, w_o_scale=None):
    """One layer step with the rounding points of the bf16 path.

    kind "dsa": RMSNorm -> projection (Q|K|V|q_I|k_I|w_I) -> RoPE on Q, K, q_I, k_I
    -> append K, V (bf16) and k_I (e4m3 + row scale) at pos0..pos0+T-1 -> indexer
    over the cache (new rows read back quantised) -> top-k -> sparse attention ->
    output projection + residual.  kind "swa": Q|K|V only, ring-buffer append,
    window attention.

    ``cache`` holds fp64-decodable storage: for DSA keys k, v (bf16 bits [cap][D]),
    k_idx (codes [cap][D_I]), k_idx_scale ([cap] fp32); for SWA k, v rings and
    ring_cap.  It is updated in place.

    ``teacher`` (optional) supplies the GPU's own stage outputs so each stage is
    checked on identical inputs: keys "qkv" (post-RoPE projection, bf16 bits
    [T][N]), "idx" ([T][top_k]), "attn" (bf16 bits [T][H_q*D]).

    W8A8: with ``w_qkvi_scale`` and ``w_o_scale`` given, ``w_qkvi_bits`` and
    ``w_o_bits`` are e4m3 codes with those row scales and both projections are
    ``project_w8a8`` of their bf16 inputs (the normalised rows, the attention output).

    Returns a dict of every stage's result.
    """
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    x = decode_bf16(x_bits)
    T = x.shape[0]
    positions = np.arange(pos0, pos0 + T)
    res = {}
    # 1. RMSNorm -> bf16
    y = bf16_round_trip(rmsnorm(x, decode_bf16(gamma_bits), eps))
    res["normed"] = y
    # 2. projection -> bf16
    w8a8 = w_qkvi_scale is not None
    if w8a8 != (w_o_scale is not None):
        raise ValueError("W8A8 needs both weight scales")
    if w8a8:
        p = bf16_round_trip(project_w8a8(y, w_qkvi_bits, w_qkvi_scale))
    else:
        p = bf16_round_trip(project(y, decode_bf16(w_qkvi_bits)))
    lay = proj_layout(kind, H_q, D, H_I, D_I)
    # 3. RoPE on Q, K (and q_I, k_I for DSA) -> bf16
    def seg(name):
        o, n = lay[name]
        return p[:, o:o + n]
    post = p.copy()
    o, n = lay["q"]
    post[:, o:o + n] = bf16_round_trip(rope(seg("q").reshape(T, H_q, D), positions, theta)).reshape(T, n)
    o, n = lay["k"]
    post[:, o:o + n] = bf16_round_trip(rope(seg("k").reshape(T, 1, D), positions, theta)).reshape(T, n)
    if kind == "dsa":
        o, n = lay["q_idx"]
        post[:, o:o + n] = bf16_round_trip(
            rope(seg("q_idx").reshape(T, H_I, D_I), positions, theta)).reshape(T, n)
        o, n = lay["k_idx"]
        post[:, o:o + n] = bf16_round_trip(
            rope(seg("k_idx").reshape(T, 1, D_I), positions, theta)).reshape(T, n)
    res["qkv"] = post
    if teacher is not None and "qkv" in teacher:
        post = decode_bf16(teacher["qkv"])

    def seg2(name):
        o, n = lay[name]
        return post[:, o:o + n]
    q = seg2("q").reshape(T, H_q, D)
    k_new = seg2("k")
    v_new = seg2("v")
    # 4. append
    if kind == "dsa":
        cache["k"][pos0:pos0 + T] = round_to_bf16(k_new)
        cache["v"][pos0:pos0 + T] = round_to_bf16(v_new)
        codes, sc = quantize_rows_e4m3(seg2("k_idx"))
        cache["k_idx"][pos0:pos0 + T] = codes
        cache["k_idx_scale"][pos0:pos0 + T] = sc
        res["k_idx_codes"], res["k_idx_scale"] = codes, sc
        L = pos0 + T
        # 5. indexer over the cache, new rows read back quantised
        krows = dequant_rows(cache["k_idx"][:L], "fp8", cache["k_idx_scale"][:L])
        q_idx = seg2("q_idx").reshape(T, H_I, D_I)
        w_idx = seg2("w_idx")
        scores = indexer_scores(q_idx, w_idx, krows, pos0)
        res["scores"] = scores
        idx, cnt = topk_indices(scores, pos0, top_k)
        res["idx"], res["count"] = idx, cnt
        if teacher is not None and "idx" in teacher:
            idx = teacher["idx"]
        attn = sparse_attention(q, lambda j: decode_bf16(cache["k"][j]),
                                lambda j: decode_bf16(cache["v"][j]), idx, sm_scale, L=L)
    else:
        cap = cache["ring_cap"]
        for t in range(T):
            cache["k"][(pos0 + t) % cap] = round_to_bf16(k_new[t])
            cache["v"][(pos0 + t) % cap] = round_to_bf16(v_new[t])
        attn = swa_attention(q, decode_bf16(cache["k"]), decode_bf16(cache["v"]), cap,
                             pos0, window, sm_scale)
    attn = bf16_round_trip(attn.reshape(T, H_q * D))
    res["attn"] = attn
    if teacher is not None and "attn" in teacher:
        attn = decode_bf16(teacher["attn"])
    if w8a8:
        out = project_w8a8(attn, w_o_bits, w_o_scale) + x
    else:
        out = project(attn, decode_bf16(w_o_bits)) + x
    res["x_out"] = bf16_round_trip(out)
    res["x_out_f64"] = out
    return res


def module_step(layers, x_bits, pos0: int, **kw):
    """Decoder layers applied in order to one block of tokens (§The execution model: the
    layers of a decode step run back to back, each on the previous layer's output).

    ``layers``: list of dicts with keys kind, gamma, w_qkvi, w_o, cache (updated in place,
    as in ``layer_step``) and optional top_k, window.  Each layer takes the bf16 output
    of the one before it (``x_bits`` for the first).  Returns the last layer's output as
    bf16 bits and the list of every layer's ``layer_step`` result.
    """
    x = np.asarray(x_bits, dtype=np.uint16)
    results = []
    for lay in layers:
        r = layer_step(lay["kind"], x, lay["gamma"], lay["w_qkvi"], lay["w_o"], lay["cache"], pos0,
                       top_k=lay.get("top_k", 2048), window=lay.get("window", 128), **kw)
        results.append(r)
        x = round_to_bf16(r["x_out_f64"])
    return x, results
