"""Seeded synthetic inputs for the DSA decode/verify step.

This module only draws random tensors and stores them in the formats the
library consumes (bf16 bit patterns, OCP e4m3fn codes with a per-row fp32
scale, fp32).  It holds none of the method's arithmetic: no scoring, no
selection, no attention, no normalisation, no rotary embedding.  Format
conversions go through PyTorch's own casts (``torch.bfloat16``,
``torch.float8_e4m3fn``); the prefilled caches are quantised with one scale per
row chosen so that the row's largest magnitude maps onto the largest finite
e4m3 value (448), which is how a cache written by the layer itself looks.

Both the CPU oracle and the GPU path read these arrays; neither side's code
lives here.

Workloads (one GPU's share of a Naive-N0.5-Flash DSA layer: 8 query heads
sharing one KV head of width 128, a 16-head indexer of width 64, top-2048;
NaiveAI research page on Naive-N0.5-Flash (naive.ai/en/research),
§Hybrid SWA-DSA Architecture and §Optimizing inside the kernel):

  tiny      L=4096,  T=1, indexer q/k integers in [-4,4], w on a 1/256 grid
  verify64k L=65536, T=8, indexer q/k ~N(0,1/64), bf16 everything
  verify256k_fp8 L=262144, T=8, indexer keys and K/V in e4m3 + row scale
  verify1m  L=2^20,  T=8, ~N(0,1), ~1% planted high-score rows, e4m3 keys
  module1m  5 SWA + 1 DSA layers at L=2^20, T=8, hidden 4096
"""
from __future__ import annotations

import dataclasses
import numpy as np
import torch

# ----------------------------------------------------------------------------
# fixed shapes of one GPU's share
H_Q = 8          # query heads per GPU (one KV group)
HEAD_DIM = 128   # attention head width
H_I = 16         # indexer heads
D_I = 64         # indexer head width
TOP_K = 2048
WINDOW = 128
HIDDEN = 4096

# tensor ids: every tensor draws from its own stream
_TID = {
    "q_idx": 1, "k_idx": 2, "w_idx": 3, "q": 4, "k": 5, "v": 6,
    "plant_set": 7, "plant_dir": 8, "x": 9, "w_qkvi": 10, "w_o": 11,
    "ring_k": 12, "ring_v": 13, "sink": 14, "gamma": 15,
}


def rng_for(seed: int, name: str, layer: int = 0) -> np.random.Generator:
    """Independent PCG64 stream per (seed, tensor, layer)."""
    return np.random.default_rng([int(seed), _TID[name], int(layer)])


# ----------------------------------------------------------------------------
# storage formats (library casts only)

def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 array -> bf16 bit patterns (uint16), round-to-nearest-even via torch."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def to_e4m3_rows(x: np.ndarray):
    """fp32 [rows, cols] -> (e4m3fn codes uint8 [rows, cols], fp32 scale [rows]).

    scale = rowmax|x| / 448 (1 for an all-zero row); codes = torch cast of x/scale.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    t = torch.from_numpy(x)
    amax = t.abs().amax(dim=1)
    scale = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    codes = (t / scale[:, None]).to(torch.float8_e4m3fn).view(torch.uint8)
    return codes.numpy().copy(), scale.numpy().astype(np.float32).copy()


def normal(seed, name, shape, std=1.0, layer=0) -> np.ndarray:
    g = rng_for(seed, name, layer)
    a = g.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


# ----------------------------------------------------------------------------
@dataclasses.dataclass
class DSAInputs:
    """Inputs of the standalone indexer / top-k / sparse-attention calls."""
    name: str
    L: int
    T: int
    pos0: int
    top_k: int
    q_idx: np.ndarray        # [T][H_I][D_I] bf16 bits
    w_idx: np.ndarray        # [T][H_I] fp32
    k_idx: np.ndarray        # [L][D_I] bf16 bits or e4m3 codes
    k_idx_scale: np.ndarray | None  # [L] fp32 (e4m3 only)
    k_idx_dtype: str         # "bf16" | "fp8"
    q: np.ndarray            # [T][H_Q][HEAD_DIM] bf16 bits
    k: np.ndarray            # [L][HEAD_DIM] bf16 bits or e4m3 codes
    v: np.ndarray
    k_scale: np.ndarray | None
    v_scale: np.ndarray | None
    kv_dtype: str
    planted: np.ndarray | None = None


def dsa_config(name: str, seed: int = 0, L: int | None = None, T: int | None = None,
               tie_stress: bool = False) -> DSAInputs:
    """Build one of the standalone-kernel workloads.

    ``L``/``T`` override the context length / block size while keeping the
    distributions (used for small parity cases and ragged tails).
    """
    if name == "tiny":
        L = L or 4096
        T = T or 1
        g = rng_for(seed, "q_idx")
        if tie_stress:
            qi = g.integers(-1, 2, size=(T, H_I, D_I)).astype(np.float32)
            ki = rng_for(seed, "k_idx").integers(-1, 2, size=(L, D_I)).astype(np.float32)
            w = np.ones((T, H_I), np.float32)
        else:
            qi = g.integers(-4, 5, size=(T, H_I, D_I)).astype(np.float32)
            ki = rng_for(seed, "k_idx").integers(-4, 5, size=(L, D_I)).astype(np.float32)
            u = rng_for(seed, "w_idx").random(size=(T, H_I))
            w = (np.floor(256.0 * u) / 256.0).astype(np.float32)
        q_idx = to_bf16_bits(qi)
        k_idx, k_idx_scale, kdt = to_bf16_bits(ki), None, "bf16"
        q = to_bf16_bits(normal(seed, "q", (T, H_Q, HEAD_DIM)))
        k = to_bf16_bits(normal(seed, "k", (L, HEAD_DIM)))
        v = to_bf16_bits(normal(seed, "v", (L, HEAD_DIM)))
        return DSAInputs(name, L, T, L - T, TOP_K, q_idx, w, k_idx, k_idx_scale, kdt,
                         q, k, v, None, None, "bf16")

    if name in ("verify64k", "verify256k_fp8"):
        L = L or (65536 if name == "verify64k" else 262144)
        T = T or 8
        qi = normal(seed, "q_idx", (T, H_I, D_I), std=0.125)
        ki = normal(seed, "k_idx", (L, D_I), std=0.125)
        w = rng_for(seed, "w_idx").random(size=(T, H_I)).astype(np.float32)
        q = to_bf16_bits(normal(seed, "q", (T, H_Q, HEAD_DIM)))
        kf = normal(seed, "k", (L, HEAD_DIM))
        vf = normal(seed, "v", (L, HEAD_DIM))
        if name == "verify64k":
            return DSAInputs(name, L, T, L - T, TOP_K, to_bf16_bits(qi), w, to_bf16_bits(ki),
                             None, "bf16", q, to_bf16_bits(kf), to_bf16_bits(vf),
                             None, None, "bf16")
        k8, ks = to_e4m3_rows(ki)
        K8, Ks = to_e4m3_rows(kf)
        V8, Vs = to_e4m3_rows(vf)
        return DSAInputs(name, L, T, L - T, TOP_K, to_bf16_bits(qi), w, k8, ks, "fp8",
                         q, K8, V8, Ks, Vs, "fp8")

    if name == "verify1m":
        L = L or (1 << 20)
        T = T or 8
        qi = normal(seed, "q_idx", (T, H_I, D_I))
        ki = normal(seed, "k_idx", (L, D_I))
        # ~1% planted rows sharing one direction with every indexer query
        n_plant = max(1, L // 100)
        gp = rng_for(seed, "plant_set")
        planted = np.sort(gp.choice(max(1, L - T), size=min(n_plant, max(1, L - T)),
                                    replace=False)).astype(np.int64)
        u = rng_for(seed, "plant_dir").standard_normal(D_I)
        u = (u / np.linalg.norm(u)).astype(np.float32)
        ki[planted] += np.float32(4.0) * u
        qi += np.float32(4.0) * u
        w = rng_for(seed, "w_idx").random(size=(T, H_I)).astype(np.float32)
        k8, ks = to_e4m3_rows(ki)
        q = to_bf16_bits(normal(seed, "q", (T, H_Q, HEAD_DIM)))
        k = to_bf16_bits(normal(seed, "k", (L, HEAD_DIM)))
        v = to_bf16_bits(normal(seed, "v", (L, HEAD_DIM)))
        return DSAInputs(name, L, T, L - T, TOP_K, to_bf16_bits(qi), w, k8, ks, "fp8",
                         q, k, v, None, None, "bf16", planted=planted)

    raise KeyError(name)


# ----------------------------------------------------------------------------
# layer-step (module) inputs

N_PROJ_DSA = H_Q * HEAD_DIM + HEAD_DIM + HEAD_DIM + H_I * D_I + D_I + H_I   # 2384
N_PROJ_SWA = H_Q * HEAD_DIM + HEAD_DIM + HEAD_DIM                         # 1280


@dataclasses.dataclass
class LayerInputs:
    kind: str                 # "dsa" | "swa"
    gamma: np.ndarray         # [HIDDEN] bf16 bits
    w_qkvi: np.ndarray        # [N_proj][HIDDEN] bf16 bits (out-features major)
    w_o: np.ndarray           # [HIDDEN][H_Q*HEAD_DIM] bf16 bits
    # DSA caches (capacity rows) or SWA rings (ring_cap rows)
    k: np.ndarray
    v: np.ndarray
    k_idx: np.ndarray | None = None        # [cap][D_I] e4m3 codes
    k_idx_scale: np.ndarray | None = None  # [cap] fp32
    capacity: int = 0


def layer_inputs(kind: str, layer: int, L: int, T: int, seed: int = 0,
                 ring_cap: int = 256, w_std: float = 0.02) -> LayerInputs:
    """One layer of the module workload: RMSNorm gamma = 1, weights ~N(0, w_std).

    DSA: caches hold positions [0, L-T) prefilled ~N(0,1); rows L-T.. are
    written by the step.  SWA: the ring (``ring_cap`` slots, position p in slot
    p % ring_cap) holds positions [L-T-(WINDOW-1), L-T) prefilled ~N(0,1).
    """
    pos0 = L - T
    gamma = to_bf16_bits(np.ones(HIDDEN, np.float32))
    n_proj = N_PROJ_DSA if kind == "dsa" else N_PROJ_SWA
    w_qkvi = to_bf16_bits(normal(seed, "w_qkvi", (n_proj, HIDDEN), std=w_std, layer=layer))
    w_o = to_bf16_bits(normal(seed, "w_o", (HIDDEN, H_Q * HEAD_DIM), std=w_std, layer=layer))
    if kind == "dsa":
        k = to_bf16_bits(normal(seed, "k", (L, HEAD_DIM), layer=layer))
        v = to_bf16_bits(normal(seed, "v", (L, HEAD_DIM), layer=layer))
        ki = normal(seed, "k_idx", (L, D_I), layer=layer)
        k8, ks = to_e4m3_rows(ki)
        # rows the step will write are left as they were drawn; the step overwrites them
        return LayerInputs("dsa", gamma, w_qkvi, w_o, k, v, k8, ks, capacity=L)
    rk = np.zeros((ring_cap, HEAD_DIM), np.float32)
    rv = np.zeros((ring_cap, HEAD_DIM), np.float32)
    lo = max(0, pos0 - (WINDOW - 1))
    pk = normal(seed, "ring_k", (pos0 - lo, HEAD_DIM), layer=layer)
    pv = normal(seed, "ring_v", (pos0 - lo, HEAD_DIM), layer=layer)
    for i, p in enumerate(range(lo, pos0)):
        rk[p % ring_cap] = pk[i]
        rv[p % ring_cap] = pv[i]
    return LayerInputs("swa", gamma, w_qkvi, w_o, to_bf16_bits(rk), to_bf16_bits(rv),
                       capacity=ring_cap)


def w8a8_weights(lay: LayerInputs):
    """The layer's bf16 weights stored as W8A8 weights: e4m3 codes with one fp32 scale
    per output row (rowmax / 448, the same storage cast as the prefilled caches).
    Returns (w_qkvi codes, w_qkvi scales, w_o codes, w_o scales)."""
    def rows(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    wq, sq = to_e4m3_rows(rows(lay.w_qkvi))
    wo, so = to_e4m3_rows(rows(lay.w_o))
    return wq, sq, wo, so


# groups of 16 integers whose squares sum to 16 (zeros padded), for exact_norm_x
_NORM_GROUPS = ((1,) * 16, (2, 2, 2, 2), (4,), (3, 2, 1, 1, 1), (2, 2, 2, 1, 1, 1, 1))


def exact_norm_x(seed: int, T: int, groups=None, scale_exp=(-2, -1, 0, 1, 2)) -> np.ndarray:
    """Residual rows [T][HIDDEN] bf16 bits whose mean square is an exact power of 4:
    each row is 256 blocks of 16 drawn from small-integer groups with squares summing
    to 16 (random order and signs), times a per-row power of two.  Every row holds at
    least one block with the row's largest magnitude (4).  With eps = 0 the RMS factor
    is an exact power of two, so normalised values are identical in any precision."""
    groups = _NORM_GROUPS if groups is None else groups
    g = rng_for(seed, "x")
    out = np.zeros((T, HIDDEN), np.float32)
    for t in range(T):
        row = []
        picks = g.integers(0, len(groups), size=HIDDEN // 16)
        picks[g.integers(0, HIDDEN // 16)] = [i for i, gr in enumerate(groups) if gr[0] == 4][0]
        for pk in picks:
            blk = np.zeros(16, np.float32)
            vals = np.array(groups[pk], np.float32)
            blk[: len(vals)] = vals * np.where(g.integers(0, 2, size=len(vals)) == 1, -1.0, 1.0)
            row.append(blk[g.permutation(16)])
        out[t] = np.concatenate(row) * np.float32(2.0 ** int(g.choice(scale_exp)))
    return to_bf16_bits(out)


def random_gamma(seed: int, std: float = 0.25) -> np.ndarray:
    """RMSNorm gain [HIDDEN] bf16 bits ~N(1, std) (the module itself uses gamma = 1)."""
    return to_bf16_bits(1.0 + normal(seed, "gamma", (HIDDEN,), std=std))


def module_x(seed: int, T: int) -> np.ndarray:
    """Residual-stream input [T][HIDDEN] bf16 bits ~N(0,1)."""
    return to_bf16_bits(normal(seed, "x", (T, HIDDEN)))


MODULE_KINDS = ("swa", "swa", "swa", "swa", "swa", "dsa")


def sink_logits(seed: int, std: float = 1.0) -> np.ndarray:
    """Per-head sink logits [H_Q] fp32 (used only where a test asks for a sink)."""
    return normal(seed, "sink", (H_Q,), std=std)
