"""The allocation-free attention entry point (dsa_sparse_attn_static) through the C ABI:
its output equals dsa_sparse_attn's on the same inputs bit for bit (same kernels), on two
calls in a row, the second with a smaller input; and it matches the oracle."""
import math

import numpy as np
import pytest
import torch

import synth
from oracle import dsa_oracle as O
from tests.gpu_util import DEV, up, down, bf16_bits

pytestmark = pytest.mark.gpu
SM = 1.0 / math.sqrt(128)


def _case(dsa, inp, k, T, out_dtype, sink=None):
    g = np.random.default_rng(inp.L + T)
    idx = np.full((T, k), -1, np.int32)
    for t in range(T):
        vis = inp.pos0 + t + 1
        n = min(k, vis)
        idx[t, :n] = np.sort(g.choice(vis, n, replace=False))
    fp8 = inp.kv_dtype == "fp8"
    args = [up(inp.q[:T]), up(inp.k), up(inp.v), up(inp.k_scale) if fp8 else None,
            up(inp.v_scale) if fp8 else None, dsa.FP8_E4M3 if fp8 else dsa.BF16, up(idx), k, T, inp.L, SM,
            None if sink is None else up(sink)]
    dt = torch.float32 if out_dtype == dsa.FP32 else torch.bfloat16
    a = torch.full((T, 8, 128), float("nan"), dtype=dt, device=DEV)
    b = torch.full((T, 8, 128), float("nan"), dtype=dt, device=DEV)
    dsa.dsa_sparse_attn_static(*args, b, out_dtype)
    ws = dsa.workspace(dsa.WS_SPARSE_ATTN, T, inp.L, k)
    dsa.dsa_sparse_attn(*args, a, out_dtype, ws)
    torch.cuda.synchronize()
    return idx, a, b


def test_static_entry_point_equals_workspace_entry_point(lib):
    dsa = lib
    inp = synth.dsa_config("verify64k", seed=3, L=9000, T=8)
    # first call: the largest shape (T = 8, k = 2048, 32 splits), fp32 output with sinks
    sink = synth.sink_logits(3)
    idx, a, b = _case(dsa, inp, 2048, 8, dsa.FP32, sink)
    assert torch.equal(a, b)
    K, V = O.decode_bf16(inp.k), O.decode_bf16(inp.v)
    ref = O.sparse_attention(O.decode_bf16(inp.q), K, V, idx, SM, sink)
    got = down(b).astype(np.float64)
    for t in range(8):
        for h in range(8):
            assert np.max(np.abs(got[t, h] - ref[t, h])) <= 1e-5 * np.max(np.abs(ref[t, h]))
    # second call in a row, smaller: T = 3, k = 300 (5 splits), e4m3 cache, bf16 output
    inp2 = synth.dsa_config("verify256k_fp8", seed=4, L=5000, T=3)
    idx2, a2, b2 = _case(dsa, inp2, 300, 3, dsa.BF16)
    assert np.array_equal(bf16_bits(a2), bf16_bits(b2))
    K2, V2 = O.dequant_rows(inp2.k, "fp8", inp2.k_scale), O.dequant_rows(inp2.v, "fp8", inp2.v_scale)
    ref2 = O.sparse_attention(O.decode_bf16(inp2.q), K2, V2, idx2, SM)
    assert np.max(np.abs(O.decode_bf16(bf16_bits(b2)) - ref2)) <= 2e-2
