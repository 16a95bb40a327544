"""Helpers for the GPU parity tests: uploads of synthetic inputs and comparison rules."""
import numpy as np
import torch

DEV = "cuda:0"


def up(a, dtype=None):
    """numpy -> device tensor (bf16 bit patterns travel as int16, e4m3 codes as uint8)."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    t = torch.from_numpy(a).to(DEV)
    return t if dtype is None else t.to(dtype)


def down(t):
    return t.detach().cpu().numpy()


def bf16_bits(t):
    """device int16/bfloat16 tensor -> numpy uint16 bit patterns"""
    if t.dtype == torch.bfloat16:
        t = t.view(torch.int16)
    return down(t).view(np.uint16)


def tie_band_ok(idx_gpu, idx_ref, scores_ref, mag_ref, pos0, k, rel=2.0 ** -16):
    """Index sets may differ only in positions whose exact score is within the
    rounding band of the k-th score.  Returns (ok, number of differing positions)."""
    T = idx_gpu.shape[0]
    ndiff = 0
    for t in range(T):
        g = set(int(x) for x in idx_gpu[t] if x >= 0)
        r = set(int(x) for x in idx_ref[t] if x >= 0)
        if len(g) != len(r):
            return False, -1
        sym = g ^ r
        if not sym:
            continue
        ndiff += len(sym)
        vis = pos0 + t + 1
        s = scores_ref[t, :vis]
        order = np.lexsort((np.arange(vis), -s))
        kk = min(k, vis)
        s_theta = order[kk - 1]
        theta = s[s_theta]
        for p in sym:
            band = rel * max(mag_ref[t, p], mag_ref[t, s_theta])
            if abs(s[p] - theta) > band:
                return False, ndiff
    return True, ndiff


def check_oproj(gx, tf_x, attn, wo_deq, x, allowance=0.0):
    """x_out = bf16(x + attn . W_o^T) against the oracle's fp64 value on the same attention
    output: one bf16 ulp of the result, the fp32 accumulation bound 2^-16 * sum |terms|
    (1024 products and the residual), and any code-flip allowance."""
    from oracle import dsa_oracle as O
    S = O.project(np.abs(attn), np.abs(wo_deq)) + np.abs(x)
    tol = 2.0 ** -7 * np.abs(tf_x) + 2.0 ** -16 * S + allowance
    bad = np.abs(gx - tf_x) > tol
    assert not bad.any(), f"{bad.sum()} output values beyond tolerance, worst {np.max(np.abs(gx - tf_x) - tol)}"
