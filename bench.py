#!/usr/bin/env python3
"""Benchmark of the DSA decode/verify hot path on one MI355X.

One step = one pass of a Naive-N0.5-Flash module's attention path for an 8-token
verify block at 1M context: five sliding-window layers and one DSA layer, each a
dsa_layer_step call (RMSNorm -> fused projection -> RoPE -> cache append -> [indexer ->
top-2048 ->] attention -> output projection + residual).  Inputs are seeded synthetic
tensors of the workload's shapes (weights ~N(0, 0.02), caches ~N(0,1), indexer keys
e4m3 with a per-row scale); they are resident in HBM before timing starts.  To keep
the 256 MB last-level cache from serving repeated reads, consecutive steps rotate
over --rotate independent copies of every weight and cache.

Printed: one JSON line with the step throughput in algorithmic HBM bytes per second,
the DSA layer-step time, the roofline of the dominant kernel (the fused indexer scan +
top-k), and the oracle's CPU time on one module step.
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
MODULE = ("swa", "swa", "swa", "swa", "swa", "dsa")
RING_CAP = 256


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--rotate", type=int, default=8,
                    help="independent input copies cycled over steps (8 x the 68 MB key scan > 2 x the "
                         "256 MB last-level cache)")
    ap.add_argument("--L", type=int, default=1 << 20)
    ap.add_argument("--T", type=int, default=8)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--no-w8a8", action="store_true", help="skip the W8A8 module timing")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the standalone timings (and oracle stage times) of the smaller configs")
    ap.add_argument("--eager", action="store_true",
                    help="skip the HIP-graph replay timing (reported beside the direct-launch step)")
    ap.add_argument("--only", choices=["module", "index_topk", "sparse_attn", "copy"], default="module",
                    help="index_topk / sparse_attn / copy: run only that call (for counter passes)")
    return ap.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the decode step runs on exactly one GPU; --gpus must be 1 "
                                   "(no multi-GPU sharding is implemented)"}))
        sys.exit(2)
    import numpy as np
    import torch
    import sparse_attention_decode_indexer_amd as dsa
    import synth

    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    L, T, K = args.L, args.T, 2048
    pos0 = L - T
    R = max(1, args.rotate)

    def up(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            a = a.view(np.int16)
        return torch.from_numpy(a).to(dev)

    # ------------------------------------------------------------------ inputs (set 0 on host)
    t0 = time.time()
    host_layers = [synth.layer_inputs(kind, i, L, T, seed=args.seed, ring_cap=RING_CAP)
                   for i, kind in enumerate(MODULE)]
    x_host = synth.module_x(args.seed, T)
    log(f"[bench] host inputs generated in {time.time() - t0:.1f}s")

    def device_set(r):
        """Set r: rows of every tensor rolled by a set-specific offset (new memory, same law)."""
        sets = []
        for lay in host_layers:
            d = {}
            for name in ("gamma", "w_qkvi", "w_o", "k", "v", "k_idx", "k_idx_scale"):
                a = getattr(lay, name)
                if a is None:
                    d[name] = None
                    continue
                t = up(a)
                if r and name != "gamma" and not (lay.kind == "swa" and name in ("k", "v")):
                    t = torch.roll(t, shifts=r * 7919, dims=0).contiguous()
                d[name] = t
            d["kind"] = lay.kind
            d["capacity"] = lay.capacity
            sets.append(d)
        return sets

    dev_sets = [device_set(r) for r in range(R if args.only == "module" else 1)]
    x0 = up(x_host)
    xs = [torch.zeros_like(x0) for _ in range(len(MODULE))]
    qkv = torch.zeros((T, synth.N_PROJ_DSA), dtype=torch.int16, device=dev)
    idx = torch.full((T, K), -1, dtype=torch.int32, device=dev)
    ws_dsa = dsa.workspace(dsa.WS_LAYER_DSA, T, L, K)
    ws_swa = dsa.workspace(dsa.WS_LAYER_SWA, T, L, 128)
    cfg_dsa = dsa.layer_config(dsa.LAYER_DSA, top_k=K)
    cfg_swa = dsa.layer_config(dsa.LAYER_SWA, window=128)
    structs = []
    for s in dev_sets:
        per = []
        for d in s:
            w = dsa.LayerWeights(d["gamma"].data_ptr(), d["w_qkvi"].data_ptr(), d["w_o"].data_ptr())
            c = dsa.LayerCache(d["k"].data_ptr(), d["v"].data_ptr(),
                               d["k_idx"].data_ptr() if d["k_idx"] is not None else None,
                               d["k_idx_scale"].data_ptr() if d["k_idx_scale"] is not None else None,
                               d["capacity"])
            per.append((d["kind"], w, c))
        structs.append(per)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    ev_dsa = []

    def step(i, record=False, st=None):
        st = stream if st is None else st
        per = structs[i % len(structs)]
        xin = x0
        for li, (kind, w, c) in enumerate(per):
            if kind == "dsa":
                if record:
                    e0 = torch.cuda.Event(enable_timing=True)
                    e1 = torch.cuda.Event(enable_timing=True)
                    e0.record(st)
                dsa.dsa_layer_step(cfg_dsa, w, c, xin, xs[li], T, pos0, idx_out=idx, qkv_out=qkv, ws=ws_dsa,
                                   stream=st)
                if record:
                    e1.record(st)
                    ev_dsa.append((e0, e1))
            else:
                dsa.dsa_layer_step(cfg_swa, w, c, xin, xs[li], T, pos0, ws=ws_swa, stream=st)
            xin = xs[li]

    # ------------------------------------------------------------------ dominant-kernel inputs
    def index_topk_inputs():
        # the DSA layer's own rotated indexer queries and head weights (from qkv_out)
        step(0)
        torch.cuda.synchronize()
        q = qkv[:, 1280:2304].contiguous()
        wv = qkv[:, 2368:2384].contiguous().view(torch.bfloat16).float().contiguous()
        return q, wv

    out = {}
    if args.only == "copy":
        # plain copy of known size, for scaling the HBM counters
        n = 256 << 20
        a = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        b = torch.empty_like(a)
        for _ in range(args.steps):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n, "launches": args.steps}))
        return

    q_i, w_i = index_topk_inputs()
    d_dsa = dev_sets[0][-1]
    ws_sel = dsa.workspace(dsa.WS_INDEX_TOPK, T, L, K)
    idx2 = torch.full((T, K), -1, dtype=torch.int32, device=dev)

    def index_topk(d):
        dsa.dsa_index_topk(q_i, w_i, d["k_idx"], d["k_idx_scale"], dsa.FP8_E4M3, T, L, pos0, K, idx2, None,
                           ws_sel, stream=stream)

    if args.only == "index_topk":
        for _ in range(args.warmup):
            index_topk(d_dsa)
        for _ in range(args.steps):
            index_topk(d_dsa)
        torch.cuda.synchronize()
        print(json.dumps({"index_topk_launches": args.steps}))
        return
    if args.only == "sparse_attn":
        # the DSA layer's own selection (idx) and rotated queries over its cache
        ws_a = dsa.workspace(dsa.WS_SPARSE_ATTN, T, L, K)
        q_a = qkv[:, 0:1024].contiguous()
        o_a = torch.zeros((T, 1024), dtype=torch.int16, device=dev)
        for i in range(args.warmup + args.steps):
            dsa.dsa_sparse_attn(q_a, d_dsa["k"], d_dsa["v"], None, None, dsa.BF16, idx, K, T, L, 1.0 / math.sqrt(128),
                                None, o_a, dsa.BF16, ws_a, stream=stream)
        torch.cuda.synchronize()
        idx_np = idx.cpu().numpy()
        union = int(np.unique(idx_np[idx_np >= 0]).size)
        print(json.dumps({"sparse_attn_launches": args.steps, "union_rows": union,
                          "gather_bytes": union * 2 * 128 * 2}))
        return

    # ------------------------------------------------------------------ timed module steps
    # Direct launches: the step time (value) and the DSA layer-step time (events around
    # its call).
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    e_start = torch.cuda.Event(enable_timing=True)
    e_end = torch.cuda.Event(enable_timing=True)
    t_host = time.perf_counter()
    e_start.record(stream)
    for i in range(args.steps):
        step(args.warmup + i, record=True)
    e_end.record(stream)
    torch.cuda.synchronize()
    t_host = time.perf_counter() - t_host
    ms_eager = e_start.elapsed_time(e_end) / args.steps
    dsa_us = [a.elapsed_time(b) * 1e3 for a, b in ev_dsa]
    log(f"[bench] {args.steps} module steps, direct launches: {ms_eager * 1e3:.1f} us/step "
        f"(host {t_host / args.steps * 1e6:.1f} us)")
    # The module entry point (dsa_module_step): one call per step, the same launches
    # enqueued back to back -- the headline step time.  For reference the same call with
    # DSA_MODULE_CHAIN=1 (the five SWA layers as one persistent launch).
    ws_mod = dsa.workspace(dsa.WS_MODULE, T, L, K)
    mod_args = []
    for per in structs:
        mod_args.append(([cfg_dsa if kind == "dsa" else cfg_swa for kind, _, _ in per],
                         [w for _, w, _ in per], [c for _, _, c in per]))

    def module_step(i, st=None):
        cfgs, ws_l, cs = mod_args[i % len(mod_args)]
        dsa.dsa_module_step(cfgs, ws_l, cs, x0, xs[-1], T, pos0, idx_out=idx, ws=ws_mod,
                            stream=stream if st is None else st)

    def time_module():
        for i in range(args.warmup):
            module_step(i)
        torch.cuda.synchronize()
        e_start.record(stream)
        for i in range(args.steps):
            module_step(args.warmup + i)
        e_end.record(stream)
        torch.cuda.synchronize()
        return e_start.elapsed_time(e_end) / args.steps

    ms_module = time_module()
    os.environ["DSA_MODULE_CHAIN"] = "1"
    ms_module_chain = time_module()
    del os.environ["DSA_MODULE_CHAIN"]
    log(f"[bench] {args.steps} module steps through dsa_module_step: {ms_module * 1e3:.1f} us/step "
        f"(SWA layers as one persistent launch: {ms_module_chain * 1e3:.1f} us/step)")
    ms_step = ms_module
    ms_graph = None
    if not args.eager:
        # For reference: one HIP graph per input set holding a whole module step (one
        # dsa_module_step call captured: 15 kernels), replayed as a serving loop would, one
        # host launch per step.
        graphs = []
        cap = torch.cuda.Stream()
        cap.wait_stream(stream)
        for r in range(len(structs)):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cap):
                module_step(r, st=torch.cuda.current_stream())
            graphs.append(g)
        stream.wait_stream(cap)
        torch.cuda.synchronize()
        for i in range(args.warmup):
            graphs[i % len(graphs)].replay()
        torch.cuda.synchronize()
        e_start.record(stream)
        for i in range(args.steps):
            graphs[(args.warmup + i) % len(graphs)].replay()
        e_end.record(stream)
        torch.cuda.synchronize()
        ms_graph = e_start.elapsed_time(e_end) / args.steps
        log(f"[bench] {args.steps} module steps, graph replay: {ms_graph * 1e3:.1f} us/step")

    # ------------------------------------------------------------------ dominant kernel, live events
    # launches back to back between one pair of events on the launch stream, cycling over
    # the input sets: the average is the kernel's duration plus the inter-kernel gap
    n_sel = max(args.steps, 10)
    for i in range(3):
        index_topk(dev_sets[i % len(dev_sets)][-1])
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(n_sel):
        index_topk(dev_sets[i % len(dev_sets)][-1])
    e1.record(stream)
    torch.cuda.synchronize()
    sel_us = [e0.elapsed_time(e1) * 1e3 / n_sel]
    assert np.array_equal(idx2.cpu().numpy().shape, (T, K))

    # ------------------------------------------------------------------ per-call distributions
    # One event pair per call, calls queued back to back.  "cold": consecutive calls cycle over
    # the rotated input sets; "warm": every call reads set 0, so the last-level cache can serve
    # repeats (labelled, never the headline).
    ws_att = dsa.workspace(dsa.WS_SPARSE_ATTN, T, L, K)
    q_att = qkv[:, 0:1024].contiguous()
    o_att = torch.zeros((T, 1024), dtype=torch.int16, device=dev)
    idx_att = idx.clone()
    sm = 1.0 / math.sqrt(128)

    def sparse_attn(d):
        dsa.dsa_sparse_attn(q_att, d["k"], d["v"], None, None, dsa.BF16, idx_att, K, T, L, sm, None,
                            o_att, dsa.BF16, ws_att, stream=stream)

    def dsa_layer(per):
        kind, w, c = per[-1]
        dsa.dsa_layer_step(cfg_dsa, w, c, xs[-2], xs[-1], T, pos0, idx_out=idx, qkv_out=qkv, ws=ws_dsa,
                           stream=stream)

    def per_call(fn, sets, n):
        for i in range(args.warmup):
            fn(sets[i % len(sets)])
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for i, (a, b) in enumerate(evs):
            a.record(stream)
            fn(sets[i % len(sets)])
            b.record(stream)
        torch.cuda.synchronize()
        return [a.elapsed_time(b) * 1e3 for a, b in evs]

    n_pc = max(args.steps, 10)
    dsa_sets = [s[-1] for s in dev_sets]
    dist = {
        "dsa_layer_step_us": {"cold": stats(dsa_us), "warm": stats(per_call(dsa_layer, structs[:1], n_pc))},
        "index_topk_us": {"cold": stats(per_call(index_topk, dsa_sets, n_pc)),
                          "warm": stats(per_call(index_topk, dsa_sets[:1], n_pc))},
        "sparse_attn_us": {"cold": stats(per_call(sparse_attn, dsa_sets, n_pc)),
                           "warm": stats(per_call(sparse_attn, dsa_sets[:1], n_pc))},
    }
    log(f"[bench] per-call medians (cold/warm, us): " + ", ".join(
        f"{k} {v['cold']['median']}/{v['warm']['median']}" for k, v in dist.items()))
    ceiling = read_ceiling(torch, dev, stream, dsa)
    log(f"[bench] read ceiling: {ceiling}")
    configs = None
    if not args.no_configs:
        configs = config_timings(args, dsa, torch, np, synth, dev, stream)

    # ------------------------------------------------------------------ W8A8 module
    # The same module with every projection weight stored as e4m3 codes + per-row fp32
    # scales and the activations quantised per token on chip; caches and inputs are the
    # bf16 run's (same rotated sets).
    w8a8 = None
    if not args.no_w8a8:
        w8_host = [synth.w8a8_weights(lay) for lay in host_layers]
        w8_sets = []
        for r in range(len(dev_sets)):
            per = []
            for li, (wq, sq, wo, so) in enumerate(w8_host):
                arrs = [up(a) for a in (wq, sq, wo, so)]
                if r:
                    arrs = [torch.roll(a, shifts=r * 7919, dims=0).contiguous() for a in arrs]
                per.append(arrs)
            w8_sets.append(per)
        structs8 = []
        for r, per in enumerate(structs):
            row = []
            for li, (kind, w, c) in enumerate(per):
                wq, sq, wo, so = w8_sets[r][li]
                w8 = dsa.LayerWeights(w.rms_gamma, wq.data_ptr(), wo.data_ptr(), dsa.FP8_E4M3, sq.data_ptr(),
                                      so.data_ptr())
                row.append((kind, w8, c))
            structs8.append(row)

        def step8(i):
            per = structs8[i % len(structs8)]
            xin = x0
            for li, (kind, w, c) in enumerate(per):
                if kind == "dsa":
                    dsa.dsa_layer_step(cfg_dsa, w, c, xin, xs[li], T, pos0, idx_out=idx, qkv_out=qkv, ws=ws_dsa,
                                       stream=stream)
                else:
                    dsa.dsa_layer_step(cfg_swa, w, c, xin, xs[li], T, pos0, ws=ws_swa, stream=stream)
                xin = xs[li]

        for i in range(args.warmup):
            step8(i)
        torch.cuda.synchronize()
        e_start.record(stream)
        for i in range(args.steps):
            step8(args.warmup + i)
        e_end.record(stream)
        torch.cuda.synchronize()
        ms8 = e_start.elapsed_time(e_end) / args.steps

        def dsa_layer8(per):
            kind, w, c = per[-1]
            dsa.dsa_layer_step(cfg_dsa, w, c, xs[-2], xs[-1], T, pos0, idx_out=idx, qkv_out=qkv, ws=ws_dsa,
                               stream=stream)
        dsa8 = {"cold": stats(per_call(dsa_layer8, structs8, n_pc)),
                "warm": stats(per_call(dsa_layer8, structs8[:1], n_pc))}
        log(f"[bench] W8A8 module: {ms8 * 1e3:.1f} us/step; DSA layer cold median {dsa8['cold']['median']} us")
        w8a8 = {"ms_per_step": round(ms8, 5), "tokens_per_s_module": round(T / (ms8 * 1e-3), 1),
                "dsa_layer_step_us": dsa8}
        del w8_sets

    # ------------------------------------------------------------------ algorithmic bytes
    idx_np = idx.cpu().numpy()
    union = np.unique(idx_np[idx_np >= 0]).size
    hidden = 4096
    scan = L * (64 + 4)                                   # e4m3 indexer keys + fp32 row scales
    gather = union * 2 * 128 * 2                          # bf16 K and V rows, union over tokens
    w_dsa = synth.N_PROJ_DSA * hidden * 2 + hidden * 1024 * 2 + hidden * 2
    w_swa = synth.N_PROJ_SWA * hidden * 2 + hidden * 1024 * 2 + hidden * 2
    act = 2 * T * hidden * 2                              # x in + x out
    append_dsa = T * (2 * 128 * 2 + 64 + 4)
    append_swa = T * 2 * 128 * 2
    ring = min(128 + T - 1, RING_CAP) * 2 * 128 * 2
    bytes_dsa = scan + gather + w_dsa + act + append_dsa + T * K * 4
    bytes_swa = w_swa + act + append_swa + ring
    bytes_step = bytes_dsa + 5 * bytes_swa
    if w8a8 is not None:
        # e4m3 weights + one fp32 scale per weight row
        w8_dsa = synth.N_PROJ_DSA * (hidden + 4) + hidden * (1024 + 4) + hidden * 2
        w8_swa = synth.N_PROJ_SWA * (hidden + 4) + hidden * (1024 + 4) + hidden * 2
        b8_dsa = bytes_dsa - w_dsa + w8_dsa
        b8_step = b8_dsa + 5 * (bytes_swa - w_swa + w8_swa)
        med8 = w8a8["dsa_layer_step_us"]["cold"]["median"]
        w8a8.update({"algorithmic_bytes_per_step": int(b8_step),
                     "GBps": round(b8_step / (w8a8["ms_per_step"] * 1e-3) / 1e9, 1),
                     "dsa_layer_step_GBps": round(b8_dsa / (med8 * 1e-6) / 1e9, 1),
                     "dsa_layer_step_frac": round(b8_dsa / (med8 * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)})
    sel_bytes = scan + T * K * 4
    sel_avg = float(np.mean(sel_us))
    achieved = sel_bytes / (sel_avg * 1e-6) / 1e9
    value = bytes_step / (ms_step * 1e-3) / 1e9
    dsa_avg = float(np.mean(dsa_us))
    # scan + gather: the key scan and the union of gathered K/V rows over the time of the two
    # calls that move them (per-call cold medians)
    sg_us = dist["index_topk_us"]["cold"]["median"] + dist["sparse_attn_us"]["cold"]["median"]
    sg_gbps = (scan + gather) / (sg_us * 1e-6) / 1e9
    scan_gather = {"bytes": int(scan + gather), "us": round(sg_us, 2), "GBps": round(sg_gbps, 1),
                   "frac_of_peak": round(sg_gbps / HBM_PEAK_GBPS, 4),
                   "frac_of_read_ceiling": round(sg_gbps / ceiling["GBps_1GiB"], 4)}

    # ------------------------------------------------------------------ oracle CPU baseline
    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(host_layers, x_host, L, T, bytes_step, with_configs=not args.no_configs)

    out = {
        "metric": "DSA layer-step µs + HBM GB/s (% roofline) at 1M ctx, 8-token verify, 1 GPU",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "ms_per_step_layer_calls": round(ms_eager, 5),
        "ms_per_step_persistent_swa": round(ms_module_chain, 5),
        "ms_per_step_graph": None if ms_graph is None else round(ms_graph, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "module1m: 5 SWA (w=128) + 1 DSA (top-2048) layer steps, L=1048576, T=8 verify block, "
                        "hidden 4096, 8 q heads / 1 KV head x 128, indexer 16x64 e4m3 keys",
            "context": L, "verify_tokens": T, "top_k": K, "rotate_sets": len(dev_sets),
            "algorithmic_bytes_per_step": int(bytes_step),
        },
        "dsa_layer_step_us": round(dsa_avg, 2),
        "dsa_layer_step_GBps": round(bytes_dsa / (dsa_avg * 1e-6) / 1e9, 1),
        "dsa_layer_step_frac": round(bytes_dsa / (dsa_avg * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
        "tokens_per_s_module": round(T / (ms_step * 1e-3), 1),
        "roofline": {
            "kernel": "select_kernel (fused indexer scan + top-k, dsa_index_topk)",
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": measured_traffic(L, T),
            "avg_us": round(sel_avg, 2),
            "algorithmic_bytes": int(sel_bytes),
        },
        "cpu_baseline": cpu,
        "w8a8": w8a8,
        "configs": configs,
        "protocol": {"per_call_calls": n_pc, "warmup_calls": args.warmup, **dist,
                     "read_ceiling": ceiling, "scan_gather": scan_gather,
                     "module_step_GBps": round(value, 1)},
    }
    print(json.dumps(out))


CONFIGS = (
    # (synth workload, label): the smaller configs of the workload list at their stated sizes
    ("tiny", "config0: L=4096, T=1, integer-valued bf16 indexer keys, bf16 K/V"),
    ("verify64k", "config1: L=65536, T=8, bf16 indexer keys ~N(0,1/64), bf16 K/V"),
    ("verify256k_fp8", "config2: L=262144, T=8, e4m3 indexer keys and e4m3 K/V with row scales"),
    ("verify1m", "config3: L=1048576, T=8, e4m3 indexer keys with 1% planted rows, bf16 K/V"),
)
# Beyond the workload list (timed on the GPU only): the config3 recipe at twice its
# context, where each workgroup's chunk exceeds the 4096 keys whose scores stay on chip
# (8192 keys per CU on 256 CUs) and the rest of the scores go through the workspace.
EXTRA_CONFIGS = (
    ("context2m", "verify1m", 1 << 21,
     "L=2097152, T=8, config3's recipe at twice the context (scores past 4096 keys per CU kept in the workspace)"),
)


def config_timings(args, dsa, torch, np, synth, dev, stream):
    """Standalone DSA path per config (fused index + top-k, then sparse attention): per-call
    p10 / median / p90 in us, cold (consecutive calls cycle over rotated input copies whose
    total exceeds the last-level cache) and warm (one copy), tokens/s = T / median step, and
    the algorithmic bytes (key scan + union of gathered K/V rows) over the cold median."""
    import math
    out = {}
    sm = 1.0 / math.sqrt(128)
    runs = [(name, name, None, label) for name, label in CONFIGS] + list(EXTRA_CONFIGS)
    for name, recipe, Lx, label in runs:
        inp = synth.dsa_config(recipe, seed=args.seed, L=Lx)
        T, Lc, K = inp.T, inp.L, inp.top_k
        fp8k = inp.k_idx_dtype == "fp8"
        fp8v = inp.kv_dtype == "fp8"
        key_row = 64 + 4 if fp8k else 128
        kv_row = (128 + 4) * 2 if fp8v else 256 * 2
        set_bytes = Lc * (key_row + kv_row)
        R = int(max(1, min(8, math.ceil(600e6 / set_bytes))))

        def up(a):
            a = np.ascontiguousarray(a)
            if a.dtype == np.uint16:
                a = a.view(np.int16)
            return torch.from_numpy(a).to(dev)
        base = {n: (None if getattr(inp, n) is None else up(getattr(inp, n)))
                for n in ("q_idx", "w_idx", "k_idx", "k_idx_scale", "q", "k", "v", "k_scale", "v_scale")}
        sets = [base]
        for r in range(1, R):
            sets.append({n: (t if t is None or n in ("q_idx", "w_idx", "q") else
                             torch.roll(t, shifts=r * 7919, dims=0).contiguous()) for n, t in base.items()})
        idx = torch.full((T, K), -1, dtype=torch.int32, device=dev)
        o = torch.zeros((T, 1024), dtype=torch.int16, device=dev)
        ws_s = dsa.workspace(dsa.WS_INDEX_TOPK, T, Lc, K)
        ws_a = dsa.workspace(dsa.WS_SPARSE_ATTN, T, Lc, K)

        def select(d):
            dsa.dsa_index_topk(d["q_idx"], d["w_idx"], d["k_idx"], d["k_idx_scale"],
                               dsa.FP8_E4M3 if fp8k else dsa.BF16, T, Lc, inp.pos0, K, idx, None, ws_s, stream=stream)

        def attend(d):
            dsa.dsa_sparse_attn(d["q"], d["k"], d["v"], d["k_scale"], d["v_scale"], dsa.FP8_E4M3 if fp8v else dsa.BF16,
                                idx, K, T, Lc, sm, None, o, dsa.BF16, ws_a, stream=stream)

        def both(d):
            select(d)
            attend(d)

        def per_call(fn, ss, n):
            for i in range(max(3, args.warmup)):
                fn(ss[i % len(ss)])
            evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
            for i, (a, b) in enumerate(evs):
                a.record(stream)
                fn(ss[i % len(ss)])
                b.record(stream)
            torch.cuda.synchronize()
            return [a.elapsed_time(b) * 1e3 for a, b in evs]
        n = max(args.steps, 10)
        res = {"label": label, "L": Lc, "T": T, "rotate_sets": R,
               "step_us": {"cold": stats(per_call(both, sets, n)), "warm": stats(per_call(both, sets[:1], n))},
               "index_topk_us": {"cold": stats(per_call(select, sets, n))},
               "sparse_attn_us": {"cold": stats(per_call(attend, sets, n))}}
        select(sets[0])
        torch.cuda.synchronize()
        ii = idx.cpu().numpy()
        union = int(np.unique(ii[ii >= 0]).size)
        alg = Lc * key_row + union * kv_row
        med = res["step_us"]["cold"]["median"]
        res.update({"tokens_per_s": round(T / (med * 1e-6), 1), "algorithmic_bytes": int(alg),
                    "GBps": round(alg / (med * 1e-6) / 1e9, 1),
                    "frac_of_peak": round(alg / (med * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)})
        log(f"[bench] {name}: step cold median {med} us, {res['tokens_per_s']} tok/s, {res['GBps']} GB/s")
        out[name] = res
        del sets, base
        torch.cuda.synchronize()
    return out


def stats(v):
    """p10 / median / p90 of per-call times in us."""
    import numpy as np
    a = np.asarray(v, dtype=np.float64)
    return {"p10": round(float(np.percentile(a, 10)), 2), "median": round(float(np.median(a)), 2),
            "p90": round(float(np.percentile(a, 90)), 2), "n": int(a.size)}


def read_ceiling(torch, dev, stream, dsa):
    """Measured HBM read ceiling: the streaming-read helper of libdsa_read_ceiling.so (a
    plain streaming read, one workgroup per CU, 64 KiB in flight per CU; not part of the
    library) over 1 GiB, and over 64 MiB per call rotated across 8 buffers (the key scan's
    size, cold in the 256 MB last-level cache); median of 20 calls, one event pair per call."""
    import ctypes as C
    lib = C.CDLL(os.path.join(os.path.dirname(dsa.LIB_PATH), "libdsa_read_ceiling.so"))
    fn = lib.dsa_read_ceiling_stream
    fn.argtypes = [C.c_void_p, C.c_size_t, C.c_void_p, C.c_void_p]
    fn.restype = C.c_int
    sink = torch.zeros(1024, dtype=torch.int32, device=dev)

    def call(b, nb):
        rc = fn(b.data_ptr(), nb, sink.data_ptr(), stream.cuda_stream)
        if rc != 0:
            raise RuntimeError(f"dsa_read_ceiling_stream failed ({rc})")

    def run(bufs, n=20):
        nb = bufs[0].numel()
        for b in bufs[:2]:
            call(b, nb)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for i, (a, e) in enumerate(evs):
            a.record(stream)
            call(bufs[i % len(bufs)], nb)
            e.record(stream)
        torch.cuda.synchronize()
        t = sorted(a.elapsed_time(e) * 1e-3 for a, e in evs)
        return nb / t[len(t) // 2] / 1e9
    big = [torch.ones(1 << 30, dtype=torch.uint8, device=dev)]
    g_big = run(big)
    del big
    small = [torch.ones(1 << 26, dtype=torch.uint8, device=dev) for _ in range(8)]
    g_small = run(small)
    del small
    torch.cuda.synchronize()
    return {"kernel": "dsa_read_ceiling_stream (one event pair per call, median of 20)",
            "GBps_1GiB": round(g_big, 1), "GBps_64MiB_rotated_x8": round(g_small, 1)}


KERNEL_SOURCES = ("sparse_attention_decode_indexer_amd/csrc/index_topk.hip",
                  "sparse_attention_decode_indexer_amd/csrc/select_core.h",
                  "sparse_attention_decode_indexer_amd/csrc/select_geometry.h",
                  "sparse_attention_decode_indexer_amd/csrc/dsa_common.h")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "select_kernel_traffic_1m.txt")


def kernel_source_sha():
    """sha256 of the selection kernel's sources with // comments and blank lines removed."""
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), encoding="utf-8") as fh:
            for line in fh:
                code = line.split("//", 1)[0].strip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()


def measured_traffic(L, T):
    """HBM bytes per select_kernel launch from the committed FETCH_SIZE/WRITE_SIZE summary
    (1M context, T = 8 only), or None when the kernel changed since the counters were taken."""
    if L != (1 << 20) or T != 8 or not os.path.exists(TRAFFIC_FILE):
        return None
    vals = {}
    with open(TRAFFIC_FILE, encoding="utf-8") as fh:
        for line in fh:
            key, _, val = line.partition(":")
            vals[key.strip()] = val.strip()
    if vals.get("source_sha256") != kernel_source_sha():
        return None
    try:
        return int(vals["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(host_layers, x_host, L, T, bytes_step, with_configs=True):
    """The oracle (fp64 numpy, unmodified) on one full module step of the same workload,
    plus (with_configs) its indexer / top-k / attention stage times on each smaller config."""
    import numpy as np
    from oracle import dsa_oracle as O
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:
        cores = os.cpu_count() or 1
    x = x_host
    layer_s = {}
    t0 = time.perf_counter()
    for lay in host_layers:
        if lay.kind == "dsa":
            cache = {"k": lay.k.copy(), "v": lay.v.copy(), "k_idx": lay.k_idx.copy(),
                     "k_idx_scale": lay.k_idx_scale.copy()}
        else:
            cache = {"k": lay.k.copy(), "v": lay.v.copy(), "ring_cap": RING_CAP}
        tc = time.perf_counter()
        r = O.layer_step(lay.kind, x, lay.gamma, lay.w_qkvi, lay.w_o, cache, L - T)
        layer_s.setdefault(lay.kind, []).append(time.perf_counter() - tc)
        x = O.round_to_bf16(r["x_out_f64"])
        log(f"[bench] oracle {lay.kind} layer: {layer_s[lay.kind][-1]:.2f}s")
        if lay.kind == "dsa":
            dsa_r, dsa_cache = r, cache
    dt = time.perf_counter() - t0
    stages = oracle_stages(O, dsa_r, dsa_cache, L, T)
    stages["dsa_layer"] = round(layer_s["dsa"][0], 3)
    stages["swa_layer_mean"] = round(sum(layer_s["swa"]) / len(layer_s["swa"]), 3)
    log(f"[bench] oracle DSA stages (s): {stages}")
    per_config = None
    if with_configs:
        import synth
        per_config = {}
        for name, _ in CONFIGS:
            inp = synth.dsa_config(name, seed=0)
            t0 = time.perf_counter()
            krows = O.dequant_rows(inp.k_idx, inp.k_idx_dtype, inp.k_idx_scale)
            sc = O.indexer_scores(O.decode_bf16(inp.q_idx), inp.w_idx, krows, inp.pos0)
            t1 = time.perf_counter()
            ix, _ = O.topk_indices(sc, inp.pos0, inp.top_k)
            t2 = time.perf_counter()
            if inp.kv_dtype == "bf16":
                Kr = lambda j, a=inp.k: O.decode_bf16(a[j])
                Vr = lambda j, a=inp.v: O.decode_bf16(a[j])
            else:
                Kr = lambda j, a=inp.k, s=inp.k_scale: O.dequant_rows(a[j], "fp8", s[j])
                Vr = lambda j, a=inp.v, s=inp.v_scale: O.dequant_rows(a[j], "fp8", s[j])
            O.sparse_attention(O.decode_bf16(inp.q), Kr, Vr, ix, 1.0 / math.sqrt(128), L=inp.L)
            t3 = time.perf_counter()
            per_config[name] = {"indexer": round(t1 - t0, 3), "topk": round(t2 - t1, 3),
                                "attention": round(t3 - t2, 3), "tokens_per_s": round(inp.T / (t3 - t0), 2)}
            log(f"[bench] oracle {name} stages (s): {per_config[name]}")
    return {"value": round(bytes_step / dt / 1e9, 4), "unit": "GB/s", "cores": int(cores), "kind": "oracle",
            "sample": f"one full module step (5 SWA + 1 DSA layers, L={L}, T={T}), fp64 numpy oracle",
            "seconds": round(dt, 2), "cpu_model": cpu_model(), "stage_seconds": stages,
            "config_stage_seconds": per_config}


def oracle_stages(O, r, cache, L, T, K=2048):
    """Wall-clock of the oracle's DSA stages, re-run on the layer step's own post-RoPE
    projection and updated cache: indexer (key dequantisation + scores), top-k, attention."""
    off = O.proj_layout("dsa")

    def seg(name):
        o, n = off[name]
        return r["qkv"][:, o:o + n]
    t0 = time.perf_counter()
    krows = O.dequant_rows(cache["k_idx"][:L], "fp8", cache["k_idx_scale"][:L])
    scores = O.indexer_scores(seg("q_idx").reshape(T, 16, 64), seg("w_idx"), krows, L - T)
    t1 = time.perf_counter()
    idx, _ = O.topk_indices(scores, L - T, K)
    t2 = time.perf_counter()
    O.sparse_attention(seg("q").reshape(T, 8, 128), lambda j: O.decode_bf16(cache["k"][j]),
                       lambda j: O.decode_bf16(cache["v"][j]), idx, 1.0 / math.sqrt(128), L=L)
    t3 = time.perf_counter()
    return {"indexer": round(t1 - t0, 3), "topk": round(t2 - t1, 3), "attention": round(t3 - t2, 3)}


def cpu_model():
    try:
        with open("/proc/cpuinfo", encoding="utf-8") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


if __name__ == "__main__":
    main()
