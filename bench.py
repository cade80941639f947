"""Benchmark of the ST-DiT attention block on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 1080p|720p] [--no-cpu] [--no-sliced]

A step is one pass of the unsliced spatial + temporal layer pair over the
1080p 8 s latent (B=1, T=51, S=8160 on a 120x68 patch grid, C=1152,
16 heads x 72, bf16): QKV projection with RMSNorm and 2D RoPE, spatial
attention, output projection storing its rows in the [B,S,T,C] relayout,
QKV projection with 1D RoPE, temporal attention, output projection storing
its rows back in [B,T,S,C] order.  Inputs are seeded synthetic tensors
already resident in HBM.

The JSON line reports the whole-step throughput in algorithmic TFLOP/s, each
kernel's median duration from HIP events recorded on the launch stream, the
same step with the two relayouts as separate passes (bit-identical result),
the standalone relayout rate next to a same-run device-to-device copy and a
plain streaming copy of the same bytes, the QKV projection with and without its
norm/RoPE epilogue, the same layer pair at the 720p 4 s shape, a
roofline entry for the dominant kernel (spatial attention; its HBM traffic
comes from the committed rocprofv3 counter summary when that summary matches
the kernel source), the slicing schedule's time (N_T = N_S = 4, T padded to
52), the spatial attention at the 4096 px image shape (3 heads x 128), and the
fp64 oracle timed on a bounded sample on the host cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

METRIC = "ST-DiT attention block TFLOP/s + relayout GB/s (% of peak) at 1080p shape"
PEAK_BF16_TFLOPS = 2516.6      # MI355X dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 flop/clk
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E

WORKLOADS = {"1080p": 3, "720p": 2}
HERE = os.path.dirname(os.path.abspath(__file__))
ATTN_SOURCE = os.path.join(HERE, "temporal_attention_amd", "csrc", "attn_bf16.hip")
ATTN_TRAFFIC = os.path.join(HERE, "profiles", "attn_spatial_1080p_traffic.txt")


def measured_traffic(path=ATTN_TRAFFIC, source=ATTN_SOURCE):
    """HBM bytes per launch of the spatial attention kernel, from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE summary, scaled by its copy-kernel
    calibration factors; None if the summary is missing or was taken on a
    different version of the kernel source."""
    try:
        kv = {}
        with open(path) as f:
            for line in f:
                if ":" in line and not line.startswith("#"):
                    k, v = line.split(":", 1)
                    kv[k.strip()] = v.strip()
        with open(source, "rb") as f:
            sha = hashlib.sha256(f.read()).hexdigest()
        if kv.get("source_sha256") != sha:
            return None
        return 1024.0 * (float(kv["fetch_kib_per_dispatch"]) * float(kv["fetch_factor"])
                         + float(kv["write_kib_per_dispatch"]) * float(kv["write_factor"]))
    except (OSError, KeyError, ValueError):
        return None


def flops_and_bytes(B, T, S, C, H, d):
    N, hd = B * T * S, H * d
    f = {
        "qkv_spatial": 2.0 * N * C * 3 * hd,
        "attn_spatial": 4.0 * S * S * d * H * B * T,
        "proj_spatial": 2.0 * N * hd * C,
        "qkv_temporal": 2.0 * N * C * 3 * hd,
        "attn_temporal": 4.0 * T * T * d * H * B * S,
        "proj_temporal": 2.0 * N * hd * C,
    }
    by = {
        "relayout_fwd": 2.0 * N * C * 2,          # read + write every element once
        "relayout_bwd": 2.0 * N * C * 2,
        "attn_temporal": 4.0 * N * hd * 2,        # read q, k, v; write o
    }
    return f, by


def _oracle_attention_task(args):
    """One (frame, head) sequence of the spatial layer's attention, single-threaded BLAS."""
    import oracle
    from threadpoolctl import threadpool_limits
    q, k, v, scale = args
    with threadpool_limits(1):
        return oracle.attention(q, k, v, scale)


def cpu_baseline(cfg_id):
    """The fp64 oracle, as it stands, on a fixed sample of the same workload, on the host's cores.

    Sample: the spatial layer on nine evenly spaced frames (all heads, all patches; about 10 s on
    16 host cores at 1080p) and the temporal layer on 160 patches x all frames.  The attention of each (frame, head) sequence -- nearly all
    of the work -- runs in a pool of one single-threaded worker per host core; the projections and
    the temporal layer run in this process with the BLAS library's threads.  Throughput =
    algorithmic flops of the sample / wall time.  Runs before the GPU is touched (the pool's
    workers are fresh interpreters).
    """
    import multiprocessing as mp

    import oracle
    import st_synth
    from threadpoolctl import threadpool_info

    inp = st_synth.make_inputs(cfg_id)
    cfg = inp["cfg"]
    B, T, S, C, H, d, gw = cfg["B"], cfg["T"], cfg["S"], cfg["C"], cfg["H"], cfg["d"], cfg["grid_w"]
    eps, base = st_synth.EPS, st_synth.ROPE_BASE
    ws = dict(w_qkv=st_synth.to_f64(inp["w_qkv_s"]), w_o=st_synth.to_f64(inp["w_o_s"]),
              g_q=inp["g_q"].astype(np.float64), g_k=inp["g_k"].astype(np.float64))
    wt = dict(w_qkv=st_synth.to_f64(inp["w_qkv_t"]), w_o=st_synth.to_f64(inp["w_o_t"]),
              g_q=inp["g_q"].astype(np.float64), g_k=inp["g_k"].astype(np.float64))
    hd, scale = H * d, 1.0 / math.sqrt(d)
    frames = sorted({round(i * (T - 1) / 8) for i in range(9)})
    cores = len(os.sched_getaffinity(0))
    pool = mp.get_context("spawn").Pool(cores)
    pool.map(_oracle_attention_task, [(np.zeros((2, d)),) * 3 + (scale,)] * cores)   # workers up and imported
    t0 = time.perf_counter()
    pos = np.tile(oracle.positions_2d(S, gw), (B, 1))
    tasks, qkv_flops = [], 0.0
    for t in frames:
        x = st_synth.to_f64(inp["x"][:, t]).reshape(B * S, C)
        q, k, v = oracle.qkv_norm_rope(x, ws["w_qkv"], ws["g_q"], ws["g_k"], eps, H, d, "2d", pos, base)
        tasks += [(q[:, h], k[:, h], v[:, h], scale) for h in range(H)]
    outs = pool.map(_oracle_attention_task, tasks, chunksize=1)
    for f in range(len(frames)):   # the output projection of each frame's attention output
        o = np.stack(outs[f * H:(f + 1) * H], axis=1).reshape(B * S, hd)
        oracle.linear(o, ws["w_o"])
    flops = len(frames) * (2.0 * S * C * 3 * hd + 4.0 * S * S * d * H + 2.0 * S * hd * C)
    P = 160
    xt = oracle.bt_to_bs(st_synth.to_f64(inp["x"][:, :, :P]))
    oracle.temporal_layer(xt, wt, H, d, eps, base)
    flops += 2.0 * P * T * C * 3 * hd + 4.0 * T * T * d * H * P + 2.0 * P * T * hd * C
    dt = time.perf_counter() - t0
    pool.close()
    pool.join()
    threads = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"spatial layer on frames {frames} (all {S} patches x {H} heads; attention per (frame, head) "
                      f"in a pool of {cores} single-threaded workers, projections on {threads} BLAS threads) + "
                      f"temporal layer on {P} patches x {T} frames; fp64 numpy, {dt:.1f} s wall",
            "seconds": round(dt, 2), "host_cores_visible": cores}


def time_slicing(x, wsd, wtd, B, T, S, gw, C, H, d, stream, reps):
    """The slicing schedule at one GPU: T padded with zero frames to a multiple of N_T, the
    spatial layer per time slice and the temporal layer per space slice (t_valid = T), on one
    stream (st_block_sliced: the rearranges, gathers and scatters ride on the projections' row
    addressing) and with them as explicit copies on a second stream (st_block_sliced_2s).
    Headline N_T = N_S = 4 (T 52) plus the sweep N_T, N_S in {1,2,4,8}."""
    import torch

    import st_synth
    import temporal_attention_amd as st

    sp = st.layer_weights(wsd["w_qkv"], wsd["w_o"], wsd["g_q"], wsd["g_k"])
    tp = st.layer_weights(wtd["w_qkv"], wtd["w_o"], wtd["g_q"], wtd["g_k"])
    side = torch.cuda.Stream()   # default priority
    xv = x.view(B, T, S, C)
    ref = {}

    def run(nt, ns, two):
        TT = -(-T // nt) * nt
        xx = xv if TT == T else torch.cat([xv, torch.zeros_like(xv[:, :TT - T])], dim=1)
        query = st.st_block_sliced_2s_workspace if two else st.st_block_sliced_workspace
        nb = query(B, TT, S, gw, C, H, d, nt, ns, st.ST_BF16)
        ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
        y = torch.empty((B, TT, S, C), dtype=torch.bfloat16, device="cuda")
        if two:
            fn = lambda: st.st_block_sliced_2s(xx, B, TT, T, S, gw, C, H, d, nt, ns, sp, tp, st_synth.EPS,  # noqa: E731
                                               st_synth.ROPE_BASE, st.ST_BF16, y, ws, nb, side_stream=side)
        else:
            fn = lambda: st.st_block_sliced(xx, B, TT, T, S, gw, C, H, d, nt, ns, sp, tp, st_synth.EPS,  # noqa: E731
                                            st_synth.ROPE_BASE, st.ST_BF16, y, ws, nb)
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        same = None
        if (1, 1) in ref:
            same = bool(torch.equal(y[:, :T], ref[(1, 1)]))
        else:
            ref[(1, 1)] = y[:, :T].clone()
        del ws, y, xx
        return TT, ms, same

    sweep = {}
    for nt in (1, 2, 4, 8):
        for ns in (1, 2, 4, 8):
            TT, ms1, same1 = run(nt, ns, False)
            e = {"T": TT, "ms_one_stream": round(ms1, 4)}
            if nt * ns > 1:
                _, ms2, same2 = run(nt, ns, True)
                e.update(ms_two_streams=round(ms2, 4), bit_identical=bool(same1 and same2))
            sweep[f"{nt}x{ns}"] = e
    base = sweep["1x1"]["ms_one_stream"]
    head = sweep["4x4"]
    sliced = {"n_t": 4, "n_s": 4, "T_padded": head["T"], "ms": head["ms_one_stream"],
              "ms_two_streams": head["ms_two_streams"], "unsliced_native_ms": base,
              "overhead": round(head["ms_one_stream"] / base - 1.0, 4),
              "overhead_two_streams": round(head["ms_two_streams"] / base - 1.0, 4),
              "bit_identical_to_unsliced": head["bit_identical"]}
    return sliced, sweep


def time_v_change(lp, reps, stream):
    """V-Major change detection over the step's V ([N, H, d]) against a cache that differs on every
    fifth token (so ~20% of vectors are active at threshold 1.0), without refreshing the cache so
    every repetition sees the same input; one more call with the refresh."""
    import torch

    import temporal_attention_amd as st

    N, H, d = lp.N, lp.H, lp.d
    v = lp.v
    cache = v.clone()
    cache.view(N, H, d)[::5] += 1.0
    mask = torch.empty((N, H), dtype=torch.uint8, device="cuda")
    idx = torch.empty(N * H, dtype=torch.int32, device="cuda")
    cnt = torch.empty(1, dtype=torch.int64, device="cuda")
    run = lambda upd: st.st_v_change(v, cache, N, H, d, 1.0, st.ST_BF16, mask, idx, cnt, upd)  # noqa: E731
    run(0)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        run(0)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    n_act = int(cnt.item())
    nbytes = 2.0 * N * H * d * 2 + N * H + 4.0 * n_act      # read both V, write mask and indices
    e0.record(stream)
    run(1)
    e1.record(stream)
    torch.cuda.synchronize()
    ms_upd = e0.elapsed_time(e1)
    return {"vectors": N * H, "active": n_act, "threshold": 1.0, "ms": round(ms, 4),
            "gbs": round(nbytes / ms / 1e6, 1), "frac_hbm_peak": round(nbytes / ms / 1e6 / PEAK_HBM_GBS, 4),
            "ms_with_cache_refresh": round(ms_upd, 4)}


def time_image_attention(reps, stream):
    """Spatial attention at the 4096 px image shape (xDiT, "Experiments": image DiTs up to
    4096 px): one sequence of 65,536 latent tokens, 3 heads x 128, seeded N(0, 1) q, k, v in
    bf16; 4*S^2*d*H = 6.597 TFLOP per launch."""
    import torch

    import temporal_attention_amd as st

    S, H, d = 65536, 3, 128
    g = torch.Generator(device="cuda")
    g.manual_seed(4096)
    q, k, v = (torch.randn((1, S, H, d), device="cuda", generator=g).to(torch.bfloat16) for _ in range(3))
    o = torch.empty_like(q)
    run = lambda: st.st_attn_spatial(q, k, v, 1, 1, S, H, d, 1.0 / math.sqrt(d), st.ST_BF16, None, 0, o)  # noqa: E731
    run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        run()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    flops = 4.0 * S * S * d * H
    return {"workload": "4096px image DiT attention, 1 x 65536 tokens, 3 heads x 128", "ms": round(ms, 4),
            "tflops": round(flops / ms / 1e9, 1), "frac_mfma_peak": round(flops / ms / 1e9 / PEAK_BF16_TFLOPS, 4)}


def time_a2a_local(B, T, S, C, P, reps, stream):
    """One rank's local pack and unpack around the P-way all-to-all at the 1080p per-GPU shape
    (T padded to a multiple of P): each moves one rank's share, B*T*S*C/P elements, once."""
    import torch

    from temporal_attention_amd import a2a

    TT = -(-T // P) * P
    tp, sp = TT // P, S // P
    xs = torch.empty((B, TT, sp, C), dtype=torch.bfloat16, device="cuda")   # contents irrelevant to a copy
    xt = torch.empty((B, tp, S, C), dtype=torch.bfloat16, device="cuda")
    buf = torch.empty((P, B, tp, sp, C), dtype=torch.bfloat16, device="cuda")
    ops = {"pack_s2t": lambda: a2a.pack_s2t(xs, buf, B, TT, S, C, P),
           "unpack_s2t": lambda: a2a.unpack_s2t(buf, xt, B, TT, S, C, P),
           "pack_t2s": lambda: a2a.pack_t2s(xt, buf, B, TT, S, C, P),
           "unpack_t2s": lambda: a2a.unpack_t2s(buf, xs, B, TT, S, C, P)}
    nbytes = 2.0 * xs.numel() * 2
    res = {"P": P, "T_padded": TT, "rank_shape": [B, TT, sp, C], "bytes_moved_per_op": int(nbytes),
           "note": "one rank's share (0.13 GB) fits the 256 MB Infinity Cache, so rates can exceed HBM's"}
    for name, fn in ops.items():
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        # Each copy is shorter than a Python call through the binding, so the GPU is
        # held busy while the host enqueues the timed calls: the events then time the
        # kernels back to back, not the host's launch rate.
        torch.cuda._sleep(20_000_000)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        res[name] = {"ms": round(ms, 4), "gbs": round(nbytes / ms / 1e6, 1)}
    return res


def time_chunked_attention(lp, B, T, S, H, d, reps, stream, n_chunks=4):
    """Spatial attention of the step's q, k, v as a 4-way key split, the work of one GPU of a
    4-way ring: st_attn_chunk per key chunk (with log-sum-exp), folded together by three
    in-place st_attn_merge calls, and the same with the merges inside the attention epilogue
    (st_attn_chunk_acc); against one st_attn_chunk over all keys."""
    import torch

    import temporal_attention_amd as st

    outer, scale = B * T, 1.0 / math.sqrt(d)
    bounds = [S * i // n_chunks for i in range(n_chunks + 1)]
    kc = [lp.k.view(outer, S, H, d)[:, a:b].contiguous() for a, b in zip(bounds, bounds[1:])]
    vc = [lp.v.view(outer, S, H, d)[:, a:b].contiguous() for a, b in zip(bounds, bounds[1:])]
    acc, part = torch.empty_like(lp.o), torch.empty_like(lp.o)
    lse_acc = torch.empty((outer, H, S), dtype=torch.float32, device="cuda")
    lse_part = torch.empty_like(lse_acc)
    times = {}

    def whole():
        st.st_attn_chunk(lp.q, lp.k, lp.v, outer, S, S, S, H, d, scale, st.ST_BF16, acc, lse_acc)

    def chunked():
        for i, (a, b) in enumerate(zip(bounds, bounds[1:])):
            dst, dl = (acc, lse_acc) if i == 0 else (part, lse_part)
            st.st_attn_chunk(lp.q, kc[i], vc[i], outer, S, b - a, b - a, H, d, scale, st.ST_BF16, dst, dl)
            if i:
                st.st_attn_merge(acc, lse_acc, part, lse_part, outer, S, H, d, st.ST_BF16, acc, lse_acc)

    def merge_only():
        st.st_attn_merge(acc, lse_acc, part, lse_part, outer, S, H, d, st.ST_BF16, acc, lse_acc)

    def fused():   # first chunk fresh, later chunks merged in the attention epilogue
        for i, (a, b) in enumerate(zip(bounds, bounds[1:])):
            fn = st.st_attn_chunk if i == 0 else st.st_attn_chunk_acc
            fn(lp.q, kc[i], vc[i], outer, S, b - a, b - a, H, d, scale, st.ST_BF16, acc, lse_acc)

    for name, fn in (("whole", whole), ("chunked", chunked), ("merge", merge_only), ("fused", fused)):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        times[name] = e0.elapsed_time(e1) / reps
    fl = 4.0 * S * S * d * H * outer
    merge_bytes = outer * S * H * (3 * d * 2 + 3 * 4)     # read two rows + lse, write one row + lse
    return {"n_chunks": n_chunks, "ms": round(times["chunked"], 4), "unchunked_with_lse_ms": round(times["whole"], 4),
            "overhead": round(times["chunked"] / times["whole"] - 1.0, 4),
            "fused_merge_ms": round(times["fused"], 4),
            "fused_merge_overhead": round(times["fused"] / times["whole"] - 1.0, 4),
            "tflops": round(fl / times["chunked"] / 1e9, 1), "merge_ms": round(times["merge"], 4),
            "merge_gbs": round(merge_bytes / times["merge"] / 1e6, 1),
            "merge_frac_hbm_peak": round(merge_bytes / times["merge"] / 1e6 / PEAK_HBM_GBS, 4)}


def median_ms(fn, reps, stream):
    """Median of `reps` single-call durations, HIP events on the launch stream, after one warm-up call."""
    import torch
    fn()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for e0, e1 in ev:
        e0.record(stream)
        fn()
        e1.record(stream)
    torch.cuda.synchronize()
    return float(np.median([e0.elapsed_time(e1) for e0, e1 in ev]))


def time_layer_pair(cfg_id, steps, warmup, stream):
    """The unsliced layer pair of one workload, step by step through the C ABI: per-kernel medians of HIP
    events on the launch stream, and the wall time per step bracketed by synchronize on both sides."""
    import torch

    import st_synth
    from temporal_attention_amd.pipeline import LayerPair

    inp = st_synth.make_inputs(cfg_id)
    cfg = inp["cfg"]
    B, T, S, C, H, d, gw = cfg["B"], cfg["T"], cfg["S"], cfg["C"], cfg["H"], cfg["d"], cfg["grid_w"]

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)

    x = dev(inp["x"])
    wsd = dict(w_qkv=dev(inp["w_qkv_s"]), w_o=dev(inp["w_o_s"]), g_q=torch.from_numpy(inp["g_q"]).cuda(),
               g_k=torch.from_numpy(inp["g_k"]).cuda())
    wtd = dict(w_qkv=dev(inp["w_qkv_t"]), w_o=dev(inp["w_o_t"]), g_q=torch.from_numpy(inp["g_q"]).cuda(),
               g_k=torch.from_numpy(inp["g_k"]).cuda())
    lp = LayerPair(B, T, S, gw, C, H, d)
    lp.set_weights(wsd, wtd)
    lsteps = lp.steps(x)
    names = [n for n, _ in lsteps]
    for _ in range(warmup):
        for _, fn in lsteps:
            fn()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(lsteps) + 1)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        ev[i][0].record(stream)
        for j, (_, fn) in enumerate(lsteps):
            fn()
            ev[i][j + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = {n: float(np.median([ev[i][j].elapsed_time(ev[i][j + 1]) for i in range(steps)]))
           for j, n in enumerate(names)}
    step_ms = float(np.median([ev[i][0].elapsed_time(ev[i][-1]) for i in range(steps)]))
    fl, by = flops_and_bytes(B, T, S, C, H, d)
    kernels = {}
    for n in names:
        e = {"ms": round(per[n], 4)}
        if n in fl:
            e["tflops"] = round(fl[n] / per[n] / 1e9, 1)
            e["frac_mfma_peak"] = round(fl[n] / per[n] / 1e9 / PEAK_BF16_TFLOPS, 4)
        if n in by:
            e["gbs"] = round(by[n] / per[n] / 1e6, 1)
            e["frac_hbm_peak"] = round(by[n] / per[n] / 1e6 / PEAK_HBM_GBS, 4)
        kernels[n] = e
    res = {"per": per, "kernels": kernels, "flops": fl, "bytes": by, "ms_per_step": wall * 1e3 / steps,
           "step_ms_median": step_ms}
    return lp, x, wsd, wtd, inp, cfg, res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="1080p", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--no-sliced", action="store_true", help="skip timing the slicing schedule")
    ap.add_argument("--no-chunked", action="store_true", help="skip timing chunked attention + merges")
    ap.add_argument("--no-a2a", action="store_true", help="skip timing the all-to-all pack/unpack")
    ap.add_argument("--no-vchange", action="store_true", help="skip timing the V-Major change detection")
    ap.add_argument("--no-image", action="store_true", help="skip timing attention at the 4096px image shape")
    ap.add_argument("--no-720p", action="store_true", help="skip the 720p layer-pair row")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); it has no multi-GPU mode",
              file=sys.stderr)
        sys.exit(2)

    cfg_id = WORKLOADS[args.workload]
    cpu = None if args.no_cpu else cpu_baseline(cfg_id)   # before the GPU is touched

    import torch

    import temporal_attention_amd as st
    from temporal_attention_amd.pipeline import LayerPair

    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    lp, x, wsd, wtd, inp, cfg, res = time_layer_pair(cfg_id, args.steps, args.warmup, stream)
    B, T, S, C, H, d, gw = cfg["B"], cfg["T"], cfg["S"], cfg["C"], cfg["H"], cfg["d"], cfg["grid_w"]
    per, kernels, fl, by = res["per"], res["kernels"], res["flops"], res["bytes"]
    ms_per_step, step_ms = res["ms_per_step"], res["step_ms_median"]
    total_flops = sum(fl.values())
    attn_achieved = fl["attn_spatial"] / per["attn_spatial"] / 1e9

    # The step stores both relayouts from the output projections.  The same step with separate
    # relayout passes (bit-identical result), and the relayout kernel on its own at full size.
    unfused = lp.steps(x, fused=False)
    for _, fn in unfused:
        fn()
    torch.cuda.synchronize()
    u0 = time.perf_counter()
    for _ in range(args.steps):
        for _, fn in unfused:
            fn()
    torch.cuda.synchronize()
    unfused_ms = (time.perf_counter() - u0) * 1e3 / args.steps
    rl = {}
    for name, fn in unfused:
        if name.startswith("relayout"):
            rl[name] = median_ms(fn, max(5, args.steps), stream)
            kernels[name + "_standalone"] = {"ms": round(rl[name], 4), "gbs": round(by[name] / rl[name] / 1e6, 1),
                                             "frac_hbm_peak": round(by[name] / rl[name] / 1e6 / PEAK_HBM_GBS, 4)}
    relayout_ms = rl["relayout_fwd"] + rl["relayout_bwd"]
    relayout_gbs = (by["relayout_fwd"] + by["relayout_bwd"]) / relayout_ms / 1e6

    # ceilings of a relayout, same run: torch's device-to-device copy of the same bytes, and a plain
    # contiguous copy by the relayout kernel itself (identity strides: one lane per 16 bytes)
    cp_dst = torch.empty_like(x)
    copy_gbs = by["relayout_fwd"] / median_ms(lambda: cp_dst.copy_(x), max(5, args.steps), stream) / 1e6
    n_el = x.numel()
    stream_ms = median_ms(lambda: st.st_relayout(x, [1], cp_dst, [1], [n_el], 1, 2), max(5, args.steps), stream)
    stream_gbs = by["relayout_fwd"] / stream_ms / 1e6
    del cp_dst
    traffic = measured_traffic()

    # The QKV projection with and without its RMSNorm + RoPE epilogue: the plain projection of the
    # same shape is st_out_proj with the 3*H*d output rows of w_qkv.  The difference is what the
    # fused norm costs; done as its own pass it would move 4*N*H*d*2 bytes (read q, k; write q, k).
    N, hd = B * T * S, H * d
    plain = torch.empty((N, 3 * hd), dtype=torch.bfloat16, device="cuda")
    qkv_plain_ms = median_ms(lambda: st.st_out_proj(x, N, C, wsd["w_qkv"], 3 * hd, st.ST_BF16, plain),
                             max(5, args.steps), stream)
    del plain
    norm_bytes = 4.0 * N * hd * 2
    epilogue = {"qkv_with_norm_rope_ms": round(per["qkv_spatial"], 4), "qkv_plain_ms": round(qkv_plain_ms, 4),
                "fused_norm_rope_ms": round(per["qkv_spatial"] - qkv_plain_ms, 4),
                "standalone_norm_rope_bytes": int(norm_bytes),
                "standalone_norm_rope_ms_at_stream_rate": round(norm_bytes / (stream_gbs * 1e6), 4),
                "note": "a separate norm/RoPE pass would read and write q and k once (at the same-run streaming "
                        "copy rate); fused into the projection epilogue it moves no extra HBM bytes"}

    out = {
        "metric": METRIC,
        "value": round(total_flops / ms_per_step / 1e9, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "ms_per_step_events": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{cfg['name']} ST-DiT layer pair (spatial + temporal; both relayouts stored by the "
                               "output projections)", "B": B, "T": T,
                   "S": S, "grid": f"{gw}x{S // gw}", "C": C, "heads": H, "head_dim": d,
                   "step_tflop": round(total_flops / 1e12, 3)},
        "ms_per_step_separate_relayouts": round(unfused_ms, 4),
        "relayout_gbs": round(relayout_gbs, 1),
        "relayout_frac_hbm_peak": round(relayout_gbs / PEAK_HBM_GBS, 4),
        "device_copy_gbs": round(copy_gbs, 1),
        "streaming_copy_gbs": round(stream_gbs, 1),
        "relayout_frac_of_streaming_copy": round(relayout_gbs / stream_gbs, 4),
        "timing": "per-kernel figures are medians over the timed steps of HIP events on the launch stream",
        "kernels": kernels,
        "qkv_epilogue": epilogue,
        "roofline": {"kernel": "attn_long_kernel<72, 2, true> (spatial attention)", "bound": "mfma",
                     "achieved": round(attn_achieved, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(attn_achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": None if traffic is None else round(traffic / 1e9, 4),
                     "traffic_unit": "GB of HBM traffic per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, calibrated)",
                     "algorithmic_bytes": round(4.0 * B * T * S * H * d * 2 / 1e9, 4)},
    }

    if cfg_id != 2 and not args.no_720p:
        # the 720p 4 s workload (B=1, T=24, S=3600 on 80x45), same launch sequence, medians
        del lp
        torch.cuda.empty_cache()
        lp2, x2, _, _, _, cfg2, r2 = time_layer_pair(2, args.steps, args.warmup, stream)
        tf2 = sum(r2["flops"].values())
        out["workload_720p"] = {"config": {k: cfg2[k] for k in ("B", "T", "S", "C", "H", "d", "grid_w")},
                                "ms_per_step": round(r2["ms_per_step"], 4),
                                "tflops": round(tf2 / r2["ms_per_step"] / 1e9, 1),
                                "kernels": r2["kernels"]}
        del lp2, x2
        torch.cuda.empty_cache()
        lp = LayerPair(B, T, S, gw, C, H, d)
        lp.set_weights(wsd, wtd)
        for _, fn in lp.steps(x):
            fn()

    if not args.no_sliced:
        out["sliced"], out["slicing_sweep"] = time_slicing(x, wsd, wtd, B, T, S, gw, C, H, d, stream,
                                                           max(2, args.steps // 5))
        torch.cuda.empty_cache()

    if not args.no_chunked:
        lp.steps(x)[0][1]()   # the spatial layer's q, k, v again (the timed steps end on the temporal layer)
        out["chunked_attention"] = time_chunked_attention(lp, B, T, S, H, d, max(2, args.steps // 2), stream)

    if not args.no_vchange:
        out["v_change"] = time_v_change(lp, max(3, args.steps), stream)

    if not args.no_a2a:
        out["a2a_local"] = time_a2a_local(B, T, S, C, 8, max(3, args.steps), stream)

    if not args.no_image:
        out["attn_image_4096px"] = time_image_attention(max(3, args.steps // 2), stream)

    if cpu is not None:
        out["cpu_baseline"] = cpu
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
