"""Benchmark of the single-GPU MoE-layer forward (route, permute, grouped FFN, combine).

One step = one moe_forward over the whole prefill batch (T=8192 tokens,
H=2048, F=768, E=128 routed experts, top-8, bf16 operands, fp32 accumulation),
inputs resident in HBM. Prints ONE JSON line with the layer's tokens/s, the
grouped FFN's MFMA roofline (live HIP-event timing, the vendor library's dense
rate on the same FLOPs beside it), per-stage times with and without the MALL
evicted and their HBM fractions, the grouped FFN with h kept on chip beside
the two-launch one, the decode-shaped layer (T=32; weight stream, graph
replay, fp8 and MX fp8 experts), the Mixtral-like layer with a shared expert
and the skewed-routing layer, ceilings measured on the same GPU (bare MFMA loop,
streaming read, the GEMM k-step, a large library GEMM), and the fp64 CPU oracle timed on the
host as a baseline.

Usage: python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--no-cpu-baseline]
       python bench.py --only {tiny,decode,prefill,mixtral_shared,skew}   (one workload's record)
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def event_time_ms(fn, reps, stream, evict=None):
    """Mean HIP-event time of fn on `stream` over `reps` calls after one untimed call. With `evict` (a device
    buffer larger than the 256 MB MALL), every rep is timed on its own after a write of that whole buffer, so the
    rep starts with its inputs out of the last-level cache; without it the reps run back to back."""
    import torch

    fn()
    if evict is None:
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        start.record(stream)
        for _ in range(reps):
            fn()
        end.record(stream)
        end.synchronize()
        return start.elapsed_time(end) / reps
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(reps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(reps)]
    for r in range(reps):
        evict.fill_(r & 0x7F)  # same stream as fn: the write completes before the rep starts
        starts[r].record(stream)
        fn()
        ends[r].record(stream)
    ends[-1].synchronize()
    return sum(a.elapsed_time(b) for a, b in zip(starts, ends)) / reps


EVICT_BYTES = 1 << 30  # > 4x the 256 MB MALL


def evict_buffer():
    import torch

    return torch.empty(EVICT_BYTES, dtype=torch.uint8, device="cuda")


def stage_times(d, I, reps):
    """Per-stage HIP-event times (ms) through the step-wise C-ABI calls, on the current stream."""
    import torch

    import top_routing_grouped_gemm_amd as moe

    s = torch.cuda.current_stream()
    T, k, E, H, F = I.T, I.k, I.E, I.H, I.F
    dev = d["x"].device
    ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    w = torch.empty((T, k), dtype=torch.float32, device=dev)
    x_perm = torch.empty((T * k, H), dtype=d["x"].dtype, device=dev)
    off = torch.empty(E + 1, dtype=torch.int32, device=dev)
    row_token = torch.empty(T * k, dtype=torch.int32, device=dev)
    inv = torch.empty((T, k), dtype=torch.int32, device=dev)
    pws = torch.empty(moe.moe_permute_workspace_bytes(T, E, k), dtype=torch.uint8, device=dev)
    fws = torch.empty(moe.moe_ffn_workspace_bytes(T, F, E, k, I.Fs, d["x"].dtype), dtype=torch.uint8, device=dev)
    y_perm = torch.empty((T * k, H), dtype=torch.float32, device=dev)
    y = torch.empty((T, H), dtype=torch.float32, device=dev)
    y_sh = torch.empty((T, H), dtype=torch.float32, device=dev) if I.Fs else None

    def route():
        moe.moe_route(d["x"], d["Wr"], d["bias"], k, I.drop, topk_ids=ids, topk_w=w)

    def permute():
        moe.moe_permute(d["x"], ids, w, E, x_perm=x_perm, expert_offsets=off, row_token=row_token, inv=inv, ws=pws)

    def ffn():  # routed experts, plus the shared expert when the workload has one
        moe.moe_grouped_ffn(x_perm, off, d["W1"], d["W2"], T, k, y_perm=y_perm, x=d["x"], W1s=d["W1s"], W2s=d["W2s"],
                            y_shared=y_sh, ws=fws)

    def combine():
        moe.moe_combine(y_perm, inv, w, y_shared=y_sh, y=y)

    def ffn_fused():  # the same routed FFN in one launch with h kept in LDS (shapes it covers only)
        moe.moe_grouped_ffn_fused(x_perm, off, d["W1"], d["W2"], T, k, y_perm=y_perm)

    route()
    permute()
    torch.cuda.synchronize()
    A = int(off[-1].item())
    counts = (off[1:] - off[:-1]).cpu()
    stages = (("route", route), ("permute", permute), ("grouped_ffn", ffn), ("combine", combine))
    out = {name: event_time_ms(fn, reps, s) for name, fn in stages}
    fused_ok = (d["x"].dtype == torch.bfloat16 and not I.Fs and F % 256 == 0 and F <= 768 and H % 256 == 0)
    fused = event_time_ms(ffn_fused, reps, s) if fused_ok else None
    ev = evict_buffer()
    cold = {name: event_time_ms(fn, reps, s, evict=ev) for name, fn in stages}
    del ev
    return out, cold, A, counts, fused


def bytes_model(I, A, experts_hit, out_bytes=4):
    """Algorithmic HBM bytes per call of each stage (each array read or written once).

    out_bytes = 4: the formats the step-wise calls actually use (fp32 y_perm, y_shared and y); out_bytes = b
    (the operand width, 2 for bf16): the method's own formats, y_perm and y in the operand type, the byte
    counts of the hot-path scope table. h never leaves the grouped FFN and is not counted."""
    b = I.elem_bytes
    o = out_bytes
    T, H, F, E, k = I.T, I.H, I.F, I.E, I.k
    Fs = I.Fs
    shared_ffn = (2 * H * Fs * b + T * H * b + T * H * o) if Fs else 0  # W1s, W2s, x read, y_shared written
    return {
        "route": T * H * b + H * E * b + T * k * 8,
        "permute": T * H * b + A * H * b + T * k * 8 * 2 + A * 4,
        "grouped_ffn": experts_hit * 2 * H * F * b + A * H * b + A * H * o + shared_ffn,
        "combine": A * H * o + T * k * 8 + T * H * o + (T * H * o if Fs else 0),
    }


def library_dense_gemm(M, K, N, reps=20):
    """Context for the grouped-GEMM roofline: the vendor library's dense bf16 GEMM (torch.mm -> hipBLASLt) with
    the same FLOPs as one expert launch (all rows in one matrix, no gather, no grouping). Returns ms."""
    import torch

    dev = torch.device("cuda:0")
    a = torch.randn(M, K, device=dev, dtype=torch.bfloat16)
    b = torch.randn(K, N, device=dev, dtype=torch.bfloat16)
    c = torch.mm(a, b)
    t = event_time_ms(lambda: torch.mm(a, b, out=c), reps, torch.cuda.current_stream())
    del a, b, c
    return t


def run_workload(name, steps, warmup, stage_reps, graph=False):
    import numpy as np
    import torch

    import gen
    import top_routing_grouped_gemm_amd as moe

    dev = torch.device("cuda:0")
    t0 = time.time()
    I = gen.make_inputs(name)
    d = gen.to_device(I, dev)
    log(f"[bench] {name}: inputs ready in {time.time() - t0:.1f}s")
    ws = torch.empty(moe.moe_workspace_bytes(I.T, I.H, I.F, I.E, I.k, I.Fs, d["x"].dtype), dtype=torch.uint8,
                     device=dev)
    y = torch.empty((I.T, I.H), dtype=torch.float32, device=dev)

    def step():
        moe.moe_forward(d["x"], d["Wr"], d["bias"], d["W1"], d["W2"], I.k, I.drop, W1s=d["W1s"], W2s=d["W2s"], y=y,
                        ws=ws)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t) * 1e3 / steps
    graph_ms = None
    if graph:  # the same layer captured once in a HIP graph and replayed (no per-kernel launch from the host)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        for _ in range(warmup):
            g.replay()
        torch.cuda.synchronize()
        t = time.perf_counter()
        for _ in range(steps):
            g.replay()
        torch.cuda.synchronize()
        graph_ms = (time.perf_counter() - t) * 1e3 / steps
        del g
    st, cold, A, counts, fused = stage_times(d, I, stage_reps)
    hit = int((counts > 0).sum())
    flops = 4.0 * A * I.H * I.F + 4.0 * I.T * I.H * I.Fs  # routed experts + shared expert
    byts = bytes_model(I, A, hit)
    byts_m = bytes_model(I, A, hit, out_bytes=I.elem_bytes)

    def frac(bm, times):
        return {k_: round(bm[k_] / (times[k_] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4) for k_ in times}

    res = {
        "T": I.T, "H": I.H, "F": I.F, "E": I.E, "k": I.k, "A": A, "experts_hit": hit,
        "rows_per_expert": {"min": int(counts.min()), "max": int(counts.max()),
                            "mean": float(counts.float().mean())},
        "ms_per_step": ms, "tokens_per_s": I.T / (ms * 1e-3),
        **({"graph_replay": {"ms_per_step": graph_ms, "tokens_per_s": I.T / (graph_ms * 1e-3)}} if graph_ms else {}),
        "stages_ms": {k: round(v, 5) for k, v in st.items()},
        "stages_ms_mall_evicted": {k: round(v, 5) for k, v in cold.items()},
        "stage_gbs": {k: round(byts[k] / (st[k] * 1e-3) / 1e9, 1) for k in st},
        "stage_hbm_frac": frac(byts, st),
        "stage_hbm_frac_mall_evicted": frac(byts, cold),
        "stage_hbm_frac_method_bytes": frac(byts_m, st),
        "stage_hbm_frac_method_bytes_mall_evicted": frac(byts_m, cold),
        "grouped_ffn_tflops": flops / (st["grouped_ffn"] * 1e-3) / 1e12,
        "grouped_ffn_mfma_frac": round(flops / (st["grouped_ffn"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "weight_stream_gbs": round((hit * 2 * I.H * I.F + 2 * I.H * I.Fs) * I.elem_bytes
                                   / (st["grouped_ffn"] * 1e-3) / 1e9, 1),
        "grouped_ffn_flops": flops,
        **({"grouped_ffn_h_on_chip": {
            "ms": round(fused, 5), "tflops": round(flops / (fused * 1e-3) / 1e12, 1),
            "vs_two_launch": round(st["grouped_ffn"] / fused, 3),
            "note": "moe_grouped_ffn_fused: W1, SiLU and W2 in one launch, h in LDS (64-row tiles); vs_two_launch "
                    "> 1 means faster than moe_grouped_ffn"}} if fused is not None else {}),
        "algorithmic_bytes": byts,
        "method_bytes": byts_m,
        "bytes_note": "algorithmic_bytes: each array once in the formats the step-wise calls use (fp32 y_perm, "
                      "y_shared, y); method_bytes: y_perm, y_shared and y in the operand type (the scope table's "
                      "counts); *_mall_evicted: each rep timed alone after a 1 GiB write that evicts the MALL",
    }
    del d, ws
    torch.cuda.empty_cache()
    return I, res


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "grouped_ffn_hbm_traffic.txt")
KERNEL_SOURCES = ("gemm_dma.hpp", "grouped_ffn.hip", "moe_common.hpp")


def measured_traffic(key):
    """HBM bytes per moe_grouped_ffn call from the committed rocprofv3 counter summary, or None when the
    grouped-FFN kernel sources changed since those counters were taken (the summary records their SHA-256)."""
    import hashlib

    try:
        text = open(TRAFFIC_FILE).read()
    except OSError:
        return None
    csrc = os.path.join(ROOT, "top_routing_grouped_gemm_amd", "csrc")
    sha = hashlib.sha256(b"".join(open(os.path.join(csrc, f), "rb").read() for f in KERNEL_SOURCES)).hexdigest()
    recorded = next((l.split(":", 1)[1].split()[0] for l in text.splitlines() if "kernel_source_sha256:" in l), None)
    if recorded != sha:
        return None
    for l in text.splitlines():
        if l.startswith(key + ":"):
            return int(l.split(":", 1)[1])
    return None


def capacity_times(name, factor, reps=50):
    """Capacity-limited routing next to plain routing on one workload: HIP-event times of moe_route and
    moe_route_capacity (router logits + capacity selection), the capacity, and the largest expert before/after."""
    import numpy as np
    import torch

    import gen
    import top_routing_grouped_gemm_amd as moe

    dev = torch.device("cuda:0")
    I = gen.make_inputs(name)
    d = gen.to_device(I, dev)
    s = torch.cuda.current_stream()
    T, H, E, k = I.T, I.H, I.E, I.k
    ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    w = torch.empty((T, k), dtype=torch.float32, device=dev)
    lib = moe.load_library()
    rws = torch.empty(max(moe.moe_route_workspace_bytes(T, H, E, d["x"].dtype), 1), dtype=torch.uint8, device=dev)
    cws = torch.empty(lib.moe_route_capacity_workspace_bytes(T, H, E, moe.MOE_BF16), dtype=torch.uint8, device=dev)

    def plain():
        moe.moe_route(d["x"], d["Wr"], d["bias"], k, I.drop, topk_ids=ids, topk_w=w, ws=rws)

    def capped():
        moe.moe_route_capacity(d["x"], d["Wr"], d["bias"], k, I.drop, factor, topk_ids=ids, topk_w=w, ws=cws)

    plain()
    torch.cuda.synchronize()
    before = int(torch.bincount(ids.flatten().long(), minlength=E).max())
    t_plain = event_time_ms(plain, reps, s)
    t_cap = event_time_ms(capped, reps, s)
    after = int(torch.bincount(ids.flatten().long(), minlength=E).max())
    cap = int(np.ceil(T * k / E * float(factor)))
    return {"workload": name, "capacity_factor": factor, "capacity": cap, "route_ms": round(t_plain, 5),
            "route_capacity_ms": round(t_cap, 5), "max_rows_per_expert": {"plain": before, "capped": after}}


def padded_times(name, reps=10):
    """Ablation: the padded fixed-shape layout (every expert padded to the largest count C) against the ragged
    grouped FFN on one workload. HIP-event times of dispatch, grouped FFN and combine for both, and the padded
    work relative to the ragged work (E*C rows against A)."""
    import torch

    import gen
    import top_routing_grouped_gemm_amd as moe

    dev = torch.device("cuda:0")
    I = gen.make_inputs(name)
    d = gen.to_device(I, dev)
    s = torch.cuda.current_stream()
    ids, w = moe.moe_route(d["x"], d["Wr"], d["bias"], I.k, I.drop)
    x_perm, off, row_token, inv = moe.moe_permute(d["x"], ids, w, I.E)
    torch.cuda.synchronize()
    counts = (off[1:] - off[:-1]).cpu()
    A, C = int(counts.sum()), int(counts.max())
    E, T, k, H = I.E, I.T, I.k, I.H
    y_perm = torch.empty((T * k, H), dtype=torch.float32, device=dev)
    fws = torch.empty(moe.moe_ffn_workspace_bytes(T, I.F, E, k, 0, d["x"].dtype), dtype=torch.uint8, device=dev)
    x_pad = torch.empty((E * C, H), dtype=d["x"].dtype, device=dev)
    inv_pad = torch.empty((T, k), dtype=torch.int32, device=dev)
    y_pad = torch.empty((E * C, H), dtype=torch.float32, device=dev)
    pws = torch.empty(moe.load_library().moe_grouped_ffn_padded_workspace_bytes(E, C, H, I.F, moe.MOE_BF16),
                      dtype=torch.uint8, device=dev)
    y = torch.empty((T, H), dtype=torch.float32, device=dev)
    rag = {
        "dispatch": event_time_ms(lambda: moe.moe_permute(d["x"], ids, w, E, x_perm=x_perm, expert_offsets=off,
                                                          row_token=row_token, inv=inv), reps, s),
        "grouped_ffn": event_time_ms(lambda: moe.moe_grouped_ffn(x_perm, off, d["W1"], d["W2"], T, k, y_perm=y_perm,
                                                                 ws=fws), reps, s),
        "combine": event_time_ms(lambda: moe.moe_combine(y_perm, inv, w, y=y), reps, s),
    }
    pad = {
        "dispatch": event_time_ms(lambda: moe.moe_pad_dispatch(d["x"], ids, off, row_token, inv, E, C, x_pad=x_pad,
                                                               inv_pad=inv_pad), reps, s),
        "grouped_ffn": event_time_ms(lambda: moe.moe_grouped_ffn_padded(x_pad, d["W1"], d["W2"], C, y_pad=y_pad,
                                                                        ws=pws), reps, s),
        "combine": event_time_ms(lambda: moe.moe_combine(y_pad, inv_pad, w, y=y), reps, s),
    }
    return {"workload": name, "rows_ragged": A, "experts": E, "pad_rows_per_expert": C, "rows_padded": E * C,
            "padding_flop_ratio": round(E * C / A, 3),
            "ragged_ms": {k_: round(v, 5) for k_, v in rag.items()},
            "padded_ms": {k_: round(v, 5) for k_, v in pad.items()},
            "grouped_ffn_speedup_of_ragged": round(pad["grouped_ffn"] / rag["grouped_ffn"], 3)}


def fp8_times(name, steps=20, reps=20):
    """fp8 expert weights next to bf16 on one workload: the one-time quantisation, the whole layer
    (moe_forward_fp8 against moe_forward) and the grouped FFN alone (HIP events), with the weight bytes each
    streams (fp8: one byte per weight plus the per-column scales)."""
    import torch

    import gen
    import top_routing_grouped_gemm_amd as moe

    dev = torch.device("cuda:0")
    I = gen.make_inputs(name)
    d = gen.to_device(I, dev)
    s = torch.cuda.current_stream()
    T, H, F, E, k = I.T, I.H, I.F, I.E, I.k
    W1q, s1 = moe.moe_quantize_fp8(d["W1"])
    W2q, s2 = moe.moe_quantize_fp8(d["W2"])
    t_quant = event_time_ms(lambda: (moe.moe_quantize_fp8(d["W1"], Wq=W1q, scales=s1),
                                     moe.moe_quantize_fp8(d["W2"], Wq=W2q, scales=s2)), 3, s)
    ws = torch.empty(moe.moe_workspace_bytes(T, H, F, E, k, 0, torch.bfloat16), dtype=torch.uint8, device=dev)
    y = torch.empty((T, H), dtype=torch.float32, device=dev)
    fwd8 = event_time_ms(lambda: moe.moe_forward_fp8(d["x"], d["Wr"], d["bias"], W1q, s1, W2q, s2, k, I.drop, y=y,
                                                     ws=ws), steps, s)
    fwd16 = event_time_ms(lambda: moe.moe_forward(d["x"], d["Wr"], d["bias"], d["W1"], d["W2"], k, I.drop, y=y,
                                                  ws=ws), steps, s)
    ids, w = moe.moe_route(d["x"], d["Wr"], d["bias"], k, I.drop)
    x_perm, off, row_token, inv = moe.moe_permute(d["x"], ids, w, E)
    torch.cuda.synchronize()
    counts = (off[1:] - off[:-1]).cpu()
    hit, A = int((counts > 0).sum()), int(counts.sum())
    y_perm = torch.empty((T * k, H), dtype=torch.float32, device=dev)
    fws = torch.empty(moe.moe_ffn_workspace_bytes(T, F, E, k, 0, torch.bfloat16), dtype=torch.uint8, device=dev)
    ffn8 = event_time_ms(lambda: moe.moe_grouped_ffn_fp8(x_perm, off, W1q, s1, W2q, s2, T, k, y_perm=y_perm, ws=fws),
                         reps, s)
    ffn16 = event_time_ms(lambda: moe.moe_grouped_ffn(x_perm, off, d["W1"], d["W2"], T, k, y_perm=y_perm, ws=fws),
                          reps, s)
    w8 = hit * (2 * H * F + 4 * (H + F))
    w16 = hit * 2 * H * F * 2
    flops = 4.0 * A * H * F
    return {"workload": name, "T": T, "H": H, "F": F, "E": E, "k": k, "A": A, "experts_hit": hit,
            "quantize_ms_once": round(t_quant, 3),
            "forward_ms": {"fp8": round(fwd8, 5), "bf16": round(fwd16, 5)},
            "tokens_per_s": {"fp8": round(T / (fwd8 * 1e-3), 1), "bf16": round(T / (fwd16 * 1e-3), 1)},
            "grouped_ffn_ms": {"fp8": round(ffn8, 5), "bf16": round(ffn16, 5)},
            "weight_bytes": {"fp8": w8, "bf16": w16},
            "weight_stream_gbs": {"fp8": round(w8 / (ffn8 * 1e-3) / 1e9, 1), "bf16": round(w16 / (ffn16 * 1e-3) / 1e9, 1)},
            "grouped_ffn_tflops": {"fp8": round(flops / (ffn8 * 1e-3) / 1e12, 1),
                                   "bf16": round(flops / (ffn16 * 1e-3) / 1e12, 1)}}


PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA


def mx_times(name, steps=20, reps=20):
    """MX fp8 experts (tokens and weights in OCP MX E4M3, products on the fp8 matrix cores) next to bf16 on one
    workload: the layer (moe_forward_mxfp8 against moe_forward, no shared expert) and the expert products
    (moe_grouped_ffn_mxfp8, which includes quantising the dispatched rows, against moe_grouped_ffn), HIP events;
    fp8 MFMA fraction against 5.0 PFLOP/s."""
    import torch

    import gen
    import top_routing_grouped_gemm_amd as moe

    dev = torch.device("cuda:0")
    I = gen.make_inputs(name)
    d = gen.to_device(I, dev)
    s = torch.cuda.current_stream()
    T, H, F, E, k = I.T, I.H, I.F, I.E, I.k
    lib = moe.load_library()
    W1q, W1s = moe.moe_quantize_mxfp8(d["W1"])
    W2q, W2s = moe.moe_quantize_mxfp8(d["W2"])
    t_quant = event_time_ms(lambda: (moe.moe_quantize_mxfp8(d["W1"], Wq=W1q, W_scale=W1s),
                                     moe.moe_quantize_mxfp8(d["W2"], Wq=W2q, W_scale=W2s)), 3, s)
    wsm = torch.empty(lib.moe_mxfp8_workspace_bytes(T, H, F, E, k), dtype=torch.uint8, device=dev)
    ws = torch.empty(moe.moe_workspace_bytes(T, H, F, E, k, 0, torch.bfloat16), dtype=torch.uint8, device=dev)
    y = torch.empty((T, H), dtype=torch.float32, device=dev)
    fwd_mx = event_time_ms(lambda: moe.moe_forward_mxfp8(d["x"], d["Wr"], d["bias"], W1q, W1s, W2q, W2s, F, k, I.drop,
                                                         y=y, ws=wsm), steps, s)
    fwd16 = event_time_ms(lambda: moe.moe_forward(d["x"], d["Wr"], d["bias"], d["W1"], d["W2"], k, I.drop, y=y,
                                                  ws=ws), steps, s)
    ids, w = moe.moe_route(d["x"], d["Wr"], d["bias"], k, I.drop)
    x_perm, off, row_token, inv = moe.moe_permute(d["x"], ids, w, E)
    xq, xs = moe.moe_quantize_mxfp8_rows(d["x"])
    t_rows = event_time_ms(lambda: moe.moe_quantize_mxfp8_rows(d["x"], xq=xq, x_scale=xs), reps, s)
    hq = torch.empty((F // 64, T * k, 64), dtype=torch.uint8, device=dev)
    hs = torch.empty((F // 128, T * k, 4), dtype=torch.uint8, device=dev)
    y_perm = torch.empty((T * k, H), dtype=torch.float32, device=dev)
    wsx = torch.empty(lib.moe_grouped_ffn_mxfp8_workspace_bytes(T, H, k), dtype=torch.uint8, device=dev)
    ffn_mx = event_time_ms(lambda: moe.moe_grouped_ffn_mxfp8(d["x"], row_token, off, W1q, W1s, W2q, W2s, F, k,
                                                             h_codes=hq, h_scale=hs, y_perm=y_perm, ws=wsx), reps, s)
    fws = torch.empty(moe.moe_ffn_workspace_bytes(T, F, E, k, 0, torch.bfloat16), dtype=torch.uint8, device=dev)
    ffn16 = event_time_ms(lambda: moe.moe_grouped_ffn(x_perm, off, d["W1"], d["W2"], T, k, y_perm=y_perm, ws=fws),
                          reps, s)
    torch.cuda.synchronize()
    A = int(off[-1].item())
    flops = 4.0 * A * H * F
    return {"workload": name, "T": T, "H": H, "F": F, "E": E, "k": k, "A": A,
            "quantize_weights_ms_once": round(t_quant, 3), "quantize_rows_ms": round(t_rows, 5),
            "forward_ms": {"mxfp8": round(fwd_mx, 5), "bf16": round(fwd16, 5)},
            "tokens_per_s": {"mxfp8": round(T / (fwd_mx * 1e-3), 1), "bf16": round(T / (fwd16 * 1e-3), 1)},
            "grouped_ffn_ms": {"mxfp8": round(ffn_mx, 5), "bf16": round(ffn16, 5)},
            "grouped_ffn_tflops": {"mxfp8": round(flops / (ffn_mx * 1e-3) / 1e12, 1),
                                   "bf16": round(flops / (ffn16 * 1e-3) / 1e12, 1)},
            "grouped_ffn_peak_frac": {"mxfp8_vs_fp8_peak": round(flops / (ffn_mx * 1e-3) / 1e12 / PEAK_FP8_TFLOPS, 4),
                                      "bf16_vs_bf16_peak": round(flops / (ffn16 * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}}


def cpu_baseline(I_name, min_seconds=10.0, max_reps=30):
    """The fp64 oracle, as it stands, on the host cores: whole prefill batches, repeated until about 10 s."""
    import numpy as np

    import gen
    import oracle

    try:
        from threadpoolctl import threadpool_info
        threads = max((p.get("num_threads", 1) for p in threadpool_info()), default=os.cpu_count())
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
    I = gen.make_inputs(I_name)
    x, Wr = I.f64(I.x), I.f64(I.Wr)
    W1, W2 = I.f64(I.W1()), I.f64(I.W2())
    reps, total, stage = 0, 0.0, {}
    while reps < max_reps and (total < min_seconds or reps == 0):
        t = time.perf_counter()
        r = oracle.forward(x, Wr, I.bias_f64(), W1, W2, I.k, I.drop)
        total += time.perf_counter() - t
        reps += 1
        for k_, v in r.times.items():
            stage[k_] = stage.get(k_, 0.0) + v
    return {"value": round(reps * I.T / total, 2), "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{reps} x the whole {I_name} batch (T={I.T} tokens), fp64 numpy/OpenBLAS, {total:.1f} s",
            "cpu": host_cpu_model(),
            "stages_s": {k_: round(v / reps, 3) for k_, v in stage.items()}}


def host_cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), or None where it is not readable."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def calibration():
    """Practical ceilings on this machine, measured with the library's calibration kernels: the bare bf16 MFMA loop
    with one and two waves per SIMD (256 workgroups of 4 / 8 waves) on one fixed operand pair, and with two waves
    per SIMD on pseudo-random operands (what a GEMM on real data can reach: the matrix cores switch more bits and
    run slower); a streaming read of 2 GiB; the grouped FFN's k-step on random bf16 operands with and without its
    feed; the vendor library's 8192^3 bf16 GEMM on normal random operands."""
    import torch

    import top_routing_grouped_gemm_amd as moe

    s = torch.cuda.current_stream()
    out = {}
    for waves, rnd in ((4, False), (8, False), (8, True)):
        iters = 4096
        sink = torch.empty(256 * waves * 64, dtype=torch.float32, device="cuda")
        flops = moe.moe_calibrate_mfma_bf16(256, waves, iters, sink, random_operands=rnd)
        ms = event_time_ms(lambda: moe.moe_calibrate_mfma_bf16(256, waves, iters, sink, random_operands=rnd), 5, s)
        key = f"mfma_32x32x16_bf16_{waves // 4}_wave_per_simd" + ("_random_operands" if rnd else "")
        out[key + "_tflops"] = round(flops / (ms * 1e-3) / 1e12, 1)
    buf = torch.empty(2 << 30, dtype=torch.uint8, device="cuda")
    for wg in (1024, 4096):
        sink = torch.empty(wg * 256, dtype=torch.float32, device="cuda")
        nbytes = moe.moe_calibrate_stream_read(buf, wg, sink)
        ms = event_time_ms(lambda: moe.moe_calibrate_stream_read(buf, wg, sink), 5, s)
        out[f"stream_read_{wg}_workgroups_gbs"] = round(nbytes / (ms * 1e-3) / 1e9, 1)
    del buf
    # the grouped FFN's 256x256 k-step alone, with its 32 KB-per-step direct-to-LDS feed from an L2-resident
    # 4 MiB span of normal random bf16, and that feed alone: the main loop's own ceiling with and without the feed
    # (mode 0 fills its LDS with pseudo-random bf16 itself)
    src = torch.randn(2 << 20, device="cuda").to(torch.bfloat16).view(torch.uint8)
    sink = torch.empty(256 * 512, dtype=torch.float32, device="cuda")
    steps = 512
    ks = {}
    for mode, key in ((0, "no_feed_tflops"), (1, "with_feed_tflops"), (2, "feed_only_tbs")):
        work = moe.moe_calibrate_gemm_kstep(mode, 256, steps, src=src, sink=sink)
        ms = event_time_ms(lambda: moe.moe_calibrate_gemm_kstep(mode, 256, steps, src=src, sink=sink), 5, s)
        ks[key] = round(work / (ms * 1e-3) / 1e12, 1)
    out["gemm_kstep_256x256"] = ks
    del src, sink
    # the vendor library on a large square bf16 GEMM: the chip's practical dense-GEMM rate, against which the
    # library's rate on this layer's shapes (roofline.library_dense_gemm) shows what the shapes themselves cost
    n = 8192
    sq = library_dense_gemm(n, n, n)
    out["library_square_gemm_8192_tflops"] = round(2.0 * n ** 3 / (sq * 1e-3) / 1e12, 1)
    out["note"] = ("bare-loop, streaming-read and GEMM k-step ceilings (library calibration kernels) and the vendor "
                   "library's 8192^3 bf16 GEMM; context for the fractions")
    return out


def ffn_only(name, reps):
    """Only the step-wise grouped FFN of one workload, `reps` times (for counter passes: one kernel pair per
    call and nothing else from the library in between)."""
    import torch

    import gen
    import top_routing_grouped_gemm_amd as moe

    dev = torch.device("cuda:0")
    I = gen.make_inputs(name)
    d = gen.to_device(I, dev)
    ids, w = moe.moe_route(d["x"], d["Wr"], d["bias"], I.k, I.drop)
    x_perm, off, row_token, inv = moe.moe_permute(d["x"], ids, w, I.E)
    y_perm = torch.empty((I.T * I.k, I.H), dtype=torch.float32, device=dev)
    fws = torch.empty(moe.moe_ffn_workspace_bytes(I.T, I.F, I.E, I.k, 0, d["x"].dtype), dtype=torch.uint8,
                      device=dev)
    torch.cuda.synchronize()
    for _ in range(reps):
        moe.moe_grouped_ffn(x_perm, off, d["W1"], d["W2"], I.T, I.k, y_perm=y_perm, ws=fws)
    torch.cuda.synchronize()
    print(json.dumps({"workload": name, "ffn_calls": reps}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--stage-reps", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--only", choices=["tiny", "decode", "prefill", "mixtral_shared", "skew"], default=None,
                    help="time one workload only (profiling runs and the per-workload table); prints its stage times")
    ap.add_argument("--ffn-only", type=int, default=0,
                    help="with --only: run only the step-wise grouped FFN this many times (counter passes)")
    ap.add_argument("--calibrate", action="store_true", help="print only the MFMA and streaming-read ceilings")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="run only a plain device-to-device copy of this many MiB (counter calibration)")
    ap.add_argument("--capacity-factor", type=float, default=0.0,
                    help="with --only: time capacity-limited routing (this factor) against plain routing")
    ap.add_argument("--padded", action="store_true",
                    help="with --only: time the padded fixed-shape layout against the ragged grouped FFN")
    ap.add_argument("--mx", action="store_true",
                    help="with --only: time MX fp8 experts (fp8 matrix cores) against bf16 (layer and grouped FFN)")
    ap.add_argument("--fp8", action="store_true",
                    help="with --only: time fp8 expert weights against bf16 (layer and grouped FFN)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this layer forward runs on a single MI355X; "
              "run it with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    import top_routing_grouped_gemm_amd as moe

    moe.load_library()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.copy_probe_mib:
        n = args.copy_probe_mib << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n}), flush=True)
        return
    if args.calibrate:
        print(json.dumps(calibration()), flush=True)
        return
    if args.only and args.ffn_only:
        ffn_only(args.only, args.ffn_only)
        return
    if args.only and args.padded:
        print(json.dumps(padded_times(args.only)), flush=True)
        return
    if args.only and args.mx:
        print(json.dumps(mx_times(args.only)), flush=True)
        return
    if args.only and args.fp8:
        print(json.dumps(fp8_times(args.only)), flush=True)
        return
    if args.only and args.capacity_factor > 0:
        print(json.dumps(capacity_times(args.only, args.capacity_factor)), flush=True)
        return
    if args.only:
        _, res = run_workload(args.only, args.steps, args.warmup, args.stage_reps)
        print(json.dumps({"workload": args.only, **res}), flush=True)
        return
    I, pre = run_workload("prefill", args.steps, args.warmup, args.stage_reps)
    line = {
        "metric": "MoE-layer tokens/s + grouped-GEMM % MFMA peak, E=128 top-8 prefill & decode",
        "value": round(pre["tokens_per_s"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(pre["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded Philox normals, random-init router and experts)",
        "config": {"workload": "prefill MoE layer T=8192 H=2048 F=768 E=128 top-8", "T": I.T, "H": I.H, "F": I.F,
                   "E": I.E, "k": I.k, "parallelism": "single GPU"},
        "roofline": {
            "kernel": "grouped_ffn (W1+SiLU launch and W2 launch)",
            "bound": "mfma",
            "achieved": round(pre["grouped_ffn_tflops"], 1),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(pre["grouped_ffn_tflops"] / PEAK_BF16_TFLOPS, 4),
            "traffic": measured_traffic("traffic_prefill_bytes"),
            "traffic_unit": "bytes per moe_grouped_ffn call (FETCH_SIZE x2 + WRITE_SIZE x1, copy-calibrated)",
            "algorithmic_bytes": pre["algorithmic_bytes"]["grouped_ffn"],
        },
        "prefill": pre,
    }
    up = library_dense_gemm(pre["A"], I.H, I.F)
    down = library_dense_gemm(pre["A"], I.F, I.H)
    line["roofline"]["library_dense_gemm"] = {
        "what": "torch.mm (hipBLASLt) bf16 dense GEMMs of the same FLOPs (A x H x F and A x F x H), no grouping",
        "ms": round(up + down, 4), "tflops": round(pre["grouped_ffn_flops"] / ((up + down) * 1e-3) / 1e12, 1),
        "frac": round(pre["grouped_ffn_flops"] / ((up + down) * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
    if not args.no_decode:
        Id, dec = run_workload("decode", max(args.steps, 50), args.warmup, max(args.stage_reps, 100), graph=True)
        wbytes = dec["experts_hit"] * 2 * Id.H * Id.F * Id.elem_bytes
        dec["weight_stream_gbs"] = round(wbytes / (dec["stages_ms"]["grouped_ffn"] * 1e-3) / 1e9, 1)
        dec["weight_stream_hbm_frac"] = round(dec["weight_stream_gbs"] / PEAK_HBM_GBS, 4)
        dec["grouped_ffn_traffic_bytes"] = measured_traffic("traffic_decode_bytes")
        line["decode"] = dec
        f8 = fp8_times("decode", max(args.steps, 50), max(args.stage_reps, 100))
        line["decode_fp8_experts"] = {k_: f8[k_] for k_ in ("forward_ms", "tokens_per_s", "grouped_ffn_ms",
                                                             "weight_bytes", "weight_stream_gbs")}
        mx = mx_times("decode", max(args.steps, 50), max(args.stage_reps, 100))
        line["decode_mxfp8_experts"] = {k_: mx[k_] for k_ in ("forward_ms", "tokens_per_s", "grouped_ffn_ms")}
    # the other full-size workloads: the Mixtral-like layer with its shared expert (MFMA-bound) and the skewed
    # layer (weight-stream bound)
    for name in ("mixtral_shared", "skew"):
        Iw, r = run_workload(name, max(5, args.steps // 4), 2, max(5, args.stage_reps // 2))
        wbytes = (r["experts_hit"] * 2 * Iw.H * Iw.F + 2 * Iw.H * Iw.Fs) * Iw.elem_bytes
        keep = ("T", "H", "F", "E", "k", "A", "experts_hit", "rows_per_expert", "ms_per_step", "tokens_per_s",
                "stages_ms", "stages_ms_mall_evicted", "stage_hbm_frac", "stage_hbm_frac_method_bytes",
                "grouped_ffn_tflops", "grouped_ffn_mfma_frac")
        line[name] = {k_: r[k_] for k_ in keep}
        line[name]["weight_stream_gbs"] = round(wbytes / (r["stages_ms"]["grouped_ffn"] * 1e-3) / 1e9, 1)
        line[name]["weight_stream_hbm_frac"] = round(line[name]["weight_stream_gbs"] / PEAK_HBM_GBS, 4)
        if Iw.Fs:
            line[name]["Fs"] = Iw.Fs
    line["calibration"] = cal = calibration()
    # the same launches against what this box's matrix cores sustain on real (high-entropy) operands: the bare
    # MFMA loop on pseudo-random operands, and the grouped FFN's own k-step fed from L2 on random bf16
    mr = cal["mfma_32x32x16_bf16_2_wave_per_simd_random_operands_tflops"]
    kf = cal["gemm_kstep_256x256"]["with_feed_tflops"]
    line["roofline"]["practical_ceilings"] = {
        "mfma_bf16_random_operands_tflops": mr, "kstep_fed_random_bf16_tflops": kf,
        "achieved_over_mfma_random": round(line["roofline"]["achieved"] / mr, 4),
        "achieved_over_kstep_fed": round(line["roofline"]["achieved"] / kf, 4),
        "note": "context only; frac stays against the published 2.5 PFLOP/s dense bf16 peak"}
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (fp64 oracle) ...")
        line["cpu_baseline"] = cpu_baseline("prefill")
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
