#!/usr/bin/env python3
"""Throughput of the QLoRA NF4 linear layer on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input:
NF4 quantization of the fp32 base weight (block absmax, nearest level, nibble
packing, 8-bit double quantization of the scales), the forward (on-chip
restore, base GEMM, fused rank-r term) and the backward (dX through the
transposed restore, dA, dB).  Inputs are resident in HBM before timing.

Default workload: attention-projection-shaped layer, W 4096 x 4096, 2048
tokens, r = 16, alpha = 32 (seeded N(0, 0.02) weights; no model is loaded).
Metric: fwd+bwd algorithmic TFLOP/s = (4 T K N + 6 T r (K + N)) per step /
step time; the quantization has no flops but its time is inside the step.

Prints ONE JSON line.  Extra fields: per-kernel times from the library's
hipEvent trace, the roofline of the dominant kernel, the oracle timed on the
host cores (cpu_baseline), and packed-weight GB/s of the few-token forward.
"""

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0       # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA

# HBM bytes per launch of the two large kernels on the attention-shaped step,
# from two rocprofv3 --pmc runs of this script (FETCH_SIZE, then WRITE_SIZE,
# KiB per dispatch, averaged over the dispatches of each kernel), scaled by
# what the same counters read for a plain 256 MiB fill and copy in the same
# runs (--copy-calibration 256): the copy's FETCH_SIZE reads 131090.9 KiB for
# 262144 KiB moved (scale 1.99973), the fill's WRITE_SIZE reads exactly
# 262144 KiB (scale 1).  Valid only for the kernel sources they were taken
# on (sha256 of the files below); reported as null once those change.
TRAFFIC_SOURCES = ("fused_gemm.hip", "fused.hpp", "restore.hpp", "common.hpp")
TRAFFIC = {
    "sha256": "fa541814e1aa5d9ef702c1df6eaf09ea4b58889738e205a5ea9722a9b7c99008",
    "fetch_scale": 262144.0 / 131090.9,
    "write_scale": 1.0,
    "fwd_gemm": {"fetch_kib": 36005.5, "write_kib": 16384.0},
    "dx_gemm": {"fetch_kib": 35835.9, "write_kib": 16384.0},
}


def traffic_bytes(kernel):
    """Measured HBM bytes per launch of `kernel`, or None if its sources changed."""
    import hashlib
    h = hashlib.sha256()
    for f in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, "nf4_bit_quantized_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    if h.hexdigest() != TRAFFIC["sha256"] or kernel not in TRAFFIC:
        return None
    t = TRAFFIC[kernel]
    return int(round((t["fetch_kib"] * TRAFFIC["fetch_scale"] + t["write_kib"] * TRAFFIC["write_scale"]) * 1024))


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true", help="skip the few-token packed-weight GB/s section")
    ap.add_argument("--mlp", action="store_true",
                    help="also time the MLP shapes of a 7B-class layer (fused products of other shapes; off by "
                         "default so that the kernel trace of the default run holds only the roofline shape)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="budget for the oracle timing")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="after the JSON line, fill then copy a buffer of this many MiB (known HBM bytes "
                         "for scaling the FETCH_SIZE / WRITE_SIZE counters)")
    return ap.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def bf16_dev(bits):
    import numpy as np
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def layer_flops(T, K, N, r):
    fwd = 2 * T * K * N + 2 * T * r * (K + N)
    bwd = 2 * T * K * N + 4 * T * r * (K + N)
    return fwd, bwd


def cpu_baseline(inp, lin, budget_s):
    """The oracle (numpy) on the same workload: quantize + dequant + fwd + bwd."""
    import numpy as np
    from threadpoolctl import threadpool_info
    from oracle import lora as olora
    from oracle import nf4 as onf4
    from oracle.bf16 import bits_to_float

    X, A, B, dY = (bits_to_float(inp[k]) for k in ("X", "A", "B", "dY"))
    times = []
    t_start = time.perf_counter()
    while True:
        t0 = time.perf_counter()
        Q = onf4.quantize(inp["W"])
        W_hat = onf4.dequantize(Q).astype(np.float64)
        olora.forward(W_hat, X, A, B, lin.alpha, lin.r)
        olora.backward(W_hat, X, A, B, dY, lin.alpha, lin.r)
        times.append(time.perf_counter() - t0)
        if time.perf_counter() - t_start > budget_s or len(times) >= 20:
            break
    fwd, bwd = layer_flops(lin.T, lin.d_in, lin.d_out, lin.r)
    per_step = sum(times) / len(times)
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    return {
        "value": round((fwd + bwd) / per_step / 1e12, 4),
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"the full {lin.name} step (quantize {lin.d_out}x{lin.d_in}, dequantize, float64 fwd+bwd "
                   f"at T={lin.T}, r={lin.r}), {len(times)} repetitions, {per_step:.3f} s each; "
                   f"host threads available {len(os.sched_getaffinity(0))}"),
    }


def decode_section(steps, warmup):
    """Packed-weight GB/s of the few-token forward (8192 <-> 28672, r=64),
    rotating 5 copies of each weight (> 512 MB) so the 256 MB MALL cannot hold them."""
    import numpy as np
    import torch
    import nf4_bit_quantized_amd as q
    import workloads

    out = {}
    copies = 5
    for T in (1, 4, 16):
        for lin in workloads.decode_70b(T):
            inp = workloads.layer_inputs(lin.d_out, lin.d_in, T, lin.r, lin.seed, with_dy=False)
            W = torch.from_numpy(inp["W"]).cuda()
            pk, cd, cs = q.qlora_quantize_nf4(W)
            del W
            reps = [(pk.clone(), cd.clone(), cs.clone()) for _ in range(copies)]
            X, A, B = (bf16_dev(inp[k]) for k in ("X", "A", "B"))
            Y = torch.empty((T, lin.d_out), dtype=torch.bfloat16, device="cuda")
            U = torch.empty((T, lin.r), dtype=torch.float32, device="cuda")
            ws = torch.empty(max(1, q.qlora_fwd_workspace_bytes(lin.d_out, lin.d_in, T, lin.r)),
                             dtype=torch.uint8, device="cuda")
            for i in range(warmup):
                p = reps[i % copies]
                q.qlora_linear_fwd(p[0], p[1], p[2], X, A, B, lin.alpha, Y=Y, U_out=U, workspace=ws)
            torch.cuda.synchronize()
            q.qlora_trace_read(reset=True)
            q.qlora_trace_select({"decode"})
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for i in range(steps):
                p = reps[i % copies]
                q.qlora_linear_fwd(p[0], p[1], p[2], X, A, B, lin.alpha, Y=Y, U_out=U, workspace=ws)
            e1.record()
            torch.cuda.synchronize()
            q.qlora_trace_enable(False)
            kt = q.qlora_trace_read(reset=True)
            call_ms = e0.elapsed_time(e1) / steps
            packed_bytes = pk.numel() + cd.numel() + cs.numel() * 4
            dec_n, dec_ms = kt.get("decode", (1, float("nan")))
            dec_avg = dec_ms / max(dec_n, 1)
            out[lin.name] = {
                "T": T, "d_out": lin.d_out, "d_in": lin.d_in,
                "packed_weight_bytes": packed_bytes,
                "call_us": round(call_ms * 1e3, 2),
                "packed_GBps_call": round(packed_bytes / (call_ms * 1e-3) / 1e9, 1),
                "decode_kernel_us": round(dec_avg * 1e3, 2),
                "packed_GBps_kernel": round(packed_bytes / (dec_avg * 1e-3) / 1e9, 1),
                "frac_hbm_kernel": round(packed_bytes / (dec_avg * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            }
            log("decode", lin.name, out[lin.name])
            del reps, pk, cd, cs
            torch.cuda.empty_cache()
    return out


def export_section(lin, steps):
    """HBM GB/s of the restored-weight export and of the merge, on the step's
    weight (rotating 8 copies of the packed weight and of the output, 336 MB,
    so the 256 MB MALL cannot hold them)."""
    import torch
    import nf4_bit_quantized_amd as q
    import workloads

    N, K, r = lin.d_out, lin.d_in, lin.r
    inp = workloads.layer_inputs(N, K, 1, r, lin.seed)
    W = torch.from_numpy(inp["W"]).cuda()
    pk, cd, cs = q.qlora_quantize_nf4(W)
    del W
    copies = 8
    reps = [(pk.clone(), cd.clone(), cs.clone()) for _ in range(copies)]
    outs = [torch.empty((N, K), dtype=torch.bfloat16, device="cuda") for _ in range(copies)]
    A, B = bf16_dev(inp["A"]), bf16_dev(inp["B"])
    weight_bytes = pk.numel() + cd.numel() + cs.numel() * 4
    out = {}
    for name, call, extra in (
            ("dequantize", lambda p, o: q.qlora_dequantize_nf4(p[0], p[1], p[2], W_hat=o), 0),
            ("merge", lambda p, o: q.qlora_merge_lora(p[0], p[1], p[2], A, B, lin.alpha, W_merged=o),
             A.numel() * 2 + B.numel() * 2)):
        for i in range(copies):
            call(reps[i], outs[i])
        torch.cuda.synchronize()
        q.qlora_trace_read(reset=True)
        q.qlora_trace_select({"export"})
        for i in range(steps):
            call(reps[i % copies], outs[i % copies])
        torch.cuda.synchronize()
        q.qlora_trace_enable(False)
        n, ms = q.qlora_trace_read(reset=True).get("export", (1, float("nan")))
        avg = ms / max(n, 1)
        nbytes = weight_bytes + N * K * 2 + extra
        out[name] = {"d_out": N, "d_in": K, "r": r if name == "merge" else 0, "bytes": nbytes,
                     "kernel_us": round(avg * 1e3, 2), "GBps": round(nbytes / (avg * 1e-3) / 1e9, 1),
                     "frac_hbm": round(nbytes / (avg * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}
        log("export", name, out[name])
    return out


def quantize16_section(lin, steps):
    """Quantization of the attention-shaped weight handed over as bf16 and as
    fp16 (2 bytes in per weight instead of 4), rotating 8 copies of the
    weight (268 MB) so the 256 MB MALL cannot hold them."""
    import torch
    import nf4_bit_quantized_amd as q
    import workloads

    N, K = lin.d_out, lin.d_in
    W = workloads.layer_inputs(N, K, 1, 1, lin.seed, with_dy=False)["W"]
    copies = 8
    out = {}
    for name, dt in (("bf16", torch.bfloat16), ("fp16", torch.float16)):
        w16 = torch.from_numpy(W).cuda().to(dt)
        reps = [w16.clone() for _ in range(copies)]
        del w16
        bufs = [q.qlora_quantize_nf4(reps[i]) for i in range(copies)]
        torch.cuda.synchronize()
        q.qlora_trace_read(reset=True)
        q.qlora_trace_select({"nf4_quantize"})
        for i in range(steps):
            q.qlora_quantize_nf4(reps[i % copies], *bufs[i % copies])
        torch.cuda.synchronize()
        q.qlora_trace_enable(False)
        n, ms = q.qlora_trace_read(reset=True).get("nf4_quantize", (1, float("nan")))
        avg = ms / max(n, 1)
        pk, cd, cs = bufs[0]
        nbytes = N * K * 2 + pk.numel() + cd.numel() + cs.numel() * 4
        out[name] = {"d_out": N, "d_in": K, "bytes": nbytes, "kernel_us": round(avg * 1e3, 2),
                     "GBps": round(nbytes / (avg * 1e-3) / 1e9, 1),
                     "frac_hbm": round(nbytes / (avg * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}
        log("quantize16", name, out[name])
        del reps, bufs
    return out


def dropout_section(lin, steps):
    """The attention-shaped step with LoRA dropout on the adapter input at the
    pages' rate (p = 0.05, seeded keep mask), beside the same step without it:
    step time, and the two dropout kernels' own time."""
    import torch
    import nf4_bit_quantized_amd as q
    import workloads

    N, K, T, r, alpha, p = lin.d_out, lin.d_in, lin.T, lin.r, lin.alpha, 0.05
    inp = workloads.layer_inputs(N, K, T, r, lin.seed)
    X, A, B, dY = (bf16_dev(inp[k]) for k in ("X", "A", "B", "dY"))
    keep = torch.from_numpy(workloads.dropout_keep_bits(T, K, p, lin.seed)).cuda()
    packed, codes, consts = q.qlora_quantize_nf4(torch.from_numpy(inp["W"]).cuda())
    Y = torch.empty((T, N), dtype=torch.bfloat16, device="cuda")
    U = torch.empty((T, r), dtype=torch.float32, device="cuda")
    dX = torch.empty((T, K), dtype=torch.bfloat16, device="cuda")
    dA = torch.empty((r, K), dtype=torch.float32, device="cuda")
    dB = torch.empty((N, r), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(q.qlora_bwd_workspace_bytes(N, K, T, r), q.qlora_fwd_workspace_bytes(N, K, T, r))
                     + T * K * 2 + 256, dtype=torch.uint8, device="cuda")
    out = {"p": p}
    for name, kw in (("plain", {}), ("dropout", {"keep": keep, "p": p})):
        def step():
            q.qlora_linear_fwd(packed, codes, consts, X, A, B, alpha, Y=Y, U_out=U, workspace=ws, **kw)
            q.qlora_linear_bwd(packed, codes, consts, X, A, B, alpha, dY, U_in=U, dX=dX, dA=dA, dB=dB, workspace=ws,
                               **kw)
        for _ in range(3):
            step()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            step()
        e1.record()
        torch.cuda.synchronize()
        out[name + "_fwd_bwd_ms"] = round(e0.elapsed_time(e1) / steps, 4)
    q.qlora_trace_read(reset=True)
    q.qlora_trace_select({"dropout"})
    for _ in range(steps):
        q.qlora_linear_bwd(packed, codes, consts, X, A, B, alpha, dY, U_in=U, dX=dX, dA=dA, dB=dB, workspace=ws,
                           keep=keep, p=p)
    torch.cuda.synchronize()
    q.qlora_trace_enable(False)
    n, ms = q.qlora_trace_read(reset=True).get("dropout", (1, float("nan")))
    out["dropout_kernels_us_per_bwd"] = round(ms / max(n, 1) * 2 * 1e3, 2)   # two launches per backward
    log("dropout", out)
    return out


def mlp_section(steps):
    """The MLP set of a 7B-class layer: gate and up 4096->11008, down
    11008->4096, 4096 tokens, r = 64, alpha = 16.  Per step: quantize of the
    three weights, then fwd + bwd of each linear (inputs resident)."""
    import torch
    import nf4_bit_quantized_amd as q
    import workloads

    lins = workloads.mlp_llama7b()
    st = []
    for lin in lins:
        N, K, T, r = lin.d_out, lin.d_in, lin.T, lin.r
        inp = workloads.layer_inputs(N, K, T, r, lin.seed)
        W = torch.from_numpy(inp["W"]).cuda()
        X, A, B, dY = (bf16_dev(inp[k]) for k in ("X", "A", "B", "dY"))
        pk, cd, cs = q.qlora_quantize_nf4(W)
        st.append(dict(lin=lin, W=W, X=X, A=A, B=B, dY=dY, pk=pk, cd=cd, cs=cs,
                       Y=torch.empty((T, N), dtype=torch.bfloat16, device="cuda"),
                       U=torch.empty((T, r), dtype=torch.float32, device="cuda"),
                       dX=torch.empty((T, K), dtype=torch.bfloat16, device="cuda"),
                       dA=torch.empty((r, K), dtype=torch.float32, device="cuda"),
                       dB=torch.empty((N, r), dtype=torch.float32, device="cuda"),
                       ws=torch.empty(max(q.qlora_bwd_workspace_bytes(N, K, T, r),
                                          q.qlora_fwd_workspace_bytes(N, K, T, r), 1),
                                      dtype=torch.uint8, device="cuda")))

    def run(quant, fwdbwd):
        for e in st:
            l = e["lin"]
            if quant:
                q.qlora_quantize_nf4(e["W"], e["pk"], e["cd"], e["cs"])
            if fwdbwd:
                q.qlora_linear_fwd(e["pk"], e["cd"], e["cs"], e["X"], e["A"], e["B"], l.alpha, Y=e["Y"], U_out=e["U"],
                                   workspace=e["ws"])
                q.qlora_linear_bwd(e["pk"], e["cd"], e["cs"], e["X"], e["A"], e["B"], l.alpha, e["dY"], U_in=e["U"],
                                   dX=e["dX"], dA=e["dA"], dB=e["dB"], workspace=e["ws"])

    out = {}
    flops = sum(sum(layer_flops(e["lin"].T, e["lin"].d_in, e["lin"].d_out, e["lin"].r)) for e in st)
    for name, quant, fb in (("fwd_bwd", False, True), ("quantize", True, False)):
        for _ in range(2):
            run(quant, fb)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            run(quant, fb)
        e1.record()
        torch.cuda.synchronize()
        out[name + "_ms"] = round(e0.elapsed_time(e1) / steps, 4)
    out["fwd_bwd_tflops"] = round(flops / (out["fwd_bwd_ms"] * 1e-3) / 1e12, 1)
    out["fwd_bwd_frac_mfma"] = round(out["fwd_bwd_tflops"] / BF16_PEAK_TFLOPS, 4)
    qbytes = sum(e["lin"].d_out * e["lin"].d_in * (4 + 0.5) + e["cd"].numel() + e["cs"].numel() * 4 for e in st)
    out["quantize_GBps"] = round(qbytes / (out["quantize_ms"] * 1e-3) / 1e9, 1)
    out["quantize_frac_hbm"] = round(out["quantize_GBps"] / HBM_PEAK_GBPS, 4)
    out["config"] = "gate/up 4096->11008, down 11008->4096, 4096 tokens, r=64, alpha=16"
    log("mlp", out)
    del st
    return out


def multi_proj_section(steps):
    """Query, key and value projections of a 70B-class layer with grouped
    queries (8192x8192, 1024x8192, 1024x8192; r = 64, alpha = 16) at 1 and 16
    tokens: one forward call over the three weights against three separate
    calls, with the weights rotated over 4 copies (173 MB of packed weight) and the outputs and
    workspace allocated once.  call_us includes the host's enqueue of each call;
    kernel_us is the weight-streaming kernels alone."""
    import torch
    import nf4_bit_quantized_amd as q

    K, r, alpha = 8192, 64, 16.0
    g = torch.Generator(device="cuda").manual_seed(0)
    sets = []
    for _ in range(4):
        layers = []
        for N in (8192, 1024, 1024):
            pk, cd, cs = q.qlora_quantize_nf4(torch.randn(N, K, device="cuda", generator=g) * 0.02)
            A = (torch.randn(r, K, device="cuda", generator=g) / r).to(torch.bfloat16)
            B = (torch.randn(N, r, device="cuda", generator=g) * 0.01).to(torch.bfloat16)
            layers.append((pk, cd, cs, A, B))
        sets.append(layers)
    packed_bytes = sum(l[0].numel() + l[1].numel() + l[2].numel() * 4 for l in sets[0])
    out = {"weights": "8192x8192 + 2 x 1024x8192", "packed_bytes": packed_bytes}
    for T in (1, 16):
        X = torch.randn(T, K, device="cuda", generator=g).to(torch.bfloat16)
        # outputs and workspace allocated once, as a serving loop holds them
        outs = [(torch.empty((T, N), dtype=torch.bfloat16, device="cuda"),
                 torch.empty((T, r), dtype=torch.float32, device="cuda")) for N in (8192, 1024, 1024)]
        n_b = ctypes.c_size_t()
        descs = (q.Nf4Desc * 3)(*[q._stored_desc(*l[:3], q.TABLE_NF4) for l in sets[0]])
        q._check(q.lib().qlora_multi_fwd_workspace_bytes(3, descs, T, r, ctypes.byref(n_b)), "workspace")
        ws_bytes = max([n_b.value] + [q.qlora_fwd_workspace_bytes(N, K, T, r) for N in (8192, 1024)])
        ws = torch.empty(max(1, ws_bytes), dtype=torch.uint8, device="cuda")
        calls = {"fused": lambda L: q.qlora_linear_fwd_multi(L, X, alpha, workspace=ws, outs=outs),
                 "separate": lambda L: [q.qlora_linear_fwd(*l[:3], X, l[3], l[4], alpha, Y=o[0], U_out=o[1],
                                                           workspace=ws) for l, o in zip(L, outs)]}
        for name, fn in calls.items():
            for i in range(8):
                fn(sets[i % 4])
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for i in range(steps):
                fn(sets[i % 4])
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) / steps * 1e3
            out[f"{name}_T{T}_call_us"] = round(us, 2)
            # the weight-streaming kernels alone (one launch fused, three separate)
            q.qlora_trace_read(reset=True)
            q.qlora_trace_select({"decode"})
            for i in range(steps):
                fn(sets[i % 4])
            torch.cuda.synchronize()
            q.qlora_trace_enable(False)
            n, ms = q.qlora_trace_read(reset=True).get("decode", (1, float("nan")))
            kus = ms / steps * 1e3
            out[f"{name}_T{T}_kernel_us"] = round(kus, 2)
            out[f"{name}_T{T}_kernel_GBps"] = round(packed_bytes / (kus * 1e-6) / 1e9, 1)
    log("multi_proj", out)
    del sets
    return out


def adamw_section(steps):
    """The AdamW update over every adapter of the 65B-class stack (8 layers x
    q, k, v, o 8192x8192, gate/up 8192->22016, down 22016->8192, r = 64) laid
    out in one fp32 arena: about 80M parameters, 30 bytes each per step."""
    import torch
    import nf4_bit_quantized_amd as q
    import workloads

    n = sum(l.r * (l.d_in + l.d_out) for l in workloads.stack_65b())
    g = torch.Generator(device="cuda").manual_seed(0)
    P = torch.randn(n, device="cuda", generator=g) * 0.02
    G = torch.randn(n, device="cuda", generator=g) * 1e-3
    M = torch.zeros(n, device="cuda")
    V = torch.zeros(n, device="cuda")
    P16 = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    for t in range(1, 4):
        q.qlora_adamw_step(P, G, M, V, t, 1e-4, weight_decay=0.01, param_bf16=P16)
    torch.cuda.synchronize()
    q.qlora_trace_read(reset=True)
    q.qlora_trace_select({"adamw"})
    for t in range(4, 4 + steps):
        q.qlora_adamw_step(P, G, M, V, t, 1e-4, weight_decay=0.01, param_bf16=P16)
    torch.cuda.synchronize()
    q.qlora_trace_enable(False)
    k, ms = q.qlora_trace_read(reset=True).get("adamw", (1, float("nan")))
    avg = ms / max(k, 1)
    nbytes = 30 * n
    out = {"params": n, "bytes": nbytes, "kernel_us": round(avg * 1e3, 2),
           "GBps": round(nbytes / (avg * 1e-3) / 1e9, 1),
           "frac_hbm": round(nbytes / (avg * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}
    log("adamw", out)
    del P, G, M, V, P16
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(sharding the layer over several GPUs is not part of this library).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import nf4_bit_quantized_amd as q
    import workloads

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    (lin,) = workloads.attn_4096()
    T, K, N, r, alpha = lin.T, lin.d_in, lin.d_out, lin.r, lin.alpha
    log(f"workload {lin}")
    inp = workloads.layer_inputs(N, K, T, r, lin.seed)

    W = torch.from_numpy(inp["W"]).cuda()
    X, A, B, dY = (bf16_dev(inp[k]) for k in ("X", "A", "B", "dY"))
    n_p, n_c, n_k = q.qlora_nf4_sizes(N, K)
    packed = torch.empty((N, K // 2), dtype=torch.uint8, device="cuda")
    codes = torch.empty(n_c, dtype=torch.uint8, device="cuda")
    consts = torch.empty(n_k // 4, dtype=torch.float32, device="cuda")
    Y = torch.empty((T, N), dtype=torch.bfloat16, device="cuda")
    U = torch.empty((T, r), dtype=torch.float32, device="cuda")
    dX = torch.empty((T, K), dtype=torch.bfloat16, device="cuda")
    dA = torch.empty((r, K), dtype=torch.float32, device="cuda")
    dB = torch.empty((N, r), dtype=torch.float32, device="cuda")
    wsf = torch.empty(max(1, q.qlora_fwd_workspace_bytes(N, K, T, r)), dtype=torch.uint8, device="cuda")
    wsb = torch.empty(max(1, q.qlora_bwd_workspace_bytes(N, K, T, r)), dtype=torch.uint8, device="cuda")

    def step():
        q.qlora_quantize_nf4(W, packed, codes, consts)
        q.qlora_linear_fwd(packed, codes, consts, X, A, B, alpha, Y=Y, U_out=U, workspace=wsf)
        q.qlora_linear_bwd(packed, codes, consts, X, A, B, alpha, dY, U_in=U, dX=dX, dA=dA, dB=dB, workspace=wsb)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: exactly K steps; the library brackets the two large kernels
    # (forward and dX products) with hipEvents on the launch stream
    q.qlora_trace_read(reset=True)
    q.qlora_trace_select({"fwd_gemm", "dx_gemm"})
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    q.qlora_trace_enable(False)
    ms_per_step = e0.elapsed_time(e1) / args.steps
    kt = q.qlora_trace_read(reset=True)

    # per-kernel breakdown: a second, untimed pass of K steps with every launch bracketed
    q.qlora_trace_enable(True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    q.qlora_trace_enable(False)
    kt_all = q.qlora_trace_read(reset=True)

    fwd_f, bwd_f = layer_flops(T, K, N, r)
    value = (fwd_f + bwd_f) / (ms_per_step * 1e-3) / 1e12

    kernels = {name: {"launches": n, "avg_us": round(ms / n * 1e3, 2), "share": None}
               for name, (n, ms) in kt_all.items()}
    total_k = sum(ms for (_, ms) in kt_all.values())
    for name, (n, ms) in kt_all.items():
        kernels[name]["share"] = round(ms / total_k, 4) if total_k > 0 else None
    # algorithmic work per launch of the two big kernels
    kernel_flops = {"fwd_gemm": 2 * T * K * N + 2 * T * r * N, "dx_gemm": 2 * T * N * K + 2 * T * r * K}
    dom = max(kernel_flops, key=lambda k: kt.get(k, (1, 0.0))[1])
    dn, dms = kt.get(dom, (1, float("nan")))
    dom_avg_s = dms / dn * 1e-3
    achieved = kernel_flops[dom] / dom_avg_s / 1e12
    roofline = {"kernel": dom, "bound": "mfma", "achieved": round(achieved, 2), "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / BF16_PEAK_TFLOPS, 4), "traffic": traffic_bytes(dom),
                "avg_launch_us": round(dom_avg_s * 1e6, 2), "flops_per_launch": kernel_flops[dom]}
    qn, qms = kt_all.get("nf4_quantize", (1, float("nan")))
    q_bytes = N * K * 4 + N * K // 2 + n_c + n_k
    quant = {"avg_us": round(qms / qn * 1e3, 2), "bytes": q_bytes,
             "GBps": round(q_bytes / (qms / qn * 1e-3) / 1e9, 1),
             "frac_hbm": round(q_bytes / (qms / qn * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}

    result = {
        "metric": "QLoRA linear fwd+bwd TFLOP/s & packed-weight GB/s; % of MI355X roofline",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded PCG64: W ~ N(0, 0.02) fp32, X, dY ~ N(0, 1) bf16, A ~ N(0, 1/r), B ~ N(0, 0.01))",
        "config": {"workload": "attention-projection QLoRA linear: W 4096x4096 NF4 (block 64, 8-bit scale "
                               "codes per 256 blocks), 2048 tokens, r=16, alpha=32; step = quantize + fwd + bwd",
                   "d_out": N, "d_in": K, "tokens": T, "r": r, "alpha": alpha},
        "roofline": roofline,
        "kernels": kernels,
        "kernels_note": "avg_us from a second pass of the same steps with every launch bracketed by hipEvents "
                        "(bracketing all ~14 launches slows a step by about a quarter); the roofline kernel "
                        "is timed inside the timed region itself, where only it is bracketed",
        "quantize": quant,
        "step_flops": fwd_f + bwd_f,
    }
    if not args.no_decode:
        result["decode_packed_weight"] = decode_section(steps=max(20, args.steps), warmup=5)
        result["export_bf16"] = export_section(lin, steps=max(20, args.steps))
        result["quantize_16bit_weight"] = quantize16_section(lin, steps=max(20, args.steps))
        result["adamw_65b_adapters"] = adamw_section(steps=max(20, args.steps))
        result["lora_dropout_attn4096"] = dropout_section(lin, steps=max(20, args.steps))
        result["qkv_gqa_70b"] = multi_proj_section(steps=max(20, args.steps))
    if args.mlp:
        result["mlp_llama7b"] = mlp_section(steps=10)
    if not args.no_cpu_baseline:
        log("timing the oracle on the host ...")
        result["cpu_baseline"] = cpu_baseline(inp, lin, args.cpu_seconds)
    print(json.dumps(result), flush=True)
    if args.copy_calibration > 0:
        nbytes = args.copy_calibration << 20
        src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        src.fill_(1)      # writes nbytes, reads none
        dst.copy_(src)    # reads nbytes, writes nbytes
        torch.cuda.synchronize()
        log(f"copy calibration: fill + copy of {nbytes} bytes")


if __name__ == "__main__":
    main()
