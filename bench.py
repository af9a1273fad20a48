#!/usr/bin/env python3
"""Throughput of the QLoRA NF4 linear layer on one MI355X.

Headline workload: the share of a 65B-class model that one GPU trains, 8
layers, each with the query, key, value and output projections (8192 x 8192)
and the gate, up (8192 -> 22016) and down (22016 -> 8192) projections, every
base weight blockwise NF4 (64-weight blocks, 8-bit scale codes per 256
blocks), 4096 tokens, rank 64, alpha 16.  One step = the forward and the
backward (dX, dA, dB; no gradient for the frozen weight) of all 56 linears,
with the inputs already resident in HBM: per layer, one call for the three
projections that share the attention input and one for the two that share
the MLP input, the backward in reverse layer order.  The weights are
quantized once, before timing (their quantization is reported on its own).

Metric: algorithmic TFLOP/s = sum over the linears of 4 T K N + 6 T r (K + N)
per step / step time (no flops are counted for the restore or for the dW
product that is never formed).

Prints ONE JSON line.  Extra fields: the roofline of the dominant kernel
(timed with hipEvents attached to its own dispatches inside the timed
region), a per-kernel table from a second pass, the other workloads (the
attention-shaped layer, the MLP set of a 7B-class layer, the few-token
forward's packed-weight GB/s, exports, optimizer, dropout, the fused products
against restoring each weight to bf16 once and multiplying with the ROCm BLAS
library), and the oracle timed on the host cores (cpu_baseline,
cpu_baselines).
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

# HBM bytes per launch of the dominant kernel on the headline step, from two
# rocprofv3 --pmc runs of this script (FETCH_SIZE, then WRITE_SIZE, KiB per
# dispatch, averaged over that kernel's dispatches), scaled by what the same
# counters read for a plain device-to-device copy of known size in the same
# runs (--copy-calibration).  Valid only for the kernel sources they were taken on
# (sha256 of the files below); reported as null once those change.
TRAFFIC_SOURCES = ("fused_gemm.hip", "fused_wide.hip", "fused_dx_wide.hip", "fused.hpp", "restore.hpp", "common.hpp")
TRAFFIC = {
    "sha256": "6812984a85af55c939c99dcfb7a2574d245f4a5fe691ccf8f856102a1ba2c4b9",
    # a 256 MiB device-to-device copy read 131084.5 KiB of FETCH_SIZE and wrote
    # 262144 KiB of WRITE_SIZE in the same runs
    "fetch_scale": 262144.0 / 131084.5,
    "write_scale": 1.0,
    # per dispatch, averaged over one 65B-class layer's launches (3 steps; dX:
    # five per layer, down's dX being two)
    "dx_gemm": {"fetch_kib": 538340.8, "write_kib": 74547.2},
    "fwd_gemm": {"fetch_kib": 705016.6, "write_kib": 211152.0},
}


def traffic_bytes(kernel):
    """Measured HBM bytes per launch of `kernel`, or None if its sources changed."""
    import hashlib
    h = hashlib.sha256()
    for f in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, "nf4_bit_quantized_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    if TRAFFIC["sha256"] is None or h.hexdigest() != TRAFFIC["sha256"] or kernel not in TRAFFIC:
        return None
    t = TRAFFIC[kernel]
    return int(round((t["fetch_kib"] * TRAFFIC["fetch_scale"] + t["write_kib"] * TRAFFIC["write_scale"]) * 1024))


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--layers", type=int, default=8, help="layers of the 65B-class stack (8 = the full share)")
    ap.add_argument("--headline-only", action="store_true", help="skip the other workloads' sections")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-full", action="store_true",
                    help="time the oracle on every workload's plan (minutes of host time), not the bounded set")
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


def fused_flops(T, K, N, r):
    """Algorithmic flops of the two fused products of one linear: the forward
    (X W_hat^T plus the rank-r term U B^T) and dX (dY W_hat plus G A)."""
    return 2 * T * K * N + 2 * T * r * N, 2 * T * N * K + 2 * T * r * K


# ---------------------------------------------------------------------------
# Headline: the 65B-class layer stack share
# ---------------------------------------------------------------------------

def stack_section(args):
    """Forward + backward of the 65B-class stack share at 4096 tokens.

    Synthetic inputs with the recipe's distributions (W ~ N(0, 0.02) fp32,
    X and dY ~ N(0, 1), A ~ N(0, 1/r), B ~ N(0, 0.01), bf16 rounded to
    nearest even), drawn on the GPU by torch's seeded generator (seed
    100 * layer + projection), since drawing 6.5e9 weights on the host would
    take minutes.  Each weight is quantized by the library, then its fp32
    copy is freed."""
    import torch
    import nf4_bit_quantized_amd as q
    import workloads

    lins = workloads.stack_65b(args.layers)
    T, r, alpha = lins[0].T, lins[0].r, lins[0].alpha
    dev = "cuda"
    gen = torch.Generator(device=dev)
    torch.cuda.reset_peak_memory_stats()
    qe0, qe1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    quant_ms = 0.0
    quant_bytes = 0
    layers = []
    for li in range(args.layers):
        projs = {}
        for lin in lins[li * 7:(li + 1) * 7]:
            name = lin.name.split(".")[1]
            gen.manual_seed(lin.seed)
            W = torch.randn(lin.d_out, lin.d_in, generator=gen, device=dev) * 0.02
            pk, cd, cs = q.qlora_quantize_nf4(W)            # allocation + first touch (untimed)
            torch.cuda.synchronize()
            qe0.record()
            q.qlora_quantize_nf4(W, pk, cd, cs)
            qe1.record()
            torch.cuda.synchronize()
            quant_ms += qe0.elapsed_time(qe1)
            quant_bytes += W.numel() * 4 + pk.numel() + cd.numel() + cs.numel() * 4
            del W
            A = (torch.randn(r, lin.d_in, generator=gen, device=dev) / r).to(torch.bfloat16)
            B = (torch.randn(lin.d_out, r, generator=gen, device=dev) * 0.01).to(torch.bfloat16)
            dY = torch.randn(T, lin.d_out, generator=gen, device=dev).to(torch.bfloat16)
            projs[name] = dict(lin=lin, w=(pk, cd, cs, A, B), dY=dY,
                               Y=torch.empty((T, lin.d_out), dtype=torch.bfloat16, device=dev),
                               U=torch.empty((T, r), dtype=torch.float32, device=dev),
                               dA=torch.empty((r, lin.d_in), dtype=torch.float32, device=dev),
                               dB=torch.empty((lin.d_out, r), dtype=torch.float32, device=dev))
        gen.manual_seed(100 * li + 99)
        groups = []
        for names, d_in in ((("q", "k", "v"), 8192), (("o",), 8192), (("gate", "up"), 8192), (("down",), 22016)):
            groups.append(dict(names=names,
                               X=torch.randn(T, d_in, generator=gen, device=dev).to(torch.bfloat16),
                               dX=torch.empty((T, d_in), dtype=torch.bfloat16, device=dev)))
        layers.append((projs, groups))

    shapes = [(8192, 8192)] * 3 + [(22016, 8192)] * 2 + [(8192, 22016)]
    ws_bytes = max(q.qlora_multi_fwd_workspace_bytes([(8192, 8192)] * 3, T, r),
                   q.qlora_multi_bwd_workspace_bytes([(8192, 8192)] * 3, T, r),
                   q.qlora_multi_fwd_workspace_bytes([(22016, 8192)] * 2, T, r),
                   q.qlora_multi_bwd_workspace_bytes([(22016, 8192)] * 2, T, r),
                   *[q.qlora_fwd_workspace_bytes(o, i, T, r) for o, i in shapes],
                   *[q.qlora_bwd_workspace_bytes(o, i, T, r) for o, i in shapes])
    ws = torch.empty(max(1, ws_bytes), dtype=torch.uint8, device=dev)

    def fwd_group(projs, g):
        P = [projs[n] for n in g["names"]]
        if len(P) == 1:
            p = P[0]
            q.qlora_linear_fwd(*p["w"][:3], g["X"], p["w"][3], p["w"][4], alpha, Y=p["Y"], U_out=p["U"],
                               workspace=ws)
        else:
            q.qlora_linear_fwd_multi([p["w"] for p in P], g["X"], alpha, workspace=ws,
                                     outs=[(p["Y"], p["U"]) for p in P])

    def bwd_group(projs, g):
        P = [projs[n] for n in g["names"]]
        if len(P) == 1:
            p = P[0]
            q.qlora_linear_bwd(*p["w"][:3], g["X"], p["w"][3], p["w"][4], alpha, p["dY"], U_in=p["U"], dX=g["dX"],
                               dA=p["dA"], dB=p["dB"], workspace=ws)
        else:
            q.qlora_linear_bwd_multi([p["w"] for p in P], g["X"], alpha, [p["dY"] for p in P],
                                     U_ins=[p["U"] for p in P], workspace=ws, dX=g["dX"],
                                     grads=[(p["dA"], p["dB"]) for p in P])

    def step():
        for projs, groups in layers:
            for g in groups:
                fwd_group(projs, g)
        for projs, groups in reversed(layers):
            for g in reversed(groups):
                bwd_group(projs, g)

    step_flops = sum(sum(layer_flops(l.T, l.d_in, l.d_out, l.r)) for l in lins)
    kflops = {"fwd_gemm": 0, "dx_gemm": 0}
    for l in lins:
        f, d = fused_flops(l.T, l.d_in, l.d_out, l.r)
        kflops["fwd_gemm"] += f
        kflops["dx_gemm"] += d

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # timed region: exactly `steps` steps; the library attaches hipEvents to
    # the dispatches of the two fused products (on the launch stream)
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
    log(f"stack: {ms_per_step:.3f} ms per step")

    # per-kernel breakdown: a second, untimed pass with every launch bracketed
    kpass = 2
    q.qlora_trace_enable(True)
    for _ in range(kpass):
        step()
    torch.cuda.synchronize()
    q.qlora_trace_enable(False)
    kt_all = q.qlora_trace_read(reset=True)
    total_k = sum(ms for (_, ms) in kt_all.values())
    kernels = {name: {"launches_per_step": n / kpass, "avg_us": round(ms / n * 1e3, 2),
                      "ms_per_step": round(ms / kpass, 3), "share": round(ms / total_k, 4) if total_k else None}
               for name, (n, ms) in kt_all.items()}

    fused = {}
    for k in ("fwd_gemm", "dx_gemm"):
        n, ms = kt.get(k, (0, float("nan")))
        if n == 0:
            continue
        flops = kflops[k] * args.steps
        fused[k] = {"launches": n, "avg_launch_us": round(ms / n * 1e3, 2),
                    "flops_per_launch": flops // n,
                    "achieved_tflops": round(flops / (ms * 1e-3) / 1e12, 2),
                    "frac": round(flops / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)}
    dom = max(fused, key=lambda k: kt[k][1])
    d = fused[dom]
    roofline = {"kernel": dom, "bound": "mfma", "achieved": d["achieved_tflops"], "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": d["frac"], "traffic": traffic_bytes(dom),
                "avg_launch_us": d["avg_launch_us"], "flops_per_launch": d["flops_per_launch"],
                "launch_note": "flops_per_launch and avg_launch_us average over the kernel's launches in the "
                               "timed region (per layer: one product over the query/key/value weights, "
                               "the output projection, one over gate/up, down); achieved = their flops / "
                               "their time"}
    value = step_flops / (ms_per_step * 1e-3) / 1e12
    out = {
        "ms_per_step": ms_per_step, "value": value, "step_flops": step_flops, "roofline": roofline,
        "fused_products": fused, "kernels": kernels,
        "kernels_note": f"from a second pass of {kpass} steps with every launch bracketed by hipEvents",
        "quantize_stack": {"weights": sum(l.d_out * l.d_in for l in lins), "bytes": quant_bytes,
                           "ms": round(quant_ms, 3),
                           "GBps": round(quant_bytes / (quant_ms * 1e-3) / 1e9, 1),
                           "frac_hbm": round(quant_bytes / (quant_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                           "note": "each weight quantized once from fp32, outside the timed step"},
        "peak_hbm_allocated_bytes": torch.cuda.max_memory_allocated(),
        "packed_weight_bytes": sum(p["w"][0].numel() + p["w"][1].numel() + p["w"][2].numel() * 4
                                   for projs, _ in layers for p in projs.values()),
        "T": T, "r": r, "alpha": alpha, "layers": args.layers,
    }
    del layers, ws
    torch.cuda.empty_cache()
    return out


# ---------------------------------------------------------------------------
# The attention-shaped layer (W 4096 x 4096, 2048 tokens, r = 16)
# ---------------------------------------------------------------------------

def attn_section(lin, steps):
    """fwd + bwd of the attention-shaped layer (quantization outside the step,
    reported beside it)."""
    import torch
    import nf4_bit_quantized_amd as q
    import workloads

    T, K, N, r, alpha = lin.T, lin.d_in, lin.d_out, lin.r, lin.alpha
    inp = workloads.layer_inputs(N, K, T, r, lin.seed)
    W = torch.from_numpy(inp["W"]).cuda()
    X, A, B, dY = (bf16_dev(inp[k]) for k in ("X", "A", "B", "dY"))
    packed, codes, consts = q.qlora_quantize_nf4(W)
    Y = torch.empty((T, N), dtype=torch.bfloat16, device="cuda")
    U = torch.empty((T, r), dtype=torch.float32, device="cuda")
    dX = torch.empty((T, K), dtype=torch.bfloat16, device="cuda")
    dA = torch.empty((r, K), dtype=torch.float32, device="cuda")
    dB = torch.empty((N, r), dtype=torch.float32, device="cuda")
    wsf = torch.empty(max(1, q.qlora_fwd_workspace_bytes(N, K, T, r)), dtype=torch.uint8, device="cuda")
    wsb = torch.empty(max(1, q.qlora_bwd_workspace_bytes(N, K, T, r)), dtype=torch.uint8, device="cuda")

    def step():
        q.qlora_linear_fwd(packed, codes, consts, X, A, B, alpha, Y=Y, U_out=U, workspace=wsf)
        q.qlora_linear_bwd(packed, codes, consts, X, A, B, alpha, dY, U_in=U, dX=dX, dA=dA, dB=dB, workspace=wsb)

    for _ in range(5):
        step()
        q.qlora_quantize_nf4(W, packed, codes, consts)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    q.qlora_trace_read(reset=True)
    q.qlora_trace_enable(True)
    for _ in range(steps):
        step()
        q.qlora_quantize_nf4(W, packed, codes, consts)
    torch.cuda.synchronize()
    q.qlora_trace_enable(False)
    kt = q.qlora_trace_read(reset=True)
    fwd_f, bwd_f = layer_flops(T, K, N, r)
    out = {"d_out": N, "d_in": K, "T": T, "r": r, "alpha": alpha, "fwd_bwd_ms": round(ms, 4),
           "tflops": round((fwd_f + bwd_f) / (ms * 1e-3) / 1e12, 1),
           "frac_mfma": round((fwd_f + bwd_f) / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
           "kernels_us": {k: round(v[1] / v[0] * 1e3, 2) for k, v in kt.items()}}
    fl = dict(zip(("fwd_gemm", "dx_gemm"), fused_flops(T, K, N, r)))
    for k in fl:
        if k in kt:
            out[f"{k}_frac_mfma"] = round(fl[k] / (kt[k][1] / kt[k][0] * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)
    qn, qms = kt.get("nf4_quantize", (1, float("nan")))
    n_c, n_k = codes.numel(), consts.numel() * 4
    q_bytes = N * K * 4 + N * K // 2 + n_c + n_k
    out["quantize"] = {"avg_us": round(qms / qn * 1e3, 2), "bytes": q_bytes,
                       "GBps": round(q_bytes / (qms / qn * 1e-3) / 1e9, 1),
                       "frac_hbm": round(q_bytes / (qms / qn * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}
    log("attn", out)
    return out


def decode_section(steps, warmup):
    """Packed-weight GB/s of the few-token forward (8192 <-> 28672, r=64),
    rotating 5 copies of each weight (> 512 MB) so the 256 MB MALL cannot hold them."""
    import numpy as np
    import torch
    import nf4_bit_quantized_amd as q
    import workloads

    out = {}
    copies = 5
    for dq, tag in ((True, ""), (False, "_fp32_scales")):
        for T in (1, 4, 16):
            for lin in workloads.decode_70b(T):
                inp = workloads.layer_inputs(lin.d_out, lin.d_in, T, lin.r, lin.seed, with_dy=False)
                W = torch.from_numpy(inp["W"]).cuda()
                pk, cd, cs = q.qlora_quantize_nf4(W, double_quant=dq)
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
                # the call rate untraced, then the kernels' own times in a traced pass
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                for i in range(steps):
                    p = reps[i % copies]
                    q.qlora_linear_fwd(p[0], p[1], p[2], X, A, B, lin.alpha, Y=Y, U_out=U, workspace=ws)
                e1.record()
                torch.cuda.synchronize()
                call_ms = e0.elapsed_time(e1) / steps
                q.qlora_trace_read(reset=True)
                q.qlora_trace_select({"decode", "decode_sum", "lora_down_gemm"})
                for i in range(steps):
                    p = reps[i % copies]
                    q.qlora_linear_fwd(p[0], p[1], p[2], X, A, B, lin.alpha, Y=Y, U_out=U, workspace=ws)
                torch.cuda.synchronize()
                q.qlora_trace_enable(False)
                kt = q.qlora_trace_read(reset=True)
                packed_bytes = pk.numel() + cd.numel() + cs.numel() * 4
                dec_n, dec_ms = kt.get("decode", (1, float("nan")))
                # a split contraction adds its ranges in a second kernel: counted with the stream
                sum_n, sum_ms = kt.get("decode_sum", (0, 0.0))
                sum_avg = sum_ms / max(dec_n, 1)
                dec_avg = dec_ms / max(dec_n, 1) + sum_avg
                u_n, u_ms = kt.get("lora_down_gemm", (1, float("nan")))
                out[lin.name + tag] = {
                    "T": T, "d_out": lin.d_out, "d_in": lin.d_in,
                    "scales": "8-bit codes + fp32 group constants" if dq else "fp32 per block (no second level)",
                    "packed_weight_bytes": packed_bytes,
                    "call_us": round(call_ms * 1e3, 2),
                    "packed_GBps_call": round(packed_bytes / (call_ms * 1e-3) / 1e9, 1),
                    "u_kernel_us": round(u_ms / max(u_n, 1) * 1e3, 2),
                    "decode_kernel_us": round(dec_avg * 1e3, 2),
                    "decode_sum_kernel_us": round(sum_avg * 1e3, 2) if sum_n else None,
                    "packed_GBps_kernel": round(packed_bytes / (dec_avg * 1e-3) / 1e9, 1),
                    "frac_hbm_kernel": round(packed_bytes / (dec_avg * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                }
                log("decode", lin.name + tag, out[lin.name + tag])
                del reps, pk, cd, cs
                torch.cuda.empty_cache()
    return out


def mall_copies(nbytes):
    """Copies of a call's operands to rotate so that together they hold more
    than twice the 256 MB MALL (2 to 8)."""
    return max(2, min(8, -(-(512 << 20) // max(nbytes, 1))))


def export_section(lin, steps):
    """HBM GB/s of the restored-weight export and of the merge on one weight,
    rotating copies of the packed weight and of the output (more than twice
    the 256 MB MALL together)."""
    import torch
    import nf4_bit_quantized_amd as q
    import workloads

    N, K, r = lin.d_out, lin.d_in, lin.r
    inp = workloads.layer_inputs(N, K, 1, r, lin.seed)
    W = torch.from_numpy(inp["W"]).cuda()
    pk, cd, cs = q.qlora_quantize_nf4(W)
    del W
    copies = mall_copies(N * K * 2 + pk.numel())
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
    del reps, outs
    torch.cuda.empty_cache()
    return out


def quantize16_section(lin, steps):
    """Quantization of one weight handed over as bf16 and as fp16 (2 bytes in
    per weight instead of 4), rotating copies of the weight (more than twice
    the 256 MB MALL together)."""
    import torch
    import nf4_bit_quantized_amd as q
    import workloads

    N, K = lin.d_out, lin.d_in
    W = workloads.layer_inputs(N, K, 1, 1, lin.seed, with_dy=False)["W"]
    copies = mall_copies(N * K * 2)
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
        torch.cuda.empty_cache()
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


def multi_proj_train_section(steps):
    """The projection groups of one 65B-class layer at 4096 tokens (r = 64,
    alpha = 16): query/key/value (three 8192 x 8192 weights) and gate/up (two
    8192 -> 22016), forward and backward, as one group call (one forward
    product over the group's weights, one dX product over their rows) against
    one call per weight.  Times in ms per group, fwd + bwd."""
    import torch
    import nf4_bit_quantized_amd as q

    K, T, r, alpha = 8192, 4096, 64, 16.0
    g = torch.Generator(device="cuda").manual_seed(1)
    out = {"tokens": T, "r": r}
    for name, shapes in (("qkv", (8192, 8192, 8192)), ("gate_up", (22016, 22016))):
        layers, dYs, outs, grads = [], [], [], []
        for N in shapes:
            pk, cd, cs = q.qlora_quantize_nf4(torch.randn(N, K, device="cuda", generator=g) * 0.02)
            layers.append((pk, cd, cs, (torch.randn(r, K, device="cuda", generator=g) / r).to(torch.bfloat16),
                           (torch.randn(N, r, device="cuda", generator=g) * 0.01).to(torch.bfloat16)))
            dYs.append(torch.randn(T, N, device="cuda", generator=g).to(torch.bfloat16))
            outs.append((torch.empty((T, N), dtype=torch.bfloat16, device="cuda"),
                         torch.empty((T, r), dtype=torch.float32, device="cuda")))
            grads.append((torch.empty((r, K), dtype=torch.float32, device="cuda"),
                          torch.empty((N, r), dtype=torch.float32, device="cuda")))
        X = torch.randn(T, K, device="cuda", generator=g).to(torch.bfloat16)
        dX = torch.empty((T, K), dtype=torch.bfloat16, device="cuda")
        ws_bytes = max(q.qlora_multi_fwd_workspace_bytes([(N, K) for N in shapes], T, r),
                       q.qlora_multi_bwd_workspace_bytes([(N, K) for N in shapes], T, r))
        ws = torch.empty(max(1, ws_bytes), dtype=torch.uint8, device="cuda")

        def fused():
            q.qlora_linear_fwd_multi(layers, X, alpha, workspace=ws, outs=outs)
            q.qlora_linear_bwd_multi(layers, X, alpha, dYs, U_ins=[o[1] for o in outs], workspace=ws, dX=dX,
                                     grads=grads)

        def separate():
            for l, o in zip(layers, outs):
                q.qlora_linear_fwd(*l[:3], X, l[3], l[4], alpha, Y=o[0], U_out=o[1], workspace=ws)
            for i, (l, o, dy, gr) in enumerate(zip(layers, outs, dYs, grads)):
                # one bf16 dX per weight; the caller would add them (not timed)
                q.qlora_linear_bwd(*l[:3], X, l[3], l[4], alpha, dy, U_in=o[1], dX=dX, dA=gr[0], dB=gr[1],
                                   workspace=ws)

        flops = sum(sum(layer_flops(T, K, N, r)) for N in shapes)
        for label, fn in (("group_call", fused), ("per_weight_calls", separate)):
            for _ in range(2):
                fn()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(steps):
                fn()
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / steps
            out[f"{name}_{label}_ms"] = round(ms, 3)
            out[f"{name}_{label}_tflops"] = round(flops / (ms * 1e-3) / 1e12, 1)
        del layers, dYs, outs, grads, X, dX, ws
    out["note"] = ("per-weight calls leave X's gradient as one bf16 tensor per weight (their sum is not "
                   "timed); the group call sums the shares in fp32 and rounds once")
    log("multi_proj_train", out)
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



# ---------------------------------------------------------------------------
# The oracle on the host cores
# ---------------------------------------------------------------------------

def dequant_matmul_section(steps):
    """The fused products against restoring the weight once and multiplying
    in bf16: for each weight shape of the 65B-class layer at 4096 tokens
    (r = 64, alpha = 16), the fused forward and dX kernels against this
    library's dequantize kernel (W_hat bf16 written to HBM) followed by
    torch's bf16 products X W_hat^T (F.linear) and dY W_hat on that W_hat
    (the ROCm BLAS library).  The second route keeps a 16-bit copy of every
    weight in HBM (2 bytes per weight instead of 0.52) and leaves out the
    rank-r term, which the fused kernels include.  Kernel times in us."""
    import torch
    import torch.nn.functional as F
    import nf4_bit_quantized_amd as q

    T, r, alpha = 4096, 64, 16.0
    g = torch.Generator(device="cuda").manual_seed(2)
    out = {"tokens": T, "r": r}
    for N, K in ((8192, 8192), (22016, 8192), (8192, 22016)):
        pk, cd, cs = q.qlora_quantize_nf4(torch.randn(N, K, device="cuda", generator=g) * 0.02)
        A = (torch.randn(r, K, device="cuda", generator=g) / r).to(torch.bfloat16)
        B = (torch.randn(N, r, device="cuda", generator=g) * 0.01).to(torch.bfloat16)
        X = torch.randn(T, K, device="cuda", generator=g).to(torch.bfloat16)
        dY = torch.randn(T, N, device="cuda", generator=g).to(torch.bfloat16)
        Y = torch.empty((T, N), dtype=torch.bfloat16, device="cuda")
        U = torch.empty((T, r), dtype=torch.float32, device="cuda")
        dX = torch.empty((T, K), dtype=torch.bfloat16, device="cuda")
        dA = torch.empty((r, K), dtype=torch.float32, device="cuda")
        dB = torch.empty((N, r), dtype=torch.float32, device="cuda")
        W_hat = torch.empty((N, K), dtype=torch.bfloat16, device="cuda")
        ws_bytes = max(q.qlora_fwd_workspace_bytes(N, K, T, r), q.qlora_bwd_workspace_bytes(N, K, T, r))
        ws = torch.empty(max(1, ws_bytes), dtype=torch.uint8, device="cuda")

        def fused():
            q.qlora_linear_fwd(pk, cd, cs, X, A, B, alpha, Y=Y, U_out=U, workspace=ws)
            q.qlora_linear_bwd(pk, cd, cs, X, A, B, alpha, dY, U_in=U, dX=dX, dA=dA, dB=dB, workspace=ws)

        for _ in range(2):
            fused()
            q.qlora_dequantize_nf4(pk, cd, cs, W_hat=W_hat)
        torch.cuda.synchronize()
        q.qlora_trace_read(reset=True)
        q.qlora_trace_select({"fwd_gemm", "dx_gemm", "export"})
        for _ in range(steps):
            fused()
            q.qlora_dequantize_nf4(pk, cd, cs, W_hat=W_hat)
        torch.cuda.synchronize()
        q.qlora_trace_enable(False)
        kt = q.qlora_trace_read(reset=True)
        # per call (a dX call can be two launches: whole rounds of 256x256
        # tiles, then the last columns on 256x128 tiles)
        us = {k: kt[k][1] / steps * 1e3 for k in ("fwd_gemm", "dx_gemm", "export")}

        def bf16_time(fn):
            for _ in range(2):
                fn()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(steps):
                fn()
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / steps * 1e3

        mm_fwd = bf16_time(lambda: F.linear(X, W_hat))
        mm_dx = bf16_time(lambda: torch.mm(dY, W_hat))
        base = 2.0 * T * K * N
        fwd_fl, dx_fl = fused_flops(T, K, N, r)
        fused_us = us["fwd_gemm"] + us["dx_gemm"]
        route_us = us["export"] + mm_fwd + mm_dx
        out[f"{N}x{K}"] = {
            "fused_fwd_us": round(us["fwd_gemm"], 1), "fused_fwd_tflops": round(fwd_fl / us["fwd_gemm"] / 1e6, 1),
            "fused_dx_us": round(us["dx_gemm"], 1), "fused_dx_tflops": round(dx_fl / us["dx_gemm"] / 1e6, 1),
            "dequantize_us": round(us["export"], 1),
            "bf16_fwd_us": round(mm_fwd, 1), "bf16_fwd_tflops": round(base / mm_fwd / 1e6, 1),
            "bf16_dx_us": round(mm_dx, 1), "bf16_dx_tflops": round(base / mm_dx / 1e6, 1),
            "fused_fwd_dx_us": round(fused_us, 1), "dequantize_then_bf16_us": round(route_us, 1),
            "fused_over_route": round(fused_us / route_us, 3),
        }
        del pk, cd, cs, A, B, X, dY, Y, U, dX, dA, dB, W_hat, ws
        torch.cuda.empty_cache()
    out["note"] = ("dequantize_then_bf16 = one dequantize per weight and step, then X W_hat^T and dY W_hat in "
                   "bf16 without the rank-r term; fused_over_route < 1 means the fused products are faster")
    log("dequant_matmul", out)
    return out


def _threads():
    from threadpoolctl import threadpool_info
    return int(max([i.get("num_threads", 1) for i in threadpool_info()] or [1]))


def time_oracle_linear(lin, T, quantize=False, backward=True):
    """Seconds of the oracle on one linear of the recipe: optionally its
    quantization, then the restore of the weight and the float64 forward
    (and backward) at T tokens."""
    import numpy as np
    import workloads
    from oracle import lora as olora
    from oracle import nf4 as onf4
    from oracle.bf16 import bits_to_float

    inp = workloads.layer_inputs(lin.d_out, lin.d_in, T, lin.r, lin.seed, with_dy=backward)
    t0 = time.perf_counter()
    Q = onf4.quantize(inp["W"])
    t_quant = time.perf_counter() - t0
    X, A, B = (bits_to_float(inp[k]) for k in ("X", "A", "B"))
    t0 = time.perf_counter()
    W_hat = onf4.dequantize(Q).astype(np.float64)
    olora.forward(W_hat, X, A, B, lin.alpha, lin.r)
    if backward:
        olora.backward(W_hat, X, A, B, bits_to_float(inp["dY"]), lin.alpha, lin.r)
    t_layer = time.perf_counter() - t0
    fwd, bwd = layer_flops(T, lin.d_in, lin.d_out, lin.r)
    flops = fwd + (bwd if backward else 0)
    out = {"layer_s": round(t_layer, 3), "tflops": round(flops / t_layer / 1e12, 4)}
    if quantize:
        out["quantize_s"] = round(t_quant, 3)
    return out


def cpu_baseline_headline():
    """The oracle on a bounded sample of the headline workload: the query
    projection of layer 0 (8192 x 8192) at all 4096 tokens, restore + forward
    + backward in float64, as TFLOP/s (the headline's unit)."""
    import workloads
    lin = workloads.stack_65b(1)[0]
    t = time_oracle_linear(lin, lin.T)
    return {
        "value": t["tflops"], "unit": "TFLOP/s", "cores": _threads(), "kind": "oracle",
        "sample": (f"one of the 56 linears of the stack: layer 0's query projection {lin.d_out}x{lin.d_in}, "
                   f"{lin.T} tokens, r={lin.r}: restore of the NF4 weight + float64 forward + backward, "
                   f"{t['layer_s']} s; the stack's step is 56 such linears (3 weight shapes); "
                   f"host threads available {len(os.sched_getaffinity(0))}"),
    }


def cpu_baselines(full):
    """The oracle timing plan per workload.  By default a bounded set (about
    half a minute of host time); with --cpu-full every planned case,
    including the few-token forward at each T and one layer of the stack
    (reported x8 as the whole share, extrapolated)."""
    import workloads
    out = {"cores": _threads(), "host_threads_available": len(os.sched_getaffinity(0))}
    (p,) = workloads.parity_256()
    out["parity_256"] = time_oracle_linear(p, p.T, quantize=True)
    (a,) = workloads.attn_4096()
    out["attn_4096"] = time_oracle_linear(a, a.T, quantize=True)
    mlp = workloads.mlp_llama7b()
    out["mlp_llama7b"] = {l.name: time_oracle_linear(l, l.T, quantize=True) for l in (mlp if full else mlp[:1])}
    if full:
        out["decode_70b"] = {f"{l.name}": time_oracle_linear(l, T, backward=False)
                             for T in (1, 4, 16) for l in workloads.decode_70b(T)}
        layer = workloads.stack_65b(1)
        per = {l.name: time_oracle_linear(l, l.T) for l in layer}
        s = sum(v["layer_s"] for v in per.values())
        flops = sum(sum(layer_flops(l.T, l.d_in, l.d_out, l.r)) for l in layer)
        out["stack_65b"] = {"one_layer": per, "one_layer_s": round(s, 2),
                            "eight_layers_s_extrapolated": round(8 * s, 2),
                            "tflops": round(flops / s / 1e12, 4)}
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(sharding the layer over several GPUs is not part of this library).", file=sys.stderr)
        sys.exit(2)

    import torch
    import workloads

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    log(f"stack: {args.layers} layers x 7 linears, 4096 tokens, r=64")
    st = stack_section(args)

    result = {
        "metric": "QLoRA linear fwd+bwd TFLOP/s & packed-weight GB/s; % of MI355X roofline",
        "value": round(st["value"], 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(st["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded: W ~ N(0, 0.02) fp32 quantized to NF4, X, dY ~ N(0, 1) bf16, A ~ N(0, 1/r), "
                "B ~ N(0, 0.01) bf16); no model weights or dataset",
        "config": {"workload": f"65B-class layer stack share: {args.layers} layers x (q, k, v, o 8192x8192; gate, up "
                               "8192->22016; down 22016->8192), NF4 block 64 + 8-bit scale codes per 256 blocks, "
                               "4096 tokens, r=64, alpha=16; step = fwd + bwd (dX, dA, dB) of every linear",
                   "layers": args.layers, "tokens": st["T"], "r": st["r"], "alpha": st["alpha"],
                   "step_flops": st["step_flops"]},
        "roofline": st["roofline"],
        "fused_products": st["fused_products"],
        "kernels": st["kernels"],
        "kernels_note": st["kernels_note"],
        "quantize_stack": st["quantize_stack"],
        "peak_hbm_allocated_bytes": st["peak_hbm_allocated_bytes"],
        "packed_weight_bytes": st["packed_weight_bytes"],
        "context": "the pages report a 65B model fine-tuned with this method on one 48 GB GPU in 24 hours "
                   "(no throughput figure); context only, not a target",
    }
    if not args.headline_only:
        (lin,) = workloads.attn_4096()
        sec_steps = max(20, args.steps)
        result["attn_4096"] = attn_section(lin, sec_steps)
        result["mlp_llama7b"] = mlp_section(steps=10)
        result["decode_packed_weight"] = decode_section(steps=sec_steps, warmup=5)
        gate = workloads.stack_65b(1)[4]  # 22016 x 8192: a size where the kernel's streaming rate shows
        result["export_bf16"] = export_section(lin, steps=sec_steps)
        result["export_bf16_22016x8192"] = export_section(gate, steps=sec_steps)
        result["quantize_16bit_weight"] = quantize16_section(lin, steps=sec_steps)
        result["quantize_16bit_weight_22016x8192"] = quantize16_section(gate, steps=sec_steps)
        result["adamw_65b_adapters"] = adamw_section(steps=sec_steps)
        result["lora_dropout_attn4096"] = dropout_section(lin, steps=sec_steps)
        result["qkv_gqa_70b"] = multi_proj_section(steps=sec_steps)
        result["projection_groups_65b"] = multi_proj_train_section(steps=10)
        result["dequant_then_bf16_65b"] = dequant_matmul_section(steps=10)
    if not args.no_cpu_baseline:
        log("timing the oracle on the host ...")
        result["cpu_baseline"] = cpu_baseline_headline()
        result["cpu_baselines"] = cpu_baselines(args.cpu_full)
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
