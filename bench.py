"""Throughput of the block-scaled quantize-then-GEMM hot path on one MI355X.

One step = one pass of the whole path over one batch: for every ViT block
and every linear layer (qkv, proj, fc1, fc2) quantize the activation and the
weight row-wise (both in one mx_quantize_batch launch) and run the
block-scaled GEMM with its bias epilogue (mx_gemm). The *_fc1gelu stacks
let fc1's epilogue write fc2's operand (mx_gemm_gelu_quantize); the *_lnq_*
stacks also take qkv's and fc1's inputs as the LayerNorm of an fp32
residual stream, normalized and quantized in one launch
(mx_layernorm_quantize). For the NVFP4 training workload a step is the fc1/fc2
pair's fprop, dgrad and wgrad GEMMs with every operand quantized along its
own K axis (row and transposed copies from one read with mx_quantize_dual,
tensor amax included).

Inputs are seeded synthetic bf16 tensors (the value recipe of
block_scaled_precision_mx_amd.workloads) generated on the device before the
timed region; every block has its own tensors so repeated launches cannot be
served from the 256 MB Infinity Cache. The JSON line reports whole-step
throughput in GEMM TFLOP/s (the GEMM flops of the step over the step time,
quantization included), the dominant GEMM kernel against the MFMA roofline
(per-launch HIP events on the stream the kernels run on), the quantizer's
algorithmic bandwidth, and the CPU oracle on a bounded sample of the same
workload.
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

# MI355X published dense peaks (TFLOP/s) and HBM bandwidth (GB/s)
PEAK_TFLOPS = {"mxfp8": 5000.0, "mxfp4": 10100.0, "fp16": 2500.0}
PEAK_HBM_GBS = 8000.0
# algorithmic bytes per quantized element: 2 read + codes + scales written
QUANT_BYTES = {"mxfp8": 2 + 1 + 1 / 32, "mxfp4": 2 + 0.5 + 1 / 32, "nvfp4": 2 + 0.5 + 1 / 16}
NVFP4_AMAX_BYTES = 2.0


WORKLOADS = ["vitl16_mxfp8_fwd_stack", "vitl16_mxfp4_fwd_stack", "vitb16_mxfp8_fwd_stack",
             "vitl16_mxfp8_fwd_stack_fc1gelu", "vitl16_mxfp4_fwd_stack_fc1gelu",
             "vitl16_mxfp8_fwd_stack_lnq_fc1gelu", "vitl16_mxfp4_fwd_stack_lnq_fc1gelu",
             "vitl16_nvfp4_fc1fc2_train", "vitl16_nvfp4_fc1fc2_train_srgrad", "vitl16_mxfp8_fc1fc2_train",
             "single_mxfp8_256x768x768"]


def parse():
    p = argparse.ArgumentParser(description=__doc__)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default="vitl16_mxfp8_fwd_stack", choices=WORKLOADS)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--copy-probe-mb", type=int, default=0,
                   help="first run one elementwise bf16 kernel (negation) reading and writing this many "
                        "MiB: a kernel of known traffic for calibrating memory counters")
    return p.parse_args()


# ------------------------------------------------------------------ workloads

class Op:
    """One launch of the path: a quantization or a GEMM (plan = kernel
    configuration). `cold`: the same launch on other input tensors of the
    same shape, used only to time the launch with inputs that are not cached."""

    def __init__(self, kind, fn, flops=0.0, nbytes=0.0, label="", plan=None, cold=()):
        self.kind, self.fn, self.flops, self.nbytes, self.label, self.plan = kind, fn, flops, nbytes, label, plan
        self.cold = list(cold)


# input bytes of a group of cold launches made of clones: twice the 256 MB
# Infinity Cache, so the group's inputs come from HBM
COLD_BYTES = 512 << 20


def build_stack(stack, dev):
    import torch
    from block_scaled_precision_mx_amd import api
    from block_scaled_precision_mx_amd import workloads as W

    ops = []
    fmt = stack.fmt
    for blk in range(stack.blocks):
        fused_out = None            # fc2's operand as fc1's fused epilogue writes it
        for lin in stack.linears:
            if fused_out is not None and lin.name == "fc2":
                # fc2's A operand comes from fc1's epilogue: no activation tensor, no quantization
                w = W.torch_normal((lin.n, lin.k), W.seed(stack.wid, blk, lin.w_id), W.W_STD, dev)
                bias = W.torch_normal((lin.n,), W.seed(stack.wid, blk, lin.bias_id), W.BIAS_STD, dev)
                qw = api.Quantized(torch.empty(api.codes_bytes(lin.n, lin.k, fmt), dtype=torch.uint8, device=dev),
                                   torch.empty(api.scales_bytes(lin.n, lin.k, fmt), dtype=torch.uint8, device=dev),
                                   fmt, lin.n, lin.k)
                out = torch.empty((stack.m, lin.n), dtype=torch.bfloat16, device=dev)
                # fc2's weight is the only tensor of this launch: two clones per
                # block make its cold-timing group larger than the Infinity Cache
                ops.append(Op("quant", lambda w=w, qw=qw: api.mx_quantize(w, fmt, "row", qw.codes, qw.scales),
                              nbytes=QUANT_BYTES[fmt] * w.numel(), label=f"quant_{lin.name}_w",
                              cold=[lambda w=w.clone(), qw=qw: api.mx_quantize(w, fmt, "row", qw.codes, qw.scales)
                                    for _ in range(2)]))
                ops.append(Op("gemm", lambda qa=fused_out, qw=qw, bias=bias, out=out: api.mx_gemm(qa, qw, bias, "bf16", out),
                              flops=2.0 * stack.m * lin.n * lin.k, label=f"gemm_{lin.name}",
                              plan=api.gemm_plan(stack.m, lin.n, lin.k, fmt)))
                continue
            w = W.torch_normal((lin.n, lin.k), W.seed(stack.wid, blk, lin.w_id), W.W_STD, dev)
            bias = W.torch_normal((lin.n,), W.seed(stack.wid, blk, lin.bias_id), W.BIAS_STD, dev)
            qa = api.Quantized(torch.empty(api.codes_bytes(stack.m, lin.k, fmt), dtype=torch.uint8, device=dev),
                               torch.empty(api.scales_bytes(stack.m, lin.k, fmt), dtype=torch.uint8, device=dev),
                               fmt, stack.m, lin.k)
            qw = api.Quantized(torch.empty(api.codes_bytes(lin.n, lin.k, fmt), dtype=torch.uint8, device=dev),
                               torch.empty(api.scales_bytes(lin.n, lin.k, fmt), dtype=torch.uint8, device=dev),
                               fmt, lin.n, lin.k)
            out = torch.empty((stack.m, lin.n), dtype=torch.bfloat16, device=dev)
            if stack.ln_quant and lin.name in ("qkv", "fc1"):
                # the input is the LayerNorm of the fp32 residual stream, normalized
                # and quantized in one launch; the weight in a launch of its own
                x = W.torch_residual((stack.m, lin.k), W.seed(stack.wid, blk, lin.a_id), dev)
                gamma, beta = W.torch_ln_params(lin.k, W.seed(stack.wid, blk, 50 + lin.a_id), dev)
                ops.append(Op("quant", lambda x=x, g=gamma, b=beta, qa=qa:
                              api.mx_layernorm_quantize(x, g, b, W.LN_EPS, fmt, out=qa),
                              nbytes=(4 + QUANT_BYTES[fmt] - 2) * x.numel(), label=f"lnquant_{lin.name}_act"))
                ops.append(Op("quant", lambda w=w, qw=qw: api.mx_quantize(w, fmt, "row", qw.codes, qw.scales),
                              nbytes=QUANT_BYTES[fmt] * w.numel(), label=f"quant_{lin.name}_w",
                              cold=[lambda w=w.clone(), qw=qw: api.mx_quantize(w, fmt, "row", qw.codes, qw.scales)
                                    for _ in range(2)]))
            else:
                a = W.torch_activation((stack.m, lin.k), W.seed(stack.wid, blk, lin.a_id), dev,
                                       gelu=lin.a_kind == "gelu")
                # the GEMM's two operands in one launch (mx_quantize_batch), just before it
                ops.append(Op("quant", lambda a=a, w=w, qa=qa, qw=qw: api.mx_quantize_batch([a, w], fmt, out=[qa, qw]),
                              nbytes=QUANT_BYTES[fmt] * (a.numel() + w.numel()), label=f"quant_{lin.name}_act_w"))
            if stack.fuse_fc1_gelu and lin.name == "fc1":
                del out
                fused_out = api.Quantized(
                    torch.empty(api.codes_bytes(stack.m, lin.n, fmt), dtype=torch.uint8, device=dev),
                    torch.empty(api.scales_bytes(stack.m, lin.n, fmt), dtype=torch.uint8, device=dev),
                    fmt, stack.m, lin.n)
                ops.append(Op("gemm", lambda qa=qa, qw=qw, bias=bias, q=fused_out:
                              api.mx_gemm_gelu_quantize(qa, qw, bias, out=q),
                              flops=2.0 * stack.m * lin.n * lin.k, label=f"gemm_{lin.name}_gelu_quant",
                              plan=api.gemm_plan(stack.m, lin.n, lin.k, fmt) + "+gelu+quant"))
                continue
            ops.append(Op("gemm", lambda qa=qa, qw=qw, bias=bias, out=out: api.mx_gemm(qa, qw, bias, "bf16", out),
                          flops=2.0 * stack.m * lin.n * lin.k, label=f"gemm_{lin.name}",
                          plan=api.gemm_plan(stack.m, lin.n, lin.k, fmt)))
    return ops


def build_train(tp, dev):
    import torch
    from block_scaled_precision_mx_amd import api
    from block_scaled_precision_mx_amd import workloads as W

    fmt = tp.fmt
    S = lambda tid: W.seed(tp.wid, 0, tid)   # noqa: E731
    X = W.torch_activation((tp.m, tp.hidden), S(tp.X), dev)
    H = W.torch_activation((tp.m, tp.mlp), S(tp.H), dev, gelu=True)
    dY1 = W.torch_normal((tp.m, tp.mlp), S(tp.DY1), W.GRAD_STD, dev)
    dY2 = W.torch_normal((tp.m, tp.hidden), S(tp.DY2), W.GRAD_STD, dev)
    W1 = W.torch_normal((tp.mlp, tp.hidden), S(tp.W1), W.W_STD, dev)
    W2 = W.torch_normal((tp.hidden, tp.mlp), S(tp.W2), W.W_STD, dev)
    b1 = W.torch_normal((tp.mlp,), S(tp.B1), W.BIAS_STD, dev)
    b2 = W.torch_normal((tp.hidden,), S(tp.B2), W.BIAS_STD, dev)
    ops = []
    q = {}

    # bytes per element of one dual quantization: the read, both copies'
    # codes and scales, and for NVFP4 the amax pass (s_t from the tensor's
    # own amax, as the config defines)
    dual_bytes = 2.0 + 2 * (QUANT_BYTES[fmt] - 2.0) + (NVFP4_AMAX_BYTES if fmt == "nvfp4" else 0.0)

    def quant_dual(name, t, sr=False):
        """Both copies of t (row, and transposed for the other GEMMs) from one
        read (mx_quantize_dual; mx_quantize_dual_sr for stochastically
        rounded gradients)."""
        r, c = t.shape
        bufs = []
        for axis, rows, length in (("row", r, c), ("col", c, r)):
            bufs.append(api.Quantized(torch.empty(api.codes_bytes(r, c, fmt, axis), dtype=torch.uint8, device=dev),
                                      torch.empty(api.scales_bytes(r, c, fmt, axis), dtype=torch.uint8, device=dev),
                                      fmt, rows, length))
        q[name + "_row"], q[name + "_col"] = bufs

        def make_fn(src):
            if sr:
                return lambda: api.mx_quantize_dual_sr(src, tp.sr_seed, None, 1.0, out=(bufs[0], bufs[1]))
            return lambda: api.mx_quantize_dual(src, fmt, None, 1.0, out=(bufs[0], bufs[1]))
        # clones of t for cold timing only (the step itself reads t)
        copies = min(64, -(-COLD_BYTES // (2 * t.numel()))) - 1
        ops.append(Op("quant", make_fn(t), nbytes=dual_bytes * t.numel(), label=f"quant_{name}_rowcol",
                      cold=[make_fn(t.clone()) for _ in range(copies)]))

    def gemm(name, a, b, bias, m, n, k):
        out = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
        ops.append(Op("gemm", lambda: api.mx_gemm(q[a], q[b], bias, "bf16", out), flops=2.0 * m * n * k,
                      label=f"gemm_{name}", plan=api.gemm_plan(m, n, k, fmt)))

    # fc1: fprop X W1^T, dgrad dY1 W1, wgrad dY1^T X
    quant_dual("X", X); quant_dual("W1", W1)
    gemm("fc1_fprop", "X_row", "W1_row", b1, tp.m, tp.mlp, tp.hidden)
    quant_dual("dY1", dY1, sr=tp.sr_grads)
    gemm("fc1_dgrad", "dY1_row", "W1_col", None, tp.m, tp.hidden, tp.mlp)
    gemm("fc1_wgrad", "dY1_col", "X_col", None, tp.mlp, tp.hidden, tp.m)
    # fc2: fprop H W2^T, dgrad dY2 W2, wgrad dY2^T H
    quant_dual("H", H); quant_dual("W2", W2)
    gemm("fc2_fprop", "H_row", "W2_row", b2, tp.m, tp.hidden, tp.mlp)
    quant_dual("dY2", dY2, sr=tp.sr_grads)
    gemm("fc2_dgrad", "dY2_row", "W2_col", None, tp.m, tp.mlp, tp.hidden)
    gemm("fc2_wgrad", "dY2_col", "H_col", None, tp.hidden, tp.mlp, tp.m)
    return ops


# ------------------------------------------------------------------ CPU oracle

def cpu_baseline(workload_name, fmt):
    """The oracle as it stands on a bounded sample of the same workload: the
    four linears of one ViT block at full M (one of the stack's blocks), or
    the fc1 fprop GEMM of the training pair at full M; returns GEMM TFLOP/s of
    quantize + dequantize + float64 GEMM."""
    import numpy as np  # noqa: F401
    from block_scaled_precision_mx_amd import workloads as W
    from oracle import gemm as G
    from oracle import quantize as Q

    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    if workload_name in W.TRAIN_PAIRS:
        tp = W.TRAIN_PAIRS[workload_name]
        rows = tp.m
        shapes = [("fc1_fprop", tp.mlp, tp.hidden, "act")]
        wid = tp.wid
    else:
        stack = W.STACKS[workload_name]
        rows = stack.m
        shapes = [(l.name, l.n, l.k, l.a_kind) for l in stack.linears]
        wid = stack.wid
    gen = []
    for i, (name, n, k, kind) in enumerate(shapes):
        a = (W.np_gelu_activation if kind == "gelu" else W.np_activation)((rows, k), W.seed(wid, 0, 3 * i))
        w = W.np_normal((n, k), W.seed(wid, 0, 3 * i + 1), W.W_STD)
        b = W.np_normal((n,), W.seed(wid, 0, 3 * i + 2), W.BIAS_STD)
        gen.append((a, w, b, n, k))
    t0 = time.perf_counter()
    flops = 0.0
    for a, w, b, n, k in gen:
        qa, qw = Q.quantize(a, fmt), Q.quantize(w, fmt)
        G.gemm_ref(qa, qw, b)
        flops += 2.0 * rows * n * k
    dt = time.perf_counter() - t0
    sample = f"{len(gen)} quantize+GEMM(s) of one block at full M: " + ", ".join(
        f"{rows}x{n}x{k}" for _, _, _, n, k in gen)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": sample, "seconds": round(dt, 3)}


# ------------------------------------------------------------------ traffic

# the sources a kernel's machine code is built from (its file and the device
# headers it includes); their hash ties a counter summary to one build
_DEVICE_HEADERS = ["block_scaled_precision_mx_amd/csrc/gemm_common.h", "block_scaled_precision_mx_amd/csrc/mx_device.h"]
KERNEL_SOURCES = {"gemm_mx_kernel": ["block_scaled_precision_mx_amd/csrc/gemm_mx.hip"] + _DEVICE_HEADERS,
                  "gemm_nv_kernel": ["block_scaled_precision_mx_amd/csrc/gemm_nv.hip"] + _DEVICE_HEADERS}


def source_sha256(kernel):
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kernel.split("<")[0]]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` on `workload` from the committed
    rocprofv3 counter summary under profiles/ (FETCH_SIZE and WRITE_SIZE,
    each scaled by its copy-kernel calibration factor). None when no summary
    exists or the kernel source changed since the counters were taken."""
    prof_dir = os.path.join(ROOT, "profiles")
    if not os.path.isdir(prof_dir):
        return None
    for name in sorted(os.listdir(prof_dir)):
        if not name.endswith(".md"):
            continue
        fields = {}
        with open(os.path.join(prof_dir, name)) as f:
            for line in f:
                if line.startswith("- ") and ": " in line:
                    k, v = line[2:].strip().split(": ", 1)
                    fields[k.strip("`")] = v.strip().strip("`")
        if fields.get("roofline_kernel") != kernel or fields.get("workload") != workload:
            continue
        if fields.get("kernel_source_sha256") != source_sha256(kernel):
            return None
        try:
            return float(fields["traffic_bytes_per_launch"])
        except (KeyError, ValueError):
            return None
    return None


# ------------------------------------------------------------------ main

def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: --gpus must be 1. The kernels here run one GPU's "
              "share of the work; nothing in this package uses a second GPU or a collective.",
              file=sys.stderr)
        sys.exit(2)
    import torch
    from block_scaled_precision_mx_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    if args.workload in W.TRAIN_PAIRS:
        wl = W.TRAIN_PAIRS[args.workload]
        fmt = wl.fmt
        ops = build_train(wl, dev)
        gemm_peak_key = "fp16" if fmt == "nvfp4" else fmt
        config = {"workload": wl.name, "M": wl.m, "hidden": wl.hidden, "mlp": wl.mlp, "tokens_per_image": W.TOKENS,
                  "batch": wl.m // W.TOKENS, "format": fmt, "gemms": "fc1/fc2 fprop+dgrad+wgrad",
                  "quantizations": "6 tensors, row and transposed copies from one read each",
                  "grad_rounding": "stochastic (Philox4x64-10)" if wl.sr_grads else "nearest-even"}
    else:
        wl = W.STACKS[args.workload]
        fmt = wl.fmt
        ops = build_stack(wl, dev)
        gemm_peak_key = fmt
        config = {"workload": wl.name, "M": wl.m, "hidden": wl.hidden, "mlp": wl.mlp, "blocks": wl.blocks,
                  "tokens_per_image": W.TOKENS, "batch": wl.m // W.TOKENS, "format": fmt,
                  "gemms_per_block": [f"{l.name} {l.n}x{l.k}" for l in wl.linears]}
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    if args.copy_probe_mb:
        n = args.copy_probe_mb * (1 << 20) // 2
        src = torch.empty(n, dtype=torch.bfloat16, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    def step():
        for op in ops:
            op.fn()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: K steps, events on the stream the kernels run on
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for _ in range(args.steps):
        step()
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ms_per_step = total_ms / args.steps

    # per-launch durations on the same stream, several launches between one
    # event pair so that the events' own overhead is spread over them.
    # GEMMs: each launch repeated REPEAT times back to back. In the step their
    # operands were written just before them, so they are cached there too
    # (rocprofv3's trace of the in-step launches agrees within 2%).
    # Quantizations: all launches of one label, each on an input no other
    # launch of the group reads (the stack's blocks, or clones of the
    # training tensors), more than the 256 MB Infinity Cache per group (428 MB
    # for the smallest, ViT-B's proj), so the inputs come from HBM as they do
    # in the step.
    REPEAT = 10
    groups = []                                   # (op indices, launches timed together)
    quant_labels = {}
    for i, op in enumerate(ops):
        if op.kind == "quant":
            quant_labels.setdefault(op.label, []).append(i)
        else:
            groups.append(([i], [op.fn] * REPEAT))
    for idx in quant_labels.values():
        fns = [f for i in idx for f in [ops[i].fn] + ops[i].cold]
        groups.append((idx, fns))
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in groups]
    per_op = [0.0] * len(ops)
    for _ in range(args.steps):
        for g, (idx, fns) in enumerate(groups):
            ev[g][0].record(stream)
            for f in fns:
                f()
            ev[g][1].record(stream)
        torch.cuda.synchronize()
        for g, (idx, fns) in enumerate(groups):
            t = ev[g][0].elapsed_time(ev[g][1]) / len(fns)
            for i in idx:
                per_op[i] += t
    per_op = [t / args.steps for t in per_op]

    gemm_flops = sum(op.flops for op in ops)
    gemm_ms = sum(t for op, t in zip(ops, per_op) if op.kind == "gemm")
    quant_bytes = sum(op.nbytes for op in ops if op.kind == "quant")
    quant_ms = sum(t for op, t in zip(ops, per_op) if op.kind == "quant")
    by_label = {}
    for op, t in zip(ops, per_op):
        d = by_label.setdefault(op.label, {"ms": 0.0, "n": 0, "flops": 0.0, "bytes": 0.0})
        d["ms"] += t
        d["n"] += 1
        d["flops"] += op.flops
        d["bytes"] += op.nbytes
    breakdown = {}
    for lab, d in by_label.items():
        e = {"us_per_launch": round(1e3 * d["ms"] / d["n"], 2)}
        if d["flops"]:
            e["tflops"] = round(d["flops"] / (d["ms"] * 1e-3) / 1e12, 1)
        if d["bytes"]:
            e["gbps"] = round(d["bytes"] / (d["ms"] * 1e-3) / 1e9, 1)
        breakdown[lab] = e

    # GEMM launches grouped by kernel configuration; the roofline reports the
    # configuration that takes the most time (the dominant kernel)
    plans = {}
    for op, t in zip(ops, per_op):
        if op.kind != "gemm":
            continue
        d = plans.setdefault(op.plan, {"ms": 0.0, "flops": 0.0, "n": 0})
        d["ms"] += t
        d["flops"] += op.flops
        d["n"] += 1
    dom = max(plans, key=lambda k: plans[k]["ms"])
    dom_d = plans[dom]
    achieved = dom_d["flops"] / (dom_d["ms"] * 1e-3) / 1e12
    peak = PEAK_TFLOPS[gemm_peak_key]
    value = gemm_flops / (ms_per_step * 1e-3) / 1e12
    result = {
        "metric": "block-scaled GEMM TFLOP/s of the whole quantize-then-GEMM step on ViT-L shapes",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8-e4m3" if fmt == "mxfp8" else ("fp4-e2m1+fp16-mfma" if fmt == "nvfp4" else "fp4-e2m1"),
        "data": "synthetic (seeded, device-generated bf16; no dataset or weights)",
        "config": config,
        "roofline": {
            "bound": "mfma",
            "kernel": dom,
            "achieved": round(achieved, 1),
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4),
            "traffic": measured_traffic(dom, config["workload"]),
            "launches_per_step": dom_d["n"],
            "avg_launch_us": round(1e3 * dom_d["ms"] / dom_d["n"], 2),
            "flops_per_launch_avg": dom_d["flops"] / dom_d["n"],
        },
        "gemm_kernels": {k: {"launches_per_step": d["n"], "avg_launch_us": round(1e3 * d["ms"] / d["n"], 2),
                             "tflops": round(d["flops"] / (d["ms"] * 1e-3) / 1e12, 1)} for k, d in plans.items()},
        "gemm_only_tflops": round(gemm_flops / (gemm_ms * 1e-3) / 1e12, 1),
        "quant": {"gbps": round(quant_bytes / (quant_ms * 1e-3) / 1e9, 1), "peak_gbps": PEAK_HBM_GBS,
                  "frac": round(quant_bytes / (quant_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                  "ms_per_step": round(quant_ms, 4)},
        "breakdown": breakdown,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(config["workload"], fmt)
    print(json.dumps(result))


if __name__ == "__main__":
    main()
