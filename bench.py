"""Throughput of the block-scaled quantize-then-GEMM hot path on one MI355X.

One step = one pass of the whole path over one batch. For the forward
stacks: for every ViT block and every linear layer (qkv, proj, fc1, fc2)
quantize the activation and the weight row-wise (both in one
mx_quantize_batch launch) and run the block-scaled GEMM with its bias
epilogue (mx_gemm). The *_fc1gelu stacks let fc1's epilogue write fc2's
operand (mx_gemm_gelu_quantize); the *_lnq_* stacks also take qkv's and
fc1's inputs as the LayerNorm of an fp32 residual stream, normalized and
quantized in one launch (mx_layernorm_quantize). For the training workloads
a step is the fprop, dgrad and wgrad GEMMs of the fc1/fc2 pair, or of all
four linears of a ViT block (twelve GEMMs), with every operand quantized
along its own K axis (row and transposed copies from one read with
mx_quantize_dual, or mx_quantize_dual_sr for stochastically rounded
gradients).

Inputs are seeded synthetic bf16 tensors (the value recipe of
block_scaled_precision_mx_amd.workloads) generated on the device before the
timed region; the stack's blocks, and the training workloads' alternating
input sets, have tensors of their own, so consecutive launches cannot be
served from the 256 MB Infinity Cache.

The JSON line reports, for the headline workload (the ViT-L MXFP8 forward
stack), whole-step throughput in GEMM TFLOP/s (the GEMM flops of the step
over the step time, quantization included); the dominant GEMM kernel (the
hand-written GEMM in the operand format that takes most of the step's GPU
time, over every tile configuration the planner picks for the step's
shapes) against the MFMA roofline, its average launch duration taken
from HIP events on the stream the kernels run on, around replays of the
step's launches grouped by label (each launch on its own operands, as in
the step); the quantizer's algorithmic
bandwidth; the CPU oracle on a bounded sample of the same workload; and,
under "configs", the same figures for every other configuration.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time
from dataclasses import dataclass

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# MI355X published dense peaks (TFLOP/s) and HBM bandwidth (GB/s)
PEAK_TFLOPS = {"mxfp8": 5000.0, "mxfp4": 10100.0, "fp16": 2500.0}
PEAK_HBM_GBS = 8000.0
# algorithmic bytes per quantized element: 2 read + codes + scales written
QUANT_BYTES = {"mxfp8": 2 + 1 + 1 / 32, "mxfp4": 2 + 0.5 + 1 / 32, "nvfp4": 2 + 0.5 + 1 / 16}
NVFP4_AMAX_BYTES = 2.0

HEADLINE = "vitl16_mxfp8_fwd_stack"
# the other configurations measured in the same run (compact records)
EXTRA_CONFIGS = ["single_mxfp8_256x768x768", "vitb16_mxfp8_fwd_stack", "vitl16_mxfp4_fwd_stack",
                 "vitl16_nvfp4_fc1fc2_train", "vitl16_mxfp8_block_train", "vitl16_p3_block_train"]
WORKLOADS = ["vitl16_mxfp8_fwd_stack", "vitl16_mxfp4_fwd_stack", "vitb16_mxfp8_fwd_stack",
             "vitl16_mxfp8_fwd_stack_fc1gelu", "vitl16_mxfp4_fwd_stack_fc1gelu",
             "vitl16_mxfp8_fwd_stack_lnq_fc1gelu", "vitl16_mxfp4_fwd_stack_lnq_fc1gelu",
             "vitl16_nvfp4_fc1fc2_train", "vitl16_nvfp4_fc1fc2_train_srgrad", "vitl16_mxfp8_fc1fc2_train",
             "vitl16_mxfp8_block_train", "vitl16_p3_block_train", "single_mxfp8_256x768x768"]
# the pages' own figures for the same kind of work (another GPU, another
# batch): context only, never a ratio
PAGES_CONTEXT = {
    "vitl16_mxfp8_block_train": "README section 5.4: the 12 GEMMs of one ViT-L block take 1042 us in MXFP8 on an "
                                "RTX 5090 (2585 us in BF16), plus 203 us of quantization; batch not stated",
    "vitl16_p3_block_train": "README section 5.4: backbone dgrad / wgrad GEMM time per step drops from 8.4-8.8 ms "
                             "(MXFP8) to 4.5-4.6 ms (NVFP4) on an RTX 5090",
}
# workspace the training workloads give their GEMMs (mx_gemm_ws): enough for
# the split-K partials of every weight-gradient GEMM of the ViT-L shapes
WORKSPACE_BYTES = 64 << 20
# input sets the fc1/fc2 training workloads rotate through, one per step:
# together they hold more than the 256 MB Infinity Cache
TRAIN_SETS = 4


def parse():
    p = argparse.ArgumentParser(description=__doc__)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default=HEADLINE, choices=WORKLOADS)
    p.add_argument("--only", action="store_true", help="measure --workload only (no other configurations)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--copy-probe-mb", type=int, default=0,
                   help="first run one elementwise bf16 kernel (negation) reading and writing this many "
                        "MiB: a kernel of known traffic for calibrating memory counters")
    return p.parse_args()


# ------------------------------------------------------------------ GEMM lists

@dataclass(frozen=True)
class GemmSpec:
    """One GEMM launch of a workload's step: C[m, n] from A [m, k], B [n, k]."""
    label: str
    m: int
    n: int
    k: int
    fmt: str
    epilogue: str = "c"          # "c": bf16 C out; "gelu_quant": fc1 writing fc2's operand
    out: str = "bf16"
    ws: bool = False             # launched by mx_gemm_ws with WORKSPACE_BYTES of workspace


def workload_gemms(name):
    """Every GEMM of one step of the workload, in launch order (needs no GPU)."""
    from block_scaled_precision_mx_amd import workloads as W
    specs = []
    if name in W.STACKS:
        st = W.STACKS[name]
        for _ in range(st.blocks):
            for lin in st.linears:
                fused = st.fuse_fc1_gelu and lin.name == "fc1"
                specs.append(GemmSpec(f"gemm_{lin.name}" + ("_gelu_quant" if fused else ""), st.m, lin.n, lin.k,
                                      st.fmt, "gelu_quant" if fused else "c", "q" if fused else "bf16"))
    elif name in W.TRAIN_PAIRS:
        tp = W.TRAIN_PAIRS[name]
        for lin, n_out, k_in in (("fc1", tp.mlp, tp.hidden), ("fc2", tp.hidden, tp.mlp)):
            specs.append(GemmSpec(f"gemm_{lin}_fprop", tp.m, n_out, k_in, tp.fmt, ws=True))
            specs.append(GemmSpec(f"gemm_{lin}_dgrad", tp.m, k_in, n_out, tp.fmt, ws=True))
            specs.append(GemmSpec(f"gemm_{lin}_wgrad", n_out, k_in, tp.m, tp.fmt, ws=True))
    elif name in W.BLOCK_TRAINS:
        bt = W.BLOCK_TRAINS[name]
        lins = bt.linears()
        for _ in range(bt.blocks):
            for lin in lins:
                specs.append(GemmSpec(f"gemm_{lin.name}_fprop", bt.m, lin.n, lin.k, bt.fwd_fmt, ws=True))
            for lin in reversed(lins):
                specs.append(GemmSpec(f"gemm_{lin.name}_dgrad", bt.m, lin.k, lin.n, bt.bwd_fmt, ws=True))
                specs.append(GemmSpec(f"gemm_{lin.name}_wgrad", lin.n, lin.k, bt.m, bt.bwd_fmt, ws=True))
    else:
        raise KeyError(name)
    return specs


def gemm_plan(spec: GemmSpec) -> str:
    from block_scaled_precision_mx_amd import api
    if spec.ws:
        return api.gemm_ws_plan(spec.m, spec.n, spec.k, spec.fmt, WORKSPACE_BYTES)
    return api.gemm_plan(spec.m, spec.n, spec.k, spec.fmt) + ("+gelu+quant" if spec.epilogue == "gelu_quant" else "")


# ------------------------------------------------------------------ workloads

class Op:
    """One launch of the path: a quantization (nbytes algorithmic) or a GEMM
    (flops, spec, plan = kernel configuration)."""

    def __init__(self, kind, fn, label, flops=0.0, nbytes=0.0, spec=None):
        self.kind, self.fn, self.label, self.flops, self.nbytes, self.spec = kind, fn, label, flops, nbytes, spec
        self.plan = gemm_plan(spec) if spec is not None else None


def _empty_q(rows, cols, fmt, axis, dev):
    import torch
    from block_scaled_precision_mx_amd import api
    stored, length = (rows, cols) if axis == "row" else (cols, rows)
    return api.Quantized(torch.empty(api.codes_bytes(rows, cols, fmt, axis), dtype=torch.uint8, device=dev),
                         torch.empty(api.scales_bytes(rows, cols, fmt, axis), dtype=torch.uint8, device=dev),
                         fmt, stored, length)


def _gemm_op(ops, spec, a, b, bias, dev, ws=None):
    """A GEMM launch: mx_gemm, or mx_gemm_ws with the workload's workspace."""
    import torch
    from block_scaled_precision_mx_amd import api
    out = torch.empty((spec.m, spec.n), dtype=torch.bfloat16, device=dev)
    if spec.ws:
        fn = lambda: api.mx_gemm_ws(a, b, bias, "bf16", ws, out)   # noqa: E731
    else:
        fn = lambda: api.mx_gemm(a, b, bias, "bf16", out)          # noqa: E731
    ops.append(Op("gemm", fn, spec.label, flops=2.0 * spec.m * spec.n * spec.k, spec=spec))


def build_stack(stack, dev):
    """A step of a forward stack: a list of ops."""
    from block_scaled_precision_mx_amd import api
    from block_scaled_precision_mx_amd import workloads as W

    specs = iter(workload_gemms(stack.name))
    ops = []
    fmt = stack.fmt
    for blk in range(stack.blocks):
        fused_out = None            # fc2's operand as fc1's fused epilogue writes it
        for lin in stack.linears:
            spec = next(specs)
            w = W.torch_normal((lin.n, lin.k), W.seed(stack.wid, blk, lin.w_id), W.W_STD, dev)
            bias = W.torch_normal((lin.n,), W.seed(stack.wid, blk, lin.bias_id), W.BIAS_STD, dev)
            qw = _empty_q(lin.n, lin.k, fmt, "row", dev)
            if fused_out is not None and lin.name == "fc2":
                # fc2's A operand comes from fc1's epilogue: only the weight is quantized
                ops.append(Op("quant", lambda w=w, qw=qw: api.mx_quantize(w, fmt, "row", qw.codes, qw.scales),
                              f"quant_{lin.name}_w", nbytes=QUANT_BYTES[fmt] * w.numel()))
                _gemm_op(ops, spec, fused_out, qw, bias, dev)
                continue
            qa = _empty_q(stack.m, lin.k, fmt, "row", dev)
            if stack.ln_quant and lin.name in ("qkv", "fc1"):
                # the input is the LayerNorm of the fp32 residual stream, normalized
                # and quantized in one launch; the weight in a launch of its own
                x = W.torch_residual((stack.m, lin.k), W.seed(stack.wid, blk, lin.a_id), dev)
                gamma, beta = W.torch_ln_params(lin.k, W.seed(stack.wid, blk, 50 + lin.a_id), dev)
                ops.append(Op("quant", lambda x=x, g=gamma, b=beta, qa=qa:
                              api.mx_layernorm_quantize(x, g, b, W.LN_EPS, fmt, out=qa),
                              f"lnquant_{lin.name}_act", nbytes=(4 + QUANT_BYTES[fmt] - 2) * x.numel()))
                ops.append(Op("quant", lambda w=w, qw=qw: api.mx_quantize(w, fmt, "row", qw.codes, qw.scales),
                              f"quant_{lin.name}_w", nbytes=QUANT_BYTES[fmt] * w.numel()))
            else:
                a = W.torch_activation((stack.m, lin.k), W.seed(stack.wid, blk, lin.a_id), dev,
                                       gelu=lin.a_kind == "gelu")
                # the GEMM's two operands in one launch (mx_quantize_batch), just before it
                ops.append(Op("quant", lambda a=a, w=w, qa=qa, qw=qw: api.mx_quantize_batch([a, w], fmt, out=[qa, qw]),
                              f"quant_{lin.name}_act_w", nbytes=QUANT_BYTES[fmt] * (a.numel() + w.numel())))
            if spec.epilogue == "gelu_quant":
                fused_out = _empty_q(stack.m, lin.n, fmt, "row", dev)
                ops.append(Op("gemm", lambda qa=qa, qw=qw, bias=bias, q=fused_out:
                              api.mx_gemm_gelu_quantize(qa, qw, bias, out=q), spec.label,
                              flops=2.0 * spec.m * spec.n * spec.k, spec=spec))
                continue
            _gemm_op(ops, spec, qa, qw, bias, dev)
    return [ops]


def _dual_bytes(fmt):
    """Bytes per element of one dual quantization: the read, both copies'
    codes and scales, and for NVFP4 the amax pass (s_t from the tensor's own
    amax, as the configuration defines)."""
    return 2.0 + 2 * (QUANT_BYTES[fmt] - 2.0) + (NVFP4_AMAX_BYTES if fmt == "nvfp4" else 0.0)


def _quant_dual(ops, label, t, fmt, dev, sr_seed=None):
    """Both copies of t (row, and transposed for the other GEMMs) from one
    read; returns (row copy, col copy)."""
    from block_scaled_precision_mx_amd import api
    r, c = t.shape
    row, col = _empty_q(r, c, fmt, "row", dev), _empty_q(r, c, fmt, "col", dev)
    if sr_seed is not None:
        fn = lambda: api.mx_quantize_dual_sr(t, sr_seed, None, 1.0, out=(row, col))   # noqa: E731
    else:
        fn = lambda: api.mx_quantize_dual(t, fmt, None, 1.0, out=(row, col))          # noqa: E731
    ops.append(Op("quant", fn, label, nbytes=_dual_bytes(fmt) * t.numel()))
    return row, col


def build_train(tp, dev):
    """TRAIN_SETS steps of the fc1/fc2 training pair, each on its own tensors."""
    from block_scaled_precision_mx_amd import workloads as W

    import torch
    fmt = tp.fmt
    ws = torch.empty(WORKSPACE_BYTES, dtype=torch.uint8, device=dev)
    sets = []
    for s in range(TRAIN_SETS):
        S = lambda tid: W.seed(tp.wid, s, tid)   # noqa: E731
        X = W.torch_activation((tp.m, tp.hidden), S(tp.X), dev)
        H = W.torch_activation((tp.m, tp.mlp), S(tp.H), dev, gelu=True)
        dY1 = W.torch_normal((tp.m, tp.mlp), S(tp.DY1), W.GRAD_STD, dev)
        dY2 = W.torch_normal((tp.m, tp.hidden), S(tp.DY2), W.GRAD_STD, dev)
        W1 = W.torch_normal((tp.mlp, tp.hidden), S(tp.W1), W.W_STD, dev)
        W2 = W.torch_normal((tp.hidden, tp.mlp), S(tp.W2), W.W_STD, dev)
        b1 = W.torch_normal((tp.mlp,), S(tp.B1), W.BIAS_STD, dev)
        b2 = W.torch_normal((tp.hidden,), S(tp.B2), W.BIAS_STD, dev)
        sr = tp.sr_seed if tp.sr_grads else None
        specs = iter(workload_gemms(tp.name))
        ops = []
        for x, w, dy, bias, lin in ((X, W1, dY1, b1, "fc1"), (H, W2, dY2, b2, "fc2")):
            x_row, x_col = _quant_dual(ops, f"quant_{lin}_x_rowcol", x, fmt, dev)
            w_row, w_col = _quant_dual(ops, f"quant_{lin}_w_rowcol", w, fmt, dev)
            _gemm_op(ops, next(specs), x_row, w_row, bias, dev, ws)                   # fprop
            dy_row, dy_col = _quant_dual(ops, f"quant_{lin}_dy_rowcol", dy, fmt, dev, sr)
            _gemm_op(ops, next(specs), dy_row, w_col, None, dev, ws)                  # dgrad
            _gemm_op(ops, next(specs), dy_col, x_col, None, dev, ws)                  # wgrad
        sets.append(ops)
    return sets


def build_block_train(bt, dev):
    """One step = the twelve GEMMs of `bt.blocks` ViT blocks with their
    quantizations, in the order a training step runs them: the forward GEMMs
    (fprop), then per linear in reverse order the backward ones (dgrad,
    wgrad). FINAL (one format): each of X, W and dY is dual-quantized once
    (X and W when the forward pass uses them, dY in the backward pass). P3
    (MXFP8 forward, NVFP4 backward): X and W are row-quantized in MXFP8 for
    fprop (one batch launch, which also reduces their amax) and quantized
    again along the other axis in NVFP4 for the backward GEMMs, with the
    tensor scale from that amax (no amax pass); dY gets both NVFP4 copies,
    stochastically rounded, from one read."""
    from block_scaled_precision_mx_amd import api
    from block_scaled_precision_mx_amd import workloads as W
    from block_scaled_precision_mx_amd._lib import AMAX_WORDS

    import torch
    specs = iter(workload_gemms(bt.name))
    lins = bt.linears()
    ff, bf = bt.fwd_fmt, bt.bwd_fmt
    ws = torch.empty(WORKSPACE_BYTES, dtype=torch.uint8, device=dev)
    sr = bt.sr_seed if bt.sr_grads else None
    ops = []
    for blk in range(bt.blocks):
        S = lambda tid: W.seed(bt.wid, blk, tid)   # noqa: E731
        saved = []
        for i, lin in enumerate(lins):                       # forward
            xi, wi, bi, di = bt.ids(i)
            x = W.torch_activation((bt.m, lin.k), S(xi), dev, gelu=lin.a_kind == "gelu")
            w = W.torch_normal((lin.n, lin.k), S(wi), W.W_STD, dev)
            bias = W.torch_normal((lin.n,), S(bi), W.BIAS_STD, dev)
            dy = W.torch_normal((bt.m, lin.n), S(di), W.GRAD_STD, dev)
            if ff == bf:
                x_row, x_col = _quant_dual(ops, f"quant_{lin.name}_x_rowcol", x, ff, dev)
                w_row, w_col = _quant_dual(ops, f"quant_{lin.name}_w_rowcol", w, ff, dev)
            else:
                x_row, w_row = _empty_q(bt.m, lin.k, ff, "row", dev), _empty_q(lin.n, lin.k, ff, "row", dev)
                # NVFP4 backward copies take X's and W's amax from this launch
                amax_xw = torch.empty(2 * AMAX_WORDS, dtype=torch.float32, device=dev) if bf == "nvfp4" else None
                ops.append(Op("quant", lambda x=x, w=w, qa=x_row, qw=w_row, a=amax_xw:
                              api.mx_quantize_batch([x, w], ff, out=[qa, qw], amax=a), f"quant_{lin.name}_x_w",
                              nbytes=QUANT_BYTES[ff] * (x.numel() + w.numel())))
                x_col, w_col = None, None
            _gemm_op(ops, next(specs), x_row, w_row, bias, dev, ws)
            saved.append((lin, x, w, dy, x_col, w_col, amax_xw if ff != bf else None))
        for lin, x, w, dy, x_col, w_col, amax_xw in reversed(saved):  # backward
            if x_col is None:
                # the backward format's copies along the token / output axis
                x_col, w_col = _empty_q(bt.m, lin.k, bf, "col", dev), _empty_q(lin.n, lin.k, bf, "col", dev)
                if amax_xw is not None:
                    ops.append(Op("quant", lambda x=x, q=x_col, a=amax_xw[:AMAX_WORDS]:
                                  api.mx_quantize_amax(x, bf, "col", a, q.codes, q.scales),
                                  f"quant_{lin.name}_x_col", nbytes=QUANT_BYTES[bf] * x.numel()))
                    ops.append(Op("quant", lambda w=w, q=w_col, a=amax_xw[AMAX_WORDS:]:
                                  api.mx_quantize_amax(w, bf, "col", a, q.codes, q.scales),
                                  f"quant_{lin.name}_w_col", nbytes=QUANT_BYTES[bf] * w.numel()))
                else:
                    ops.append(Op("quant", lambda x=x, q=x_col: api.mx_quantize(x, bf, "col", q.codes, q.scales),
                                  f"quant_{lin.name}_x_col", nbytes=QUANT_BYTES[bf] * x.numel()))
                    ops.append(Op("quant", lambda w=w, q=w_col: api.mx_quantize(w, bf, "col", q.codes, q.scales),
                                  f"quant_{lin.name}_w_col", nbytes=QUANT_BYTES[bf] * w.numel()))
            dy_row, dy_col = _quant_dual(ops, f"quant_{lin.name}_dy_rowcol", dy, bf, dev, sr)
            _gemm_op(ops, next(specs), dy_row, w_col, None, dev, ws)   # dgrad: dX = dY W
            _gemm_op(ops, next(specs), dy_col, x_col, None, dev, ws)   # wgrad: dW = dY^T X
    return [ops]


def build(name, dev):
    """(step op lists, description) of a workload; the GEMMs built are checked
    against workload_gemms."""
    from block_scaled_precision_mx_amd import workloads as W
    if name in W.STACKS:
        wl = W.STACKS[name]
        sets = build_stack(wl, dev)
        config = {"workload": wl.name, "M": wl.m, "hidden": wl.hidden, "mlp": wl.mlp, "blocks": wl.blocks,
                  "tokens_per_image": W.TOKENS, "batch": wl.m // W.TOKENS, "format": wl.fmt,
                  "gemms_per_block": [f"{l.name} {l.n}x{l.k}" for l in wl.linears]}
        peak_key = wl.fmt
    elif name in W.TRAIN_PAIRS:
        wl = W.TRAIN_PAIRS[name]
        sets = build_train(wl, dev)
        config = {"workload": wl.name, "M": wl.m, "hidden": wl.hidden, "mlp": wl.mlp, "tokens_per_image": W.TOKENS,
                  "batch": wl.m // W.TOKENS, "format": wl.fmt, "gemms": "fc1/fc2 fprop+dgrad+wgrad",
                  "quantizations": "6 tensors, row and transposed copies from one read each",
                  "grad_rounding": "stochastic (Philox4x64-10)" if wl.sr_grads else "nearest-even",
                  "input_sets": TRAIN_SETS}
        peak_key = "fp16" if wl.fmt == "nvfp4" else wl.fmt
    else:
        wl = W.BLOCK_TRAINS[name]
        sets = build_block_train(wl, dev)
        config = {"workload": wl.name, "M": wl.m, "hidden": wl.hidden, "mlp": wl.mlp, "blocks": wl.blocks,
                  "tokens_per_image": W.TOKENS, "batch": wl.m // W.TOKENS, "fprop_format": wl.fwd_fmt,
                  "dgrad_wgrad_format": wl.bwd_fmt, "gemms_per_block": 12,
                  "grad_rounding": "stochastic (Philox4x64-10)" if wl.sr_grads else "nearest-even"}
        peak_key = "fp16" if wl.bwd_fmt == "nvfp4" else wl.fwd_fmt
    want = [(s.label, s.m, s.n, s.k, s.fmt) for s in workload_gemms(name)]
    for ops in sets:
        got = [(o.spec.label, o.spec.m, o.spec.n, o.spec.k, o.spec.fmt) for o in ops if o.kind == "gemm"]
        if got != want:
            raise RuntimeError(f"{name}: built GEMMs differ from workload_gemms")
    return sets, config, peak_key


# ------------------------------------------------------------------ timing

# host time allowed per launch while a replay's launches are enqueued, before
# the first replay has measured it
LEAD_US_PER_LAUNCH = 40.0


def measure(sets, steps, warmup, stream):
    """ms per step over `steps` timed steps (step s runs input set
    s % len(sets)), then the average duration of every launch, per label:
    each replay runs all launches of one label (every block's, every set's,
    each on its own tensors as in the step) back to back between one pair of
    HIP events on the stream the kernels run on, so that the events' own
    overhead is spread over many launches, after a spin that lets the host
    enqueue them all first (sized from the host time a first, untimed
    replay took); `steps` replays are averaged.
    Returns (ms per step, [(op, average ms)] for the ops of every set)."""
    import torch

    def step(s):
        for op in sets[s % len(sets)]:
            op.fn()

    for s in range(warmup):
        step(s)
    torch.cuda.synchronize()
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    t_start.record(stream)
    for s in range(steps):
        step(s)
    t_end.record(stream)
    torch.cuda.synchronize()
    ms_per_step = t_start.elapsed_time(t_end) / steps

    groups = {}
    for ops in sets:
        for op in ops:
            groups.setdefault(op.label, []).append(op)
    per_label = {lab: 0.0 for lab in groups}
    # the spin kernel counts the counter its clock read uses; its rate, once
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    torch.cuda._sleep(1_000_000)
    e1.record(stream)
    torch.cuda.synchronize()
    spin_per_us = 1.0e6 / max(e0.elapsed_time(e1) * 1.0e3, 1.0)
    # host microseconds per launch of each label, as the last replay took them
    host_us = {lab: LEAD_US_PER_LAUNCH for lab in groups}
    # the replays run back to back with no synchronization between them (a
    # GPU left idle by one runs the next replay's first labels slower: the
    # first two labels after a synchronization measured up to 2.5x their
    # kernels' own time in the trace); the events are read at the end
    events = []
    for rep in range(steps + 1):                # replay 0 only measures the host side
        ev = {lab: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for lab in groups}
        for lab, ops in groups.items():
            # a spin on the stream ahead of the start event keeps the GPU busy
            # while the host enqueues the label's launches (1.5 times the time
            # the host took last time), so the events time the kernels back to
            # back and not the host's launch rate
            torch.cuda._sleep(int(spin_per_us * 1.5 * host_us[lab] * len(ops)))
            ev[lab][0].record(stream)
            h0 = time.perf_counter()
            for op in ops:
                op.fn()
            host_us[lab] = max(LEAD_US_PER_LAUNCH, (time.perf_counter() - h0) * 1.0e6 / len(ops))
            ev[lab][1].record(stream)
        if rep > 0:
            events.append(ev)
    torch.cuda.synchronize()
    for ev in events:
        for lab, ops in groups.items():
            per_label[lab] += ev[lab][0].elapsed_time(ev[lab][1]) / len(ops)
    timed = [(op, per_label[op.label] / steps) for ops in sets for op in ops]
    return ms_per_step, timed, len(sets)


def summarize(timed, n_sets):
    """Per-label, per-kernel-configuration and quantization figures from the
    grouped replays. `timed` holds (op, average duration in ms) for the
    ops of all n_sets input sets; per-step figures divide by n_sets."""
    by_label, plans = {}, {}
    gemm_ms = quant_ms = quant_bytes = gemm_flops = 0.0
    for op, t in timed:
        d = by_label.setdefault(op.label, {"ms": 0.0, "n": 0, "flops": 0.0, "bytes": 0.0})
        d["ms"] += t
        d["n"] += 1
        d["flops"] += op.flops
        d["bytes"] += op.nbytes
        if op.kind == "gemm":
            gemm_ms += t
            gemm_flops += op.flops
            p = plans.setdefault(op.plan, {"ms": 0.0, "flops": 0.0, "n": 0})
            p["ms"] += t
            p["flops"] += op.flops
            p["n"] += 1
        else:
            quant_ms += t
            quant_bytes += op.nbytes
    breakdown = {}
    for lab, d in by_label.items():
        e = {"us_per_launch": round(1e3 * d["ms"] / d["n"], 2), "launches_per_step": d["n"] // n_sets}
        if d["flops"]:
            e["tflops"] = round(d["flops"] / (d["ms"] * 1e-3) / 1e12, 1)
        if d["bytes"]:
            e["gbps"] = round(d["bytes"] / (d["ms"] * 1e-3) / 1e9, 1)
        breakdown[lab] = e
    kernels = {p: {"launches_per_step": d["n"] // n_sets, "avg_launch_us": round(1e3 * d["ms"] / d["n"], 2),
                   "tflops": round(d["flops"] / (d["ms"] * 1e-3) / 1e12, 1), "ms_per_step": d["ms"] / n_sets,
                   "flops_per_launch_avg": d["flops"] / d["n"]} for p, d in plans.items()}
    quant = None
    if quant_ms:
        gbps = quant_bytes / (quant_ms * 1e-3) / 1e9
        quant = {"gbps": round(gbps, 1), "peak_gbps": PEAK_HBM_GBS, "frac": round(gbps / PEAK_HBM_GBS, 4),
                 "ms_per_step": round(quant_ms / n_sets, 4)}
    return {"breakdown": breakdown, "kernels": kernels, "quant": quant,
            "gemm_only_tflops": round(gemm_flops / (gemm_ms * 1e-3) / 1e12, 1)}


# ------------------------------------------------------------------ CPU oracle

def cpu_baseline(workload_name, fmt):
    """The oracle as it stands on a bounded sample of the same workload: the
    four linears of one ViT block at full M (one of the stack's blocks);
    returns GEMM TFLOP/s of quantize + dequantize + float64 GEMM."""
    from block_scaled_precision_mx_amd import workloads as W
    from oracle import gemm as G
    from oracle import quantize as Q

    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threads = 1
    stack = W.STACKS[workload_name]
    rows = stack.m
    gen = []
    for lin in stack.linears:
        a = (W.np_gelu_activation if lin.a_kind == "gelu" else W.np_activation)((rows, lin.k),
                                                                                W.seed(stack.wid, 0, lin.a_id))
        w = W.np_normal((lin.n, lin.k), W.seed(stack.wid, 0, lin.w_id), W.W_STD)
        b = W.np_normal((lin.n,), W.seed(stack.wid, 0, lin.bias_id), W.BIAS_STD)
        gen.append((a, w, b, lin.n, lin.k))
    t0 = time.perf_counter()
    flops = 0.0
    for a, w, b, n, k in gen:
        qa, qw = Q.quantize(a, fmt), Q.quantize(w, fmt)
        G.gemm_ref(qa, qw, b)
        flops += 2.0 * rows * n * k
    dt = time.perf_counter() - t0
    sample = (f"the {len(gen)} quantize+GEMMs of one block at full M ("
              + ", ".join(f"{rows}x{n}x{k}" for _, _, _, n, k in gen)
              + "); quantization single-threaded numpy, GEMMs float64 BLAS")
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": sample, "seconds": round(dt, 3), "host_cpus": os.cpu_count(),
            "blas_threads": threads}


# ------------------------------------------------------------------ traffic

# the sources a kernel's machine code is built from (its file and the device
# headers it includes); their hash ties a counter summary to one build
_CSRC = "block_scaled_precision_mx_amd/csrc/"
_DEVICE_HEADERS = [_CSRC + "gemm_common.h", _CSRC + "mx_device.h"]
KERNEL_SOURCES = {"gemm_mx_kernel": [_CSRC + "gemm_mx.hip"] + _DEVICE_HEADERS}


def source_sha256(kernel):
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kernel.split("<")[0]]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def library_sha256():
    """Hash of every source the library is built from (ties a record to a build)."""
    h = hashlib.sha256()
    files = sorted(os.listdir(os.path.join(ROOT, _CSRC)))
    for name in files + ["../../include/mx.h"]:
        p = os.path.join(ROOT, _CSRC, name)
        if os.path.isfile(p) and not name.endswith((".so", ".o")):
            with open(p, "rb") as f:
                h.update(f.read())
    return h.hexdigest()[:16]


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


# ------------------------------------------------------------------ roofline

# the matrix-core peak each GEMM kernel family is priced against (NVFP4 runs
# on the fp16 matrix instructions)
FAMILY_PEAK = {"gemm_mx_kernel<mxfp8>": "mxfp8", "gemm_mx_kernel<mxfp4>": "mxfp4", "gemm_mx_kernel<nvfp4>": "fp16"}


def kernel_families(kernels):
    """The GEMM kernel per operand format, over all its tile configurations
    (the planner picks one per shape: 'gemm_mx_kernel<mxfp8, 192x256>',
    '..., 192x256, l2pf>', '...>+splitk4' all belong to
    'gemm_mx_kernel<mxfp8>'): launches, time and flops per step summed, so
    that achieved = the family's flops over its time."""
    fam = {}
    for p, d in kernels.items():
        key = p.split(",")[0] + ">"
        f = fam.setdefault(key, {"launches_per_step": 0, "ms_per_step": 0.0, "flops": 0.0, "configurations": []})
        f["launches_per_step"] += d["launches_per_step"]
        f["ms_per_step"] += d["ms_per_step"]
        f["flops"] += d["flops_per_launch_avg"] * d["launches_per_step"]
        f["configurations"].append(p)
    for f in fam.values():
        f["avg_launch_us"] = 1e3 * f["ms_per_step"] / f["launches_per_step"]
        f["flops_per_launch_avg"] = f["flops"] / f["launches_per_step"]
        f["configurations"].sort()
    return fam


# ------------------------------------------------------------------ main

def run_workload(name, steps, warmup, dev):
    """Build, time and summarize one workload; frees its buffers afterwards."""
    import torch
    from block_scaled_precision_mx_amd import workloads as W
    sets, config, peak_key = build(name, dev)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ms_per_step, timed, n_sets = measure(sets, steps, warmup, stream)
    summ = summarize(timed, n_sets)
    flops = sum(op.flops for op in sets[0])
    fam = kernel_families(summ["kernels"])
    dom = max(fam, key=lambda k: fam[k]["ms_per_step"])
    d = fam[dom]
    achieved = d["flops_per_launch_avg"] / (d["avg_launch_us"] * 1e-6) / 1e12
    peak = PEAK_TFLOPS[FAMILY_PEAK[dom]]
    res = {"ms_per_step": ms_per_step, "value": flops / (ms_per_step * 1e-3) / 1e12, "config": config,
           "roofline": {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 1), "peak": peak,
                        "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                        "traffic": measured_traffic(dom, name), "launches_per_step": d["launches_per_step"],
                        "avg_launch_us": round(d["avg_launch_us"], 2), "flops_per_launch_avg": d["flops_per_launch_avg"],
                        "configurations": d["configurations"]},
           "summary": summ, "fmt": config.get("format", config.get("fprop_format"))}
    if name in W.BLOCK_TRAINS:
        res["us_per_block"] = round(1e3 * ms_per_step / W.BLOCK_TRAINS[name].blocks, 1)
    del sets, timed
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def compact(name, res):
    """The record of a configuration other than the headline."""
    s = res["summary"]
    out = {"ms_per_step": round(res["ms_per_step"], 4), "tflops": round(res["value"], 1),
           "gemm_only_tflops": s["gemm_only_tflops"],
           "roofline": {k: res["roofline"][k] for k in ("kernel", "achieved", "peak", "frac", "avg_launch_us",
                                                         "launches_per_step", "configurations")},
           "gemm_kernels": {p: {k: v for k, v in d.items() if k in ("launches_per_step", "avg_launch_us", "tflops")}
                            for p, d in s["kernels"].items()}}
    if s["quant"]:
        out["quant"] = s["quant"]
    if "us_per_block" in res:
        out["us_per_block"] = res["us_per_block"]
    if name in PAGES_CONTEXT:
        out["pages_context"] = PAGES_CONTEXT[name]
    return out


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: --gpus must be 1. The kernels here run one GPU's "
              "share of the work; nothing in this package uses a second GPU or a collective.",
              file=sys.stderr)
        sys.exit(2)
    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    if args.copy_probe_mb:
        n = args.copy_probe_mb * (1 << 20) // 2
        src = torch.empty(n, dtype=torch.bfloat16, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    res = run_workload(args.workload, args.steps, args.warmup, dev)
    print(f"[bench] {args.workload}: {res['ms_per_step']:.4f} ms/step", file=sys.stderr, flush=True)
    fmt = res["fmt"]
    summ = res["summary"]
    result = {
        "metric": "block-scaled GEMM TFLOP/s of the whole quantize-then-GEMM step on ViT-L shapes",
        "value": round(res["value"], 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(res["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8-e4m3" if fmt == "mxfp8" else ("fp4-e2m1+fp16-mfma" if fmt == "nvfp4" else "fp4-e2m1"),
        "data": "synthetic (seeded, device-generated bf16; no dataset or weights)",
        "config": res["config"],
        "roofline": res["roofline"],
        "gemm_kernels": {p: {k: v for k, v in d.items() if k in ("launches_per_step", "avg_launch_us", "tflops")}
                         for p, d in summ["kernels"].items()},
        "gemm_only_tflops": summ["gemm_only_tflops"],
        "quant": summ["quant"],
        "breakdown": summ["breakdown"],
        "library_sha256": library_sha256(),
    }
    if not args.only:
        configs = {}
        for name in EXTRA_CONFIGS:
            if name == args.workload:
                continue
            r = run_workload(name, min(args.steps, 10), min(args.warmup, 2), dev)
            print(f"[bench] {name}: {r['ms_per_step']:.4f} ms/step", file=sys.stderr, flush=True)
            configs[name] = compact(name, r)
        result["configs"] = configs
    if not args.no_cpu_baseline and args.workload in __import__(
            "block_scaled_precision_mx_amd.workloads", fromlist=["STACKS"]).STACKS:
        result["cpu_baseline"] = cpu_baseline(args.workload, fmt)
    print(json.dumps(result))


if __name__ == "__main__":
    main()
