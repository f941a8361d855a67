"""GPU parity of mx_gemm_ws, the GEMM that may split K over a workspace (the
weight-gradient GEMMs contract over the 11235 tokens; lightly-train README
"DINOv3 + EoMT on RTX 5090", sections 5.4 and 5.5).

Every output is checked against the oracle's rule (2^-12 S, plus the MXFP8
matrix instruction's adder term where needed) for problems whose plan splits
K, in every format: split counts that leave ragged stage ranges, bias added
once after the partial sums, fp32 output, N % 8 != 0 (the element-wise
reduction), and a workspace too small for the preferred split. The
workspace is guarded by canary bytes: nothing may be written past the
S M N fp32 partials. At full size the training workloads' weight-gradient
GEMMs are checked on sampled outputs with the workspace the benchmark gives
them."""
import numpy as np
import pytest

import bench
from block_scaled_precision_mx_amd import api
from block_scaled_precision_mx_amd import workloads as W
from oracle import gemm as G
from oracle import quantize as Q
from gpu_util import Guarded, f64_of, log, quantize_guarded, to_device_bf16

pytestmark = pytest.mark.gpu

# every output: (M, N, K, fmt, out, bias)
SPLIT_FULL = [
    (1024, 1024, 11235, "mxfp8", "bf16", True),
    (1024, 1024, 11235, "mxfp4", "bf16", True),
    (1024, 1024, 11235, "nvfp4", "bf16", True),
    (1024, 1001, 11235, "mxfp8", "f32", True),     # N % 8 != 0: element-wise reduction
    (1024, 1001, 11235, "nvfp4", "bf16", False),
    (300, 260, 7000, "mxfp8", "bf16", True),        # 11 / 7 / 14 splits: ragged stage ranges
    (300, 260, 7000, "mxfp4", "f32", False),
    (300, 260, 7000, "nvfp4", "bf16", True),
    (3072, 1024, 11235, "mxfp8", "bf16", False),   # the large tile, split
    (3072, 1024, 11235, "nvfp4", "bf16", False),
    (4096, 1024, 11235, "mxfp8", "bf16", False),   # fc1's and fc2's weight gradients, every output
    (1024, 4096, 11235, "mxfp8", "bf16", False),
    (4096, 1024, 11235, "nvfp4", "bf16", False),   # NVFP4: 128x256 tiles, 2 splits (half: 128x128 unsplit)
    (1024, 4096, 11235, "nvfp4", "bf16", True),
    (1000, 770, 9000, "nvfp4", "f32", True),       # 128x256 in 8 ragged splits, ragged M and N (half: 128x128)
    (1234, 2050, 9999, "nvfp4", "bf16", False),    # 192x256 in 4 splits (half: 128x256 in 2)
]
_ORACLE = {}   # (M, N, K, fmt, bias) -> (inputs, quantized operands, reference): shared by both workspace sizes
# the weight-gradient GEMMs of the training workloads, with the benchmark's
# workspace: (workload, GEMM label)
WGRAD = [(name, s.label) for name in ("vitl16_mxfp8_block_train", "vitl16_p3_block_train", "vitl16_nvfp4_fc1fc2_train",
                                      "vitl16_mxfp8_fc1fc2_train")
         for s in bench.workload_gemms(name)[:12] if s.label.endswith("wgrad")]


def parity_cases():
    """(M, N, K, fmt, out, epilogue, workspace bytes) of every mx_gemm_ws this module runs."""
    cases = []
    for (m, n, k, fmt, out, _) in SPLIT_FULL:
        ws = api.gemm_workspace_bytes(m, n, k, fmt)
        cases += [(m, n, k, fmt, out, "c", ws), (m, n, k, fmt, out, "c", ws // 2)]
    for name, label in WGRAD:
        s = next(s for s in bench.workload_gemms(name) if s.label == label)
        cases.append((s.m, s.n, s.k, s.fmt, "bf16", "c", bench.WORKSPACE_BYTES))
    return cases


def run_ws(a, b, fmt, bias_bits, out_dtype, ws_bytes, a_axis="row", b_axis="row"):
    """mx_gemm_ws into a guarded C with a guarded workspace of ws_bytes."""
    qa = quantize_guarded(to_device_bf16(a), fmt, a_axis)
    qb = quantize_guarded(to_device_bf16(b), fmt, b_axis)
    bias = None if bias_bits is None else to_device_bf16(bias_bits.reshape(1, -1)).reshape(-1)
    M, N = qa.rows, qb.rows
    gws = Guarded(ws_bytes)
    gc = Guarded(M * N * (2 if out_dtype == "bf16" else 4))
    import torch
    out = gc.typed(torch.bfloat16 if out_dtype == "bf16" else torch.float32, (M, N))
    api.mx_gemm_ws(qa, qb, bias, out_dtype, gws.view if ws_bytes else None, out)
    gws.check("workspace")
    gc.check("C")
    return f64_of(out)


def check_every_output(got, qa, qb, bias_bits, out_dtype, ref=None):
    c, s = G.gemm_ref(qa, qb, bias_bits) if ref is None else ref
    ok = G.accept(got, c, s, out_dtype)
    if qa.fmt == "mxfp8" and not ok.all():
        r, q = np.nonzero(~ok)
        log(f"{r.size} outputs beyond 2^-12 S; checked with the adder term")
        ok[r, q] = G.accept(got[r, q], c[r, q], s[r, q], out_dtype, G.mxfp8_group_term(qa, qb, r, q))
    bad = np.argwhere(~ok)
    assert bad.size == 0, f"{len(bad)} outside the bound, e.g. {[(tuple(i), got[tuple(i)], c[tuple(i)]) for i in bad[:3]]}"


@pytest.mark.parametrize("ws_part", ["full", "half"])
@pytest.mark.parametrize("m,n,k,fmt,out_dtype,with_bias", SPLIT_FULL)
def test_gemm_ws_every_output(m, n, k, fmt, out_dtype, with_bias, ws_part):
    need = api.gemm_workspace_bytes(m, n, k, fmt)
    assert need > 0, "the case must split K"
    ws = need if ws_part == "full" else need // 2
    plan = api.gemm_ws_plan(m, n, k, fmt, ws)
    log(f"gemm_ws plan={plan} m={m} n={n} k={k} fmt={fmt} out={out_dtype} ws={ws}")
    if ws_part == "full":
        assert "+splitk" in plan
    key = (m, n, k, fmt, with_bias)
    if key not in _ORACLE:
        a = W.np_activation((m, k), seed=m + k)
        b = W.np_normal((n, k), seed=n + k, std=W.W_STD)
        bias = W.np_normal((n,), seed=n, std=W.BIAS_STD) if with_bias else None
        qa, qb = Q.quantize(a, fmt), Q.quantize(b, fmt)
        _ORACLE.clear()
        _ORACLE[key] = (a, b, bias, qa, qb, G.gemm_ref(qa, qb, bias))
    a, b, bias, qa, qb, ref = _ORACLE[key]
    got = run_ws(a, b, fmt, bias, out_dtype, ws)
    check_every_output(got, qa, qb, bias, out_dtype, ref)


@pytest.mark.parametrize("name,label", WGRAD)
def test_gemm_ws_training_wgrad_full_size(name, label):
    """A weight-gradient GEMM of a training workload at full size (K = 11235
    tokens, K_pad 11264), through mx_gemm_ws with the benchmark's workspace:
    A = dY^T and B = X^T, both column-quantized; sampled outputs and the
    corners of the first and last tile."""
    spec = next(s for s in bench.workload_gemms(name) if s.label == label)
    lin = label.split("_")[1]
    if name in W.BLOCK_TRAINS:
        bt = W.BLOCK_TRAINS[name]
        i = [l.name for l in bt.linears()].index(lin)
        L = bt.linears()[i]
        xi, _, _, di = bt.ids(i)
        S = lambda tid: W.seed(bt.wid, 0, tid)   # noqa: E731
        dy = W.np_normal((bt.m, L.n), S(di), W.GRAD_STD)
        x = (W.np_gelu_activation if L.a_kind == "gelu" else W.np_activation)((bt.m, L.k), S(xi))
    else:
        tp = W.TRAIN_PAIRS[name]
        S = lambda tid: W.seed(tp.wid, 0, tid)   # noqa: E731
        if lin == "fc1":
            dy, x = W.np_normal((tp.m, tp.mlp), S(tp.DY1), W.GRAD_STD), W.np_activation((tp.m, tp.hidden), S(tp.X))
        else:
            dy, x = W.np_normal((tp.m, tp.hidden), S(tp.DY2), W.GRAD_STD), W.np_gelu_activation((tp.m, tp.mlp), S(tp.H))
    assert (dy.shape[1], x.shape[1], dy.shape[0]) == (spec.m, spec.n, spec.k)
    plan = api.gemm_ws_plan(spec.m, spec.n, spec.k, spec.fmt, bench.WORKSPACE_BYTES)
    log(f"gemm_ws full-size {name} {label} plan={plan}")
    got = run_ws(dy, x, spec.fmt, None, "bf16", bench.WORKSPACE_BYTES, "col", "col")
    qa, qb = Q.quantize(dy, spec.fmt, "col"), Q.quantize(x, spec.fmt, "col")
    rng = np.random.default_rng(7)
    rows = rng.integers(0, qa.rows, 3000)
    cols = rng.integers(0, qb.rows, 3000)
    rows[:6] = [qa.rows - 1, qa.rows - 1, 0, qa.rows - 1, 0, qa.rows // 2]
    cols[:6] = [qb.rows - 1, 0, qb.rows - 1, qb.rows // 2, 0, qb.rows - 1]
    c, s = G.gemm_ref_entries(qa, qb, rows, cols)
    ok = G.accept_entries(got[rows, cols], c, s, "bf16", qa, qb, rows, cols)
    assert ok.all(), f"{(~ok).sum()} of {rows.size} sampled outputs outside the bound"
    assert np.isfinite(got).all()
