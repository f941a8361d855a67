"""GPU parity of mx_gemm against the oracle's exact dequantized GEMM.

Every output must satisfy the acceptance rule |C - C_ref| <= 2^-12 S
(S = sum |a b| + |bias|), applied before the final bf16 rounding. Cases with
unit scales and small-integer codes have an exactly representable result,
so the fp32 output must equal it exactly: they pin the lane / K / scale-byte
mapping of the matrix instructions. Full ViT shapes are checked on sampled
outputs in the launch configuration the benchmark uses."""
import numpy as np
import pytest
import torch

from block_scaled_precision_mx_amd import api
from block_scaled_precision_mx_amd import workloads as W
from oracle import formats as F
from oracle import gemm as G
from oracle import quantize as Q
from gpu_util import f64_of, log, to_device_bf16

pytestmark = pytest.mark.gpu
FMTS = ["mxfp8", "mxfp4", "nvfp4"]


def run_gpu(a_bits, b_bits, fmt, bias_bits=None, out_dtype="bf16", a_axis="row", b_axis="row"):
    a = api.mx_quantize(to_device_bf16(a_bits), fmt, a_axis)
    b = api.mx_quantize(to_device_bf16(b_bits), fmt, b_axis)
    bias = None if bias_bits is None else to_device_bf16(bias_bits.reshape(1, -1)).reshape(-1)
    return f64_of(api.mx_gemm(a, b, bias, out_dtype))


def check_full(a_bits, b_bits, fmt, bias_bits=None, out_dtype="bf16", a_axis="row", b_axis="row"):
    log(f"gemm fmt={fmt} A{a_bits.shape}/{a_axis} B{b_bits.shape}/{b_axis} bias={bias_bits is not None} out={out_dtype}")
    got = run_gpu(a_bits, b_bits, fmt, bias_bits, out_dtype, a_axis, b_axis)
    qa, qb = Q.quantize(a_bits, fmt, a_axis), Q.quantize(b_bits, fmt, b_axis)
    c, s = G.gemm_ref(qa, qb, bias_bits)
    ok = G.accept(got, c, s, out_dtype)
    bad = np.argwhere(~ok)
    assert bad.size == 0, f"{len(bad)} outside the bound, e.g. {[(tuple(i), got[tuple(i)], c[tuple(i)]) for i in bad[:3]]}"
    return got, c, s


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("mnk", [(1, 1, 1), (1, 1, 32), (3, 5, 99), (17, 33, 129), (128, 128, 128),
                                 (130, 260, 384), (300, 200, 1000), (513, 257, 640)])
@pytest.mark.parametrize("out_dtype", ["bf16", "f32"])
def test_gemm_random(fmt, mnk, out_dtype):
    m, n, k = mnk
    a = W.np_activation((m, k), seed=m + 7 * k)
    b = W.np_normal((n, k), seed=n + 11 * k, std=W.W_STD)
    bias = W.np_normal((n,), seed=n, std=W.BIAS_STD)
    check_full(a, b, fmt, bias if m % 2 else None, out_dtype)


@pytest.mark.parametrize("fmt", FMTS)
def test_gemm_single_layer_config(fmt):
    """The single-layer workload: A 256x768 activations, B 768x768 weights, bias."""
    wl = W.SINGLE_LAYER
    lin = wl.linears[0]
    a = W.np_activation((wl.m, lin.k), W.seed(wl.wid, 0, lin.a_id))
    b = W.np_normal((lin.n, lin.k), W.seed(wl.wid, 0, lin.w_id), W.W_STD)
    bias = W.np_normal((lin.n,), W.seed(wl.wid, 0, lin.bias_id), W.BIAS_STD)
    for out_dtype in ("bf16", "f32"):
        check_full(a, b, fmt, bias, out_dtype)


def exact_operand(rows, k, fmt, rng, big_block=0):
    """Inputs whose quantization is exact with unit (MX) or known scales:
    small grid values, every block holding one maximal element. For NVFP4 the
    tensor scale is pinned to 1 by a lone 2688 in block `big_block` of row 0
    (A and B use different blocks, so no product of two 2688s appears)."""
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6.0])
    x = rng.choice(grid, (rows, k)) * rng.choice([-1.0, 1.0], (rows, k))
    bs = Q.block_size(fmt)
    x[:, ::bs] = 6.0 if fmt != "mxfp8" else 448.0 / 64   # E2M1: block max 6 -> e=0; E4M3: 7 -> e=-6
    if fmt == "nvfp4":
        x[0, big_block * bs:(big_block + 1) * bs] = 0.0
        x[0, big_block * bs] = 2688.0          # s_t = 1
    return W.to_bf16_bits(x)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("mnk", [(16, 16, 128), (64, 48, 512), (200, 136, 1024), (256, 512, 4096)])
def test_gemm_integer_exact(fmt, mnk):
    """Quantization is exact and every partial sum is a multiple of 2^-12 far
    below 2^24 ulps, so fp32 accumulation in any order gives the exact value."""
    m, n, k = mnk
    rng = np.random.default_rng(m * n + k)
    a, b = exact_operand(m, k, fmt, rng, 0), exact_operand(n, k, fmt, rng, 1)
    qa, qb = Q.quantize(a, fmt), Q.quantize(b, fmt)
    assert np.array_equal(qa.dequantize(), F.bf16_to_f64(a))
    log(f"gemm exact fmt={fmt} {mnk}")
    got = run_gpu(a, b, fmt, None, "f32")
    want = F.bf16_to_f64(a) @ F.bf16_to_f64(b).T
    assert np.array_equal(got, want), np.argwhere(got != want)[:5].tolist()


@pytest.mark.parametrize("fmt", FMTS)
def test_gemm_scale_shift(fmt):
    """Scaling A by 2^5 scales the (bias-free, fp32) GPU result by exactly 2^5."""
    a = W.np_activation((96, 256), seed=5)
    b = W.np_normal((80, 256), seed=6, std=W.W_STD)
    log(f"gemm scale shift {fmt}")
    c0 = run_gpu(a, b, fmt, None, "f32")
    c5 = run_gpu(W.to_bf16_bits(F.bf16_to_f64(a) * 32.0), b, fmt, None, "f32")
    assert np.array_equal(c5, c0 * 32.0)


@pytest.mark.parametrize("fmt", FMTS)
def test_gemm_training_operands(fmt):
    """dgrad and wgrad operands come from column quantization (TN layout);
    m = 300 tokens is a ragged K for wgrad (K_pad 384)."""
    m, h, f = 300, 96, 160
    x = W.np_activation((m, h), seed=1)
    dy = W.np_normal((m, f), seed=2, std=W.GRAD_STD)
    w = W.np_normal((f, h), seed=3, std=W.W_STD)
    # dgrad: dX[m, h] = dY[m, f] * W[f, h]  -> A = dY (row), B = W^T (col of W)
    check_full(dy, w, fmt, None, "bf16", "row", "col")
    # wgrad: dW[f, h] = dY^T * X            -> A = dY^T (col), B = X^T (col)
    check_full(dy, x, fmt, None, "bf16", "col", "col")


def sampled_check(a_bits, b_bits, fmt, bias_bits, a_axis="row", b_axis="row", n_samples=4000, seed=0):
    log(f"gemm full-size fmt={fmt} A{a_bits.shape}/{a_axis} B{b_bits.shape}/{b_axis}")
    got = run_gpu(a_bits, b_bits, fmt, bias_bits, "bf16", a_axis, b_axis)
    qa, qb = Q.quantize(a_bits, fmt, a_axis), Q.quantize(b_bits, fmt, b_axis)
    rng = np.random.default_rng(seed)
    rows = rng.integers(0, qa.rows, n_samples)
    cols = rng.integers(0, qb.rows, n_samples)
    # include the last tile's corners
    rows[:4] = [qa.rows - 1, qa.rows - 1, 0, qa.rows - 1]
    cols[:4] = [qb.rows - 1, 0, qb.rows - 1, qb.rows // 2]
    c, s = G.gemm_ref_entries(qa, qb, rows, cols, bias_bits)
    ok = G.accept(got[rows, cols], c, s, "bf16")
    assert ok.all(), f"{(~ok).sum()} of {n_samples} sampled outputs outside the bound"
    assert np.isfinite(got).all()


@pytest.mark.parametrize("fmt,lin", [
    ("mxfp8", "qkv"), ("mxfp8", "fc2"), ("mxfp4", "fc1"), ("mxfp4", "proj"),
])
def test_gemm_vitl_full_size(fmt, lin):
    wl = W.VITL_MXFP8 if fmt == "mxfp8" else W.VITL_MXFP4
    L = {l.name: l for l in wl.linears}[lin]
    a = (W.np_gelu_activation if L.a_kind == "gelu" else W.np_activation)((wl.m, L.k), W.seed(wl.wid, 0, L.a_id))
    b = W.np_normal((L.n, L.k), W.seed(wl.wid, 0, L.w_id), W.W_STD)
    bias = W.np_normal((L.n,), W.seed(wl.wid, 0, L.bias_id), W.BIAS_STD)
    sampled_check(a, b, fmt, bias)


def test_gemm_vitb_fc1_full_size():
    wl = W.VITB_MXFP8
    L = wl.linears[2]
    a = W.np_activation((wl.m, L.k), W.seed(wl.wid, 0, L.a_id))
    b = W.np_normal((L.n, L.k), W.seed(wl.wid, 0, L.w_id), W.W_STD)
    bias = W.np_normal((L.n,), W.seed(wl.wid, 0, L.bias_id), W.BIAS_STD)
    sampled_check(a, b, "mxfp8", bias)


@pytest.mark.parametrize("which", ["fprop_fc1", "dgrad_fc2", "wgrad_fc1"])
def test_gemm_nvfp4_training_full_size(which):
    tp = W.TRAIN_PAIR
    if which == "fprop_fc1":
        a = W.np_activation((tp.m, tp.hidden), W.seed(tp.wid, 0, tp.X))
        b = W.np_normal((tp.mlp, tp.hidden), W.seed(tp.wid, 0, tp.W1), W.W_STD)
        bias = W.np_normal((tp.mlp,), W.seed(tp.wid, 0, tp.B1), W.BIAS_STD)
        sampled_check(a, b, "nvfp4", bias)
    elif which == "dgrad_fc2":
        dy2 = W.np_normal((tp.m, tp.hidden), W.seed(tp.wid, 0, tp.DY2), W.GRAD_STD)
        w2 = W.np_normal((tp.hidden, tp.mlp), W.seed(tp.wid, 0, tp.W2), W.W_STD)
        sampled_check(dy2, w2, "nvfp4", None, "row", "col")
    else:
        dy1 = W.np_normal((tp.m, tp.mlp), W.seed(tp.wid, 0, tp.DY1), W.GRAD_STD)
        x = W.np_activation((tp.m, tp.hidden), W.seed(tp.wid, 0, tp.X))
        sampled_check(dy1, x, "nvfp4", None, "col", "col")


@pytest.mark.parametrize("which", ["fprop_fc2", "dgrad_fc1", "wgrad_fc2"])
def test_gemm_mxfp8_training_full_size(which):
    """The MXFP8 training pair at full size, in the benchmark's launch
    configuration: wgrad contracts over the 11235 tokens (K_pad 11264)."""
    tp = W.TRAIN_PAIR_MXFP8
    S = lambda tid: W.seed(tp.wid, 0, tid)   # noqa: E731
    if which == "fprop_fc2":
        h = W.np_gelu_activation((tp.m, tp.mlp), S(tp.H))
        w2 = W.np_normal((tp.hidden, tp.mlp), S(tp.W2), W.W_STD)
        b2 = W.np_normal((tp.hidden,), S(tp.B2), W.BIAS_STD)
        sampled_check(h, w2, "mxfp8", b2)
    elif which == "dgrad_fc1":
        dy1 = W.np_normal((tp.m, tp.mlp), S(tp.DY1), W.GRAD_STD)
        w1 = W.np_normal((tp.mlp, tp.hidden), S(tp.W1), W.W_STD)
        sampled_check(dy1, w1, "mxfp8", None, "row", "col")
    else:
        dy2 = W.np_normal((tp.m, tp.hidden), S(tp.DY2), W.GRAD_STD)
        h = W.np_gelu_activation((tp.m, tp.mlp), S(tp.H))
        sampled_check(dy2, h, "mxfp8", None, "col", "col")


@pytest.mark.parametrize("fmt,k", [("mxfp8", 128), ("mxfp8", 384), ("mxfp4", 384), ("mxfp4", 640)])
def test_gemm_many_tiles_full(fmt, k):
    """More output tiles than resident workgroups (ragged M), every output
    checked: workgroups walk several tiles with the next tile's first K-stage
    in flight across the boundary and the previous tile's stores pending.
    K = 128 (fp8) is a single stage per tile; K = 384 / 640 (fp4) end on a
    half stage."""
    m, n = 4160, 4096
    a = W.np_activation((m, k), seed=91 + k)
    b = W.np_normal((n, k), seed=92 + k, std=W.W_STD)
    bias = W.np_normal((n,), seed=93, std=W.BIAS_STD)
    log(f"gemm many tiles plan={api.gemm_plan(m, n, k, fmt)}")
    check_full(a, b, fmt, bias, "bf16")


@pytest.mark.parametrize("mnk,plan", [
    ((1000, 1000, 512), "128x128"),     # few tiles: two 4-wave workgroups per CU
    ((4160, 4096, 384), "192x256"),     # more tiles than workgroups, ragged M
    ((2048, 8192, 256), "128x128"),     # two rounds of 128x128 workgroups, every slot walks 2 tiles
])
def test_gemm_nvfp4_tile_shapes(mnk, plan):
    """Each NVFP4 tile shape the host can choose, every output checked."""
    m, n, k = mnk
    assert api.gemm_plan(m, n, k, "nvfp4").endswith(plan + ">")
    a = W.np_activation((m, k), seed=71 + k)
    b = W.np_normal((n, k), seed=72 + k, std=W.W_STD)
    bias = W.np_normal((n,), seed=73, std=W.BIAS_STD)
    log(f"gemm nvfp4 plan={api.gemm_plan(m, n, k, 'nvfp4')} m={m} n={n} k={k}")
    check_full(a, b, "nvfp4", bias, "bf16")


@pytest.mark.parametrize("fmt", FMTS)
def test_gemm_bias_2byte_aligned(fmt):
    """A bias pointer that is only 2-byte aligned (a view at element offset 1)
    takes the kernel's element-wise bias path; the result must not change."""
    m, n, k = 520, 1024, 256
    a = W.np_activation((m, k), seed=31)
    b = W.np_normal((n, k), seed=32, std=W.W_STD)
    bias = W.np_normal((n,), seed=33, std=W.BIAS_STD)
    qa = api.mx_quantize(to_device_bf16(a), fmt, "row")
    qb = api.mx_quantize(to_device_bf16(b), fmt, "row")
    padded = np.zeros(n + 1, dtype=np.uint16)
    padded[1:] = bias
    dev_bias = to_device_bf16(padded.reshape(1, -1)).reshape(-1)
    aligned = dev_bias[1:].clone()
    offset = dev_bias[1:]
    assert offset.data_ptr() % 16 == 2
    log(f"gemm bias alignment fmt={fmt}")
    got_offset = f64_of(api.mx_gemm(qa, qb, offset, "bf16"))
    got_aligned = f64_of(api.mx_gemm(qa, qb, aligned, "bf16"))
    assert np.array_equal(got_offset, got_aligned)
    c, s = G.gemm_ref(Q.quantize(a, fmt), Q.quantize(b, fmt), bias)
    assert G.accept(got_offset, c, s, "bf16").all()
