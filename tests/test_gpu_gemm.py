"""GPU parity of mx_gemm against the oracle's exact dequantized GEMM.

Every output must satisfy the acceptance rule |C - C_ref| <= 2^-12 S
(S = sum |a b| + |bias|), applied before the final bf16 rounding; for MXFP8
the matrix instruction's adder term H (oracle.gemm.mxfp8_group_term) is
added where 2^-12 S alone rejects. Cases with
unit scales and small-integer codes have an exactly representable result,
so the fp32 output must equal it exactly: they pin the lane / K / scale-byte
mapping of the matrix instructions. Full ViT shapes are checked on sampled
outputs (the last tile's corners included) with the kernel configuration
the benchmark launches for them; every kernel configuration is also checked
on every output of a problem with more tiles than resident workgroups.

Every C buffer is guarded by canary bytes on both sides (gpu_util.Guarded).
The case tables below are module-level so that a CPU test can check that
every kernel configuration the benchmark launches is exercised here."""
import numpy as np
import pytest

from block_scaled_precision_mx_amd import api
from block_scaled_precision_mx_amd import workloads as W
from oracle import formats as F
from oracle import gemm as G
from oracle import quantize as Q
from gpu_util import f64_of, gemm_guarded, log, quantize_guarded, to_device_bf16

pytestmark = pytest.mark.gpu
FMTS = ["mxfp8", "mxfp4", "nvfp4"]

# ---------------------------------------------------------------- case tables
# (M, N, K) of test_gemm_random, run for every format and both output dtypes
RANDOM_MNK = [(1, 1, 1), (1, 1, 32), (3, 5, 99), (17, 33, 129), (128, 128, 128), (130, 260, 384), (300, 200, 1000),
              (513, 257, 640)]
# (M, N, K) of test_gemm_integer_exact (fp32 out, every format)
INTEGER_MNK = [(16, 16, 128), (64, 48, 512), (200, 136, 1024), (256, 512, 4096)]
# every output of problems with more tiles than resident workgroups:
# (M, N, K, fmt, out, expected tile)
MANY_TILES = [
    (4160, 4096, 128, "mxfp8", "bf16", "192x256"),   # one K-stage per tile
    (4160, 4096, 384, "mxfp8", "bf16", "192x256"),
    (4160, 4096, 384, "mxfp4", "bf16", "192x256"),   # fp4 ends on a half stage
    (4160, 4096, 640, "mxfp4", "bf16", "192x256"),
    (8000, 4096, 256, "mxfp8", "bf16", "256x256"),   # two tiles per workgroup, ragged M
    (8000, 4096, 256, "mxfp4", "bf16", "256x256"),
    (8000, 4000, 384, "mxfp8", "bf16", "256x256"),   # ragged M and N
    (8000, 4000, 640, "mxfp4", "bf16", "256x256"),
    (6000, 4104, 128, "mxfp8", "f32", "256x256"),    # fp32 out: stored from registers
    (8000, 4001, 256, "mxfp4", "bf16", "256x256"),   # N % 8 != 0: element stores
    (4160, 4096, 384, "mxfp8", "f32", "192x256"),    # register epilogue between tiles
    (4160, 4092, 384, "mxfp4", "bf16", "192x256"),
    (1000, 1000, 512, "mxfp8", "f32", "128x128"),    # two 4-wave workgroups per CU (the MX
    (1000, 1000, 512, "mxfp4", "bf16", "128x128"),   # small tile never walks a second tile)
    (1000, 1000, 512, "nvfp4", "bf16", "128x128"),   # few tiles: two 4-wave workgroups per CU
    (4160, 4096, 384, "nvfp4", "bf16", "192x256"),
    (2048, 8192, 256, "nvfp4", "bf16", "128x128"),   # every slot walks 2 tiles
    (4160, 4096, 4200, "mxfp8", "bf16", "192x256, l2pf"),   # >= 32 stages: L2 prefetch, ragged M and K
    (4160, 4040, 384, "mxfp8", "bf16", "192x256"),   # N % 64 != 0: per-wave 128-byte row segments cut at N
    (4160, 4040, 384, "nvfp4", "bf16", "192x256"),   # per-wave 256-byte row segments cut at N
]
# forward linears of the stacks at full size, sampled outputs: (workload, linear)
FULL_SIZE_FWD = [(wl, lin) for wl in ("vitl16_mxfp8_fwd_stack", "vitl16_mxfp4_fwd_stack", "vitb16_mxfp8_fwd_stack")
                 for lin in ("qkv", "proj", "fc1", "fc2")]
# training GEMMs at full size, sampled outputs: (training workload, GEMM)
TRAIN_GEMMS = ["fc1_fprop", "fc1_dgrad", "fc1_wgrad", "fc2_fprop", "fc2_dgrad", "fc2_wgrad"]
FULL_SIZE_TRAIN = [(tp, g) for tp in ("vitl16_nvfp4_fc1fc2_train", "vitl16_mxfp8_fc1fc2_train") for g in TRAIN_GEMMS]
# the backward GEMMs of a whole ViT-L block that the fc1/fc2 pair does not
# have (qkv's and proj's dgrad and wgrad), in both backward formats:
# (block-training workload, linear, GEMM)
FULL_SIZE_BLOCK = [(bt, lin, g) for bt in ("vitl16_mxfp8_block_train", "vitl16_p3_block_train")
                   for lin in ("qkv", "proj") for g in ("dgrad", "wgrad")]


def train_gemm_shape(tp, which):
    """(M, N, K, a_axis, b_axis, has_bias) of one fc1/fc2 training GEMM."""
    lin, kind = which.split("_")
    n_out, k_in = (tp.mlp, tp.hidden) if lin == "fc1" else (tp.hidden, tp.mlp)
    if kind == "fprop":      # Y = X W^T + b
        return tp.m, n_out, k_in, "row", "row", True
    if kind == "dgrad":      # dX = dY W          -> A = dY (row), B = W^T (col of W)
        return tp.m, k_in, n_out, "row", "col", False
    return n_out, k_in, tp.m, "col", "col", False   # dW = dY^T X -> A = dY^T, B = X^T


def parity_cases():
    """(M, N, K, fmt, out, epilogue) of every mx_gemm this module runs."""
    cases = []
    for fmt in FMTS:
        cases += [(m, n, k, fmt, o, "c") for (m, n, k) in RANDOM_MNK for o in ("bf16", "f32")]
        cases += [(m, n, k, fmt, "f32", "c") for (m, n, k) in INTEGER_MNK]
        cases += [(256, 768, 768, fmt, o, "c") for o in ("bf16", "f32")]
    cases += [(m, n, k, fmt, o, "c") for (m, n, k, fmt, o, _) in MANY_TILES]
    for wname, lin in FULL_SIZE_FWD:
        wl = W.STACKS[wname]
        L = {l.name: l for l in wl.linears}[lin]
        cases.append((wl.m, L.n, L.k, wl.fmt, "bf16", "c"))
    for tname, which in FULL_SIZE_TRAIN:
        tp = W.TRAIN_PAIRS[tname]
        m, n, k = train_gemm_shape(tp, which)[:3]
        cases.append((m, n, k, tp.fmt, "bf16", "c"))
    for bname, lin, which in FULL_SIZE_BLOCK:
        bt = W.BLOCK_TRAINS[bname]
        m, n, k = block_gemm_shape(bt, lin, which)[:3]
        cases.append((m, n, k, bt.bwd_fmt, "bf16", "c"))
    return cases


def block_gemm_shape(bt, lin_name, which):
    """(M, N, K, a_axis, b_axis) of a backward GEMM of a block-training workload."""
    L = {l.name: l for l in bt.linears()}[lin_name]
    if which == "dgrad":     # dX[M, K_L] = dY[M, N_L] W[N_L, K_L]
        return bt.m, L.k, L.n, "row", "col"
    return L.n, L.k, bt.m, "col", "col"             # dW[N_L, K_L] = dY^T X


# ---------------------------------------------------------------- helpers

def run_gpu(a_bits, b_bits, fmt, bias_bits=None, out_dtype="bf16", a_axis="row", b_axis="row"):
    a = quantize_guarded(to_device_bf16(a_bits), fmt, a_axis)
    b = quantize_guarded(to_device_bf16(b_bits), fmt, b_axis)
    bias = None if bias_bits is None else to_device_bf16(bias_bits.reshape(1, -1)).reshape(-1)
    return f64_of(gemm_guarded(a, b, bias, out_dtype))


def check_full(a_bits, b_bits, fmt, bias_bits=None, out_dtype="bf16", a_axis="row", b_axis="row"):
    log(f"gemm fmt={fmt} A{a_bits.shape}/{a_axis} B{b_bits.shape}/{b_axis} bias={bias_bits is not None} out={out_dtype}")
    got = run_gpu(a_bits, b_bits, fmt, bias_bits, out_dtype, a_axis, b_axis)
    qa, qb = Q.quantize(a_bits, fmt, a_axis), Q.quantize(b_bits, fmt, b_axis)
    c, s = G.gemm_ref(qa, qb, bias_bits)
    ok = G.accept(got, c, s, out_dtype)
    if fmt == "mxfp8" and not ok.all():
        # the MXFP8 matrix instruction's adder term, where 2^-12 S alone rejects
        r, q = np.nonzero(~ok)
        log(f"{r.size} outputs beyond 2^-12 S; checked with the adder term")
        ok[r, q] = G.accept(got[r, q], c[r, q], s[r, q], out_dtype, G.mxfp8_group_term(qa, qb, r, q))
    bad = np.argwhere(~ok)
    assert bad.size == 0, f"{len(bad)} outside the bound, e.g. {[(tuple(i), got[tuple(i)], c[tuple(i)]) for i in bad[:3]]}"
    return got, c, s


def sampled_check(a_bits, b_bits, fmt, bias_bits, a_axis="row", b_axis="row", n_samples=4000, seed=0):
    log(f"gemm full-size fmt={fmt} A{a_bits.shape}/{a_axis} B{b_bits.shape}/{b_axis}")
    got = run_gpu(a_bits, b_bits, fmt, bias_bits, "bf16", a_axis, b_axis)
    qa, qb = Q.quantize(a_bits, fmt, a_axis), Q.quantize(b_bits, fmt, b_axis)
    rng = np.random.default_rng(seed)
    rows = rng.integers(0, qa.rows, n_samples)
    cols = rng.integers(0, qb.rows, n_samples)
    # the corners of the first and the last tile
    rows[:6] = [qa.rows - 1, qa.rows - 1, 0, qa.rows - 1, 0, qa.rows // 2]
    cols[:6] = [qb.rows - 1, 0, qb.rows - 1, qb.rows // 2, 0, qb.rows - 1]
    c, s = G.gemm_ref_entries(qa, qb, rows, cols, bias_bits)
    ok = G.accept_entries(got[rows, cols], c, s, "bf16", qa, qb, rows, cols)
    assert ok.all(), f"{(~ok).sum()} of {n_samples} sampled outputs outside the bound"
    assert np.isfinite(got).all()


# ---------------------------------------------------------------- tests

@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("mnk", RANDOM_MNK)
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
@pytest.mark.parametrize("mnk", INTEGER_MNK)
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


@pytest.mark.parametrize("wname,lin", FULL_SIZE_FWD)
def test_gemm_forward_full_size(wname, lin):
    """Every forward linear of the ViT-L MXFP8 / MXFP4 and ViT-B MXFP8 stacks
    at full size (block 0's tensors), in the kernel configuration the
    benchmark launches for it (ViT-L MXFP8 fc1 runs the 256x256 tile)."""
    wl = W.STACKS[wname]
    L = {l.name: l for l in wl.linears}[lin]
    log(f"plan {api.gemm_plan(wl.m, L.n, L.k, wl.fmt)}")
    a = (W.np_gelu_activation if L.a_kind == "gelu" else W.np_activation)((wl.m, L.k), W.seed(wl.wid, 0, L.a_id))
    b = W.np_normal((L.n, L.k), W.seed(wl.wid, 0, L.w_id), W.W_STD)
    bias = W.np_normal((L.n,), W.seed(wl.wid, 0, L.bias_id), W.BIAS_STD)
    sampled_check(a, b, wl.fmt, bias)


def train_operands(tp, which):
    """Seeded bf16 operands (A source, B source, bias) of one fc1/fc2 training GEMM."""
    S = lambda tid: W.seed(tp.wid, 0, tid)   # noqa: E731
    lin, kind = which.split("_")
    if lin == "fc1":
        x, w = W.np_activation((tp.m, tp.hidden), S(tp.X)), W.np_normal((tp.mlp, tp.hidden), S(tp.W1), W.W_STD)
        dy, bias = W.np_normal((tp.m, tp.mlp), S(tp.DY1), W.GRAD_STD), W.np_normal((tp.mlp,), S(tp.B1), W.BIAS_STD)
    else:
        x, w = W.np_gelu_activation((tp.m, tp.mlp), S(tp.H)), W.np_normal((tp.hidden, tp.mlp), S(tp.W2), W.W_STD)
        dy, bias = W.np_normal((tp.m, tp.hidden), S(tp.DY2), W.GRAD_STD), W.np_normal((tp.hidden,), S(tp.B2), W.BIAS_STD)
    if kind == "fprop":
        return x, w, bias
    if kind == "dgrad":
        return dy, w, None
    return dy, x, None


@pytest.mark.parametrize("tname,which", FULL_SIZE_TRAIN)
def test_gemm_training_full_size(tname, which):
    """The fc1/fc2 training GEMMs (NVFP4 and MXFP8) at full size: wgrad
    contracts over the 11235 tokens (K_pad 11264); dgrad and wgrad take
    column-quantized operands."""
    tp = W.TRAIN_PAIRS[tname]
    m, n, k, a_axis, b_axis, _ = train_gemm_shape(tp, which)
    log(f"plan {api.gemm_plan(m, n, k, tp.fmt)}")
    a, b, bias = train_operands(tp, which)
    sampled_check(a, b, tp.fmt, bias, a_axis, b_axis)


@pytest.mark.parametrize("bname,lin,which", FULL_SIZE_BLOCK)
def test_gemm_block_backward_full_size(bname, lin, which):
    """qkv's and proj's dgrad and wgrad of a ViT-L block at full size, in the
    backward format of the FINAL (MXFP8) and P3 (NVFP4) block workloads:
    dgrad 11235 x 1024 x {3072, 1024}, wgrad {3072, 1024} x 1024 x 11235."""
    bt = W.BLOCK_TRAINS[bname]
    i = [l.name for l in bt.linears()].index(lin)
    L = bt.linears()[i]
    xi, wi, _, di = bt.ids(i)
    S = lambda tid: W.seed(bt.wid, 0, tid)   # noqa: E731
    m, n, k, a_axis, b_axis = block_gemm_shape(bt, lin, which)
    log(f"plan {api.gemm_plan(m, n, k, bt.bwd_fmt)}")
    dy = W.np_normal((bt.m, L.n), S(di), W.GRAD_STD)
    if which == "dgrad":
        b = W.np_normal((L.n, L.k), S(wi), W.W_STD)
    else:
        b = W.np_activation((bt.m, L.k), S(xi))
    sampled_check(dy, b, bt.bwd_fmt, None, a_axis, b_axis)


@pytest.mark.parametrize("m,n,k,fmt,out_dtype,tile", MANY_TILES)
def test_gemm_many_tiles_full(m, n, k, fmt, out_dtype, tile):
    """More output tiles than resident workgroups (ragged M, and ragged N where
    listed), every output checked, for each tile shape the host can choose:
    workgroups walk several tiles with the next tile's first K-stage in flight
    across the boundary and the previous tile's stores pending."""
    plan = api.gemm_plan(m, n, k, fmt)
    assert plan.endswith(tile + ">"), plan
    a = W.np_activation((m, k), seed=91 + k)
    b = W.np_normal((n, k), seed=92 + k, std=W.W_STD)
    bias = W.np_normal((n,), seed=93, std=W.BIAS_STD)
    log(f"gemm many tiles plan={plan} m={m} n={n} k={k} out={out_dtype}")
    check_full(a, b, fmt, bias, out_dtype)


@pytest.mark.parametrize("fmt", FMTS)
def test_gemm_bias_2byte_aligned(fmt):
    """A bias pointer that is only 2-byte aligned (a view at element offset 1)
    takes the kernel's element-wise bias path; the result must not change."""
    m, n, k = 520, 1024, 256
    a = W.np_activation((m, k), seed=31)
    b = W.np_normal((n, k), seed=32, std=W.W_STD)
    bias = W.np_normal((n,), seed=33, std=W.BIAS_STD)
    qa = quantize_guarded(to_device_bf16(a), fmt, "row")
    qb = quantize_guarded(to_device_bf16(b), fmt, "row")
    padded = np.zeros(n + 1, dtype=np.uint16)
    padded[1:] = bias
    dev_bias = to_device_bf16(padded.reshape(1, -1)).reshape(-1)
    aligned = dev_bias[1:].clone()
    offset = dev_bias[1:]
    assert offset.data_ptr() % 16 == 2
    log(f"gemm bias alignment fmt={fmt}")
    got_offset = f64_of(gemm_guarded(qa, qb, offset, "bf16"))
    got_aligned = f64_of(gemm_guarded(qa, qb, aligned, "bf16"))
    assert np.array_equal(got_offset, got_aligned)
    qa_ref, qb_ref = Q.quantize(a, fmt), Q.quantize(b, fmt)
    c, s = G.gemm_ref(qa_ref, qb_ref, bias)
    r, q = np.nonzero(np.ones_like(c, dtype=bool))
    assert G.accept_entries(got_offset[r, q], c[r, q], s[r, q], "bf16", qa_ref, qb_ref, r, q).all()
