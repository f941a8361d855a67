"""GPU parity of mx_gemm_gelu_quantize (fc1 writing fc2's operand): every
scale byte and code of the fused output must be explained by the oracle's
intervals (oracle.fused.check_rows): the GEMM's accuracy rule, the exact
GELU within the stated fp32 allowance, bf16 roundings, then the MX row
quantization. With an exactly representable accumulation the only slack is
the GELU allowance. Ragged N exercises the zero padding up to K_pad(N);
several tiles per workgroup exercise the epilogue's store accounting."""
import numpy as np
import pytest
import torch

from block_scaled_precision_mx_amd import api
from block_scaled_precision_mx_amd import workloads as W
from oracle import formats as F
from oracle import fused as FU
from oracle import gemm as G
from oracle import quantize as Q
from gpu_util import bytes_of, guarded_quantized, log, quantize_guarded, to_device_bf16
from test_gpu_gemm import exact_operand

pytestmark = pytest.mark.gpu
MX = ["mxfp8", "mxfp4"]
EXACT_MNK = [(64, 136, 256), (200, 512, 1024)]
RANDOM_MNK = [(1, 8, 32), (37, 96, 300), (300, 520, 640), (513, 264, 128)]
MANY_TILES_MNK = (4160, 4096, 384)


def parity_cases():
    """(M, N, K, fmt, out, epilogue) of every mx_gemm_gelu_quantize this module runs."""
    cases = []
    for fmt in MX:
        cases += [(m, n, k, fmt, "q", "gelu_quant") for (m, n, k) in EXACT_MNK + RANDOM_MNK]
        cases += [(130, 264, 256, fmt, "q", "gelu_quant"), MANY_TILES_MNK + (fmt, "q", "gelu_quant")]
        wl = W.VITL_MXFP8 if fmt == "mxfp8" else W.VITL_MXFP4
        L = {l.name: l for l in wl.linears}["fc1"]
        cases.append((wl.m, L.n, L.k, fmt, "q", "gelu_quant"))
        n_edge = 32 * len(EDGE_EXPONENTS)
        cases += [(3, n_edge, 64, fmt, "q", "gelu_quant"), (4096, 3 * n_edge, 64, fmt, "q", "gelu_quant")]
    return cases


def run_fused(a_bits, b_bits, fmt, bias_bits=None, bias_offset=0):
    qa = quantize_guarded(to_device_bf16(a_bits), fmt, "row")
    qb = quantize_guarded(to_device_bf16(b_bits), fmt, "row")
    bias = None
    if bias_bits is not None:
        padded = np.concatenate([np.zeros(bias_offset, dtype=np.uint16), bias_bits])
        bias = to_device_bf16(padded.reshape(1, -1)).reshape(-1)[bias_offset:]
    m, n = a_bits.shape[0], b_bits.shape[0]
    gc, gs = guarded_quantized(m, n, fmt, "row")
    q = api.mx_gemm_gelu_quantize(qa, qb, bias, out=api.Quantized(gc.view, gs.view, fmt, m, n))
    gc.check("fused output codes")
    gs.check("fused output scales")
    return bytes_of(q.codes).reshape(m, -1), bytes_of(q.scales).reshape(m, -1)


def check(a_bits, b_bits, fmt, bias_bits=None, rows=None, gemm_tol=G.TOL, bias_offset=0):
    m, n = a_bits.shape[0], b_bits.shape[0]
    log(f"gemm+gelu+quant fmt={fmt} M={m} N={n} K={a_bits.shape[1]} rows={'all' if rows is None else len(rows)}")
    codes, scales = run_fused(a_bits, b_bits, fmt, bias_bits, bias_offset)
    qa, qb = Q.quantize(a_bits, fmt), Q.quantize(b_bits, fmt)
    if rows is None:
        rows = np.arange(m)
        c, s = G.gemm_ref(qa, qb, bias_bits)
    else:
        rows = np.asarray(rows)
        rr = np.repeat(rows, n)
        cc = np.tile(np.arange(n), len(rows))
        c, s = G.gemm_ref_entries(qa, qb, rr, cc, bias_bits)
        c, s = c.reshape(len(rows), n), s.reshape(len(rows), n)
    ok_c, ok_s = FU.check_rows(FU.unpack_codes(codes[rows], fmt), scales[rows], c, s, fmt, n, gemm_tol)
    if fmt == "mxfp8" and gemm_tol > 0 and not (ok_c.all() and ok_s.all()):
        # rows with a rejected element or block: again with the MXFP8 matrix
        # instruction's adder term H added to the GEMM allowance
        redo = np.flatnonzero(~ok_c.all(axis=1) | ~ok_s.all(axis=1))
        log(f"{redo.size} rows beyond 2^-12 S; checked with the adder term")
        rr, cc = np.repeat(rows[redo], n), np.tile(np.arange(n), redo.size)
        h = G.mxfp8_group_term(qa, qb, rr, cc).reshape(redo.size, n)
        c2, s2 = c[redo], s[redo]
        ok_c[redo], ok_s[redo] = FU.check_rows(FU.unpack_codes(codes[rows[redo]], fmt), scales[rows[redo]], c2, s2,
                                               fmt, n, gemm_tol, h)
    bad = np.argwhere(~ok_c)
    assert bad.size == 0, f"{len(bad)} codes outside their intervals, first {bad[:5].tolist()}"
    assert ok_s.all(), f"{(~ok_s).sum()} scale bytes outside their range, first {np.argwhere(~ok_s)[:5].tolist()}"
    return codes, scales


@pytest.mark.parametrize("fmt", MX)
@pytest.mark.parametrize("mnk", EXACT_MNK)
def test_fused_exact_accumulation(fmt, mnk):
    """Exactly quantized operands (A scaled by 2^-7 so h spans GELU's curved
    range) make every accumulation exact: no GEMM slack."""
    m, n, k = mnk
    rng = np.random.default_rng(m + n + k)
    a = W.to_bf16_bits(F.bf16_to_f64(exact_operand(m, k, fmt, rng, 0)) * 2.0 ** -7)
    b = exact_operand(n, k, fmt, rng, 1)
    check(a, b, fmt, None, gemm_tol=0.0)


@pytest.mark.parametrize("fmt", MX)
@pytest.mark.parametrize("mnk", RANDOM_MNK)
def test_fused_random(fmt, mnk):
    m, n, k = mnk
    a = W.np_activation((m, k), seed=m + 1)
    b = W.np_normal((n, k), seed=n + 2, std=W.W_STD * 4)
    bias = W.np_normal((n,), seed=k + 3, std=W.BIAS_STD * 10)
    check(a, b, fmt, bias)


@pytest.mark.parametrize("fmt", MX)
def test_fused_unaligned_bias(fmt):
    """A bias that is not 16-byte aligned is read from global memory instead
    of being copied to LDS."""
    a = W.np_activation((130, 256), seed=7)
    b = W.np_normal((264, 256), seed=8, std=W.W_STD * 4)
    bias = W.np_normal((264,), seed=9, std=0.5)
    check(a, b, fmt, bias, bias_offset=3)


@pytest.mark.parametrize("fmt", MX)
def test_fused_many_tiles(fmt):
    """More output tiles than resident workgroups: each workgroup's epilogue
    stores stay in flight across the next tile's first stage."""
    m, n, k = MANY_TILES_MNK
    a = W.np_activation((m, k), seed=31)
    b = W.np_normal((n, k), seed=32, std=W.W_STD * 2)
    bias = W.np_normal((n,), seed=33, std=W.BIAS_STD)
    rows = np.concatenate([np.arange(0, m, 97), [m - 1]])
    check(a, b, fmt, bias, rows=rows)


@pytest.mark.parametrize("fmt", MX)
def test_fused_vitl_fc1_full_size(fmt):
    """fc1 of ViT-L at the workload's full size (11235 x 4096 x 1024),
    sampled rows including the last tile's."""
    wl = W.VITL_MXFP8 if fmt == "mxfp8" else W.VITL_MXFP4
    L = {l.name: l for l in wl.linears}["fc1"]
    a = W.np_activation((wl.m, L.k), W.seed(wl.wid, 0, L.a_id))
    b = W.np_normal((L.n, L.k), W.seed(wl.wid, 0, L.w_id), W.W_STD)
    bias = W.np_normal((L.n,), W.seed(wl.wid, 0, L.bias_id), W.BIAS_STD)
    rows = np.concatenate([np.arange(0, wl.m, 389), [wl.m - 1]])
    check(a, b, fmt, bias, rows=rows)


# biased bf16 exponents of the pre-activations below: zero and subnormals (0),
# the bottom of the normal range (1, 2), |h| below 2^-16 (50 .. 110), the
# GELU curve (111 .. 130, both ends), |h| >= 16 up to the largest finite (131 ..
# 254); each 32-column block holds one exponent
EDGE_EXPONENTS = [0, 1, 2, 50, 100, 110, 111, 112, 118, 120, 124, 125, 126, 127, 128, 129, 130, 131, 132, 140,
                  200, 254]


@pytest.mark.parametrize("fmt", MX)
@pytest.mark.parametrize("m, reps", [(3, 1), (4096, 3)])
def test_fused_gelu_every_exponent_range(fmt, m, reps):
    """h = bias exactly (A is zero, so every accumulation is 0): each 32-column
    block holds bf16 pre-activations of one exponent, half of them negative,
    with random mantissas and, in the exponent-0 block, signed zeros. Covers
    every branch of the epilogue's GELU: the in-range values, the closed
    forms below 2^-16 and from 16 up, and the directly evaluated zero,
    subnormal and smallest-normal inputs; the block scale follows each
    block's own magnitude, so every code is checked at its exponent. The
    small problem runs the 128 x 128 tile (GELU evaluated in fp32 for every
    element), the large one a tile that reads GELU from its LDS table."""
    rng = np.random.default_rng(1234)
    blocks = []
    for e in EDGE_EXPONENTS * reps:
        mant = rng.integers(0, 128, 32)
        sign = np.repeat([0, 1], 16)
        blk = (sign << 15) | (e << 7) | mant
        if e == 0:
            blk[[0, 16]] = [0x0000, 0x8000]
        blocks.append(blk)
    bias = np.concatenate(blocks).astype(np.uint16)
    n = bias.size
    plan = api.gemm_plan(m, n, 64, fmt)
    assert ("128x128" in plan) == (m == 3), plan
    a = np.zeros((m, 64), dtype=np.uint16)
    b = W.np_normal((n, 64), seed=77, std=W.W_STD)
    rows = None if m == 3 else np.array([0, 1, 2000, m - 1])
    check(a, b, fmt, bias, rows=rows, gemm_tol=0.0)
