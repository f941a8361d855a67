"""GPU parity of mx_layernorm_quantize (LayerNorm of the fp32 residual stream
leaving its kernel as the next GEMM's MX operand): every scale byte and code
must be explained by the oracle's intervals (oracle.layernorm.check_rows):
the exact LayerNorm within the stated fp32 allowance, one bf16 rounding,
then the MX row quantization. Ragged widths exercise the zero padding up to
K_pad, a strided or unaligned x the scalar loads, constant rows the zero
variance, a large row offset the mean's rounding."""
import numpy as np
import pytest
import torch

from block_scaled_precision_mx_amd import api
from oracle import fused as FU
from oracle import layernorm as L
from gpu_util import bytes_of, guarded_quantized, log

pytestmark = pytest.mark.gpu
MX = ["mxfp8", "mxfp4"]


def residual(rows, cols, seed, offset=0.0, scale=1.0):
    """A residual-stream-like fp32 tensor: N(0, scale) plus a per-row offset
    drawn around `offset`, with 0.1% of the entries scaled by 50."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, cols)) * scale + offset * (1 + 0.1 * rng.standard_normal((rows, 1)))
    x = np.where(rng.random((rows, cols)) < 1e-3, x * 50.0, x)
    return x.astype(np.float32)


def params(cols, seed):
    rng = np.random.default_rng(seed)
    return (1 + 0.2 * rng.standard_normal(cols)).astype(np.float32), (0.1 * rng.standard_normal(cols)).astype(np.float32)


def run(x, g, b, eps, fmt, ld=None, offset=0):
    """x [rows, cols] placed in a device buffer with leading dimension ld,
    starting `offset` floats into it."""
    rows, cols = x.shape
    ld = cols if ld is None else ld
    buf = torch.zeros(offset + rows * ld + 4, dtype=torch.float32)
    view = buf[offset: offset + rows * ld].view(rows, ld)
    view[:, :cols] = torch.from_numpy(x)
    dev = buf.cuda()
    xd = dev[offset: offset + rows * ld].view(rows, ld)[:, :cols]
    gc, gs = guarded_quantized(rows, cols, fmt, "row")
    q = api.mx_layernorm_quantize(xd, torch.from_numpy(g).cuda(), torch.from_numpy(b).cuda(), eps, fmt,
                                  out=api.Quantized(gc.view, gs.view, fmt, rows, cols))
    gc.check("codes")
    gs.check("scales")
    return bytes_of(q.codes).reshape(rows, -1), bytes_of(q.scales).reshape(rows, -1)


def check(x, g, b, eps, fmt, rows=None, **kw):
    log(f"layernorm+quant fmt={fmt} rows={x.shape[0]} cols={x.shape[1]} {kw}")
    codes, scales = run(x, g, b, eps, fmt, **kw)
    sel = np.arange(x.shape[0]) if rows is None else np.asarray(rows)
    ok_c, ok_s = L.check_rows(FU.unpack_codes(codes[sel], fmt), scales[sel], x[sel], g, b, eps, fmt)
    bad = np.argwhere(~ok_c)
    assert bad.size == 0, f"{len(bad)} codes outside their intervals, first {bad[:5].tolist()}"
    assert ok_s.all(), f"{(~ok_s).sum()} scale bytes outside their range, first {np.argwhere(~ok_s)[:5].tolist()}"


@pytest.mark.parametrize("fmt", MX)
@pytest.mark.parametrize("rc", [(1, 32), (3, 100), (37, 1000), (64, 1024), (130, 768), (17, 2000), (6, 1536),
                                (9, 4096), (5, 4000), (7, 6000), (3, 8192)])
def test_layernorm_quantize_shapes(fmt, rc):
    """Widths up to 512, 1024 and 2048 take the register-resident kernel with
    one, two and four 512-column chunks per row; wider rows the three-pass
    kernel, up to the C ABI's 8192 columns."""
    r, c = rc
    x = residual(r, c, seed=r * 7 + c)
    g, b = params(c, seed=c)
    check(x, g, b, 1e-6, fmt)


@pytest.mark.parametrize("fmt", MX)
def test_layernorm_quantize_strided_and_unaligned(fmt):
    x = residual(40, 520, seed=3)
    g, b = params(520, seed=4)
    check(x, g, b, 1e-5, fmt, ld=600)
    check(x, g, b, 1e-5, fmt, ld=521, offset=1)


@pytest.mark.parametrize("fmt", MX)
def test_layernorm_quantize_constant_rows_and_offset(fmt):
    """Constant rows (variance 0: the output is beta) and rows whose mean is
    far above their spread (the mean's fp32 rounding dominates)."""
    x = residual(24, 1024, seed=5, offset=500.0, scale=0.5)
    x[3] = np.float32(2.5)
    x[11] = np.float32(-7.0)
    g, b = params(1024, seed=6)
    check(x, g, b, 1e-6, fmt)


@pytest.mark.parametrize("fmt", MX)
@pytest.mark.parametrize("c", [64, 520])
def test_layernorm_quantize_more_rows_than_one_grid(fmt, c):
    """262148 rows: the grid (65536 workgroups of 4 rows) walks the rows
    twice, the waves loading their second row while they finish the first;
    sampled rows from both passes and the last one."""
    r = 262148
    x = residual(r, c, seed=8)
    g, b = params(c, seed=9)
    check(x, g, b, 1e-6, fmt, rows=np.concatenate([np.arange(0, r, 4099), [262143, 262144, r - 1]]))


@pytest.mark.parametrize("fmt", MX)
def test_layernorm_quantize_vitl_residual_full_size(fmt):
    """The ViT-L residual stream at the workload's full size (11235 x 1024),
    sampled rows including the last."""
    x = residual(11235, 1024, seed=10, offset=0.5, scale=2.0)
    g, b = params(1024, seed=11)
    check(x, g, b, 1e-6, fmt, rows=np.concatenate([np.arange(0, 11235, 251), [11234]]))
