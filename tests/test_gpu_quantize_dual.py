"""GPU parity of mx_quantize_dual (one read -> row copy and transposed copy):
both copies must equal the oracle's quantizations byte for byte (codes,
scales, NVFP4 trailer), with the tensor's own NVFP4 scale and with the
delayed scale (headroom x an earlier amax), including a delayed amax read
from the very trailer the call rewrites, ragged and strided shapes, special
values and the full ViT-L sizes of the training workload."""
import numpy as np
import pytest
import torch

from block_scaled_precision_mx_amd import api
from block_scaled_precision_mx_amd import workloads as W
from oracle import formats as F
from oracle import quantize as Q
from gpu_util import bytes_of, guarded_quantized, log, to_device_bf16
from test_gpu_quantize import special

pytestmark = pytest.mark.gpu
FMTS = ["mxfp8", "mxfp4", "nvfp4"]


def check_copy(q, ref, what):
    got_codes = bytes_of(q.codes).reshape(ref.rows, -1)
    bad = np.argwhere(got_codes != ref.packed_codes())
    assert bad.size == 0, f"{what}: {len(bad)} code mismatches, first {bad[:5].tolist()}"
    got_scales, exp_scales = bytes_of(q.scales), ref.scale_buffer()
    assert np.array_equal(got_scales, exp_scales), f"{what}: scales differ at {np.argwhere(got_scales != exp_scales)[:10].tolist()}"


def guarded_pair(rows, cols, fmt):
    """Guarded buffers for the row and the column copy of [rows, cols]."""
    g = [guarded_quantized(rows, cols, fmt, axis) for axis in ("row", "col")]
    out = (api.Quantized(g[0][0].view, g[0][1].view, fmt, rows, cols),
           api.Quantized(g[1][0].view, g[1][1].view, fmt, cols, rows))
    return out, [b for pair in g for b in pair]


def check_guards(guards):
    for b, what in zip(guards, ("row codes", "row scales", "col codes", "col scales")):
        b.check(what)


def compare_dual(bits, fmt, amax_prev=None, headroom=32.0, src=None):
    rows, cols = bits.shape
    log(f"quantize_dual fmt={fmt} shape={rows}x{cols} amax_prev={amax_prev} headroom={headroom}")
    x = to_device_bf16(bits) if src is None else src
    ap = None if amax_prev is None else torch.tensor([amax_prev], dtype=torch.float32, device="cuda")
    out, guards = guarded_pair(rows, cols, fmt)
    row, col = api.mx_quantize_dual(x, fmt, ap, headroom, out=out)
    check_guards(guards)
    rref, cref = Q.quantize_dual(bits, fmt, amax_prev, headroom)
    check_copy(row, rref, "row copy")
    check_copy(col, cref, "col copy")
    return row, col


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("shape", [(1, 1), (3, 32), (37, 300), (130, 99), (129, 257), (300, 1030), (256, 768)])
def test_dual_random(fmt, shape):
    compare_dual(W.np_activation(shape, seed=hash(shape) % 1000 + 5), fmt)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("shape", [(7, 64), (64, 1100), (200, 130)])
def test_dual_special_values(fmt, shape):
    compare_dual(special(*shape, seed=sum(shape) + 1), fmt)


@pytest.mark.parametrize("fmt", FMTS)
def test_dual_strided_source(fmt):
    base = W.np_activation((96, 400), seed=18)
    x = to_device_bf16(base)[:, 8:8 + 300]
    bits = np.ascontiguousarray(base[:, 8:8 + 300])
    compare_dual(bits, fmt, src=x)


@pytest.mark.parametrize("amax_prev,headroom", [(3.5, 32.0), (1.0, 1.0), (50.0, 0.5), (1.0e-3, 16.0), (0.0, 32.0)])
def test_dual_nvfp4_delayed_scale(amax_prev, headroom):
    """Delayed tensor scale: from headroom x an earlier amax, with block
    saturation when the earlier amax is small; the trailers record this
    tensor's own amax."""
    bits = special(150, 300, seed=31)
    compare_dual(bits, "nvfp4", amax_prev, headroom)


def every_block_amax(seed):
    """One 16-element block per finite bf16 magnitude (0 .. 0x7F7F): element
    0 is the magnitude itself (the block amax, sign alternating), the other 15
    are seeded values of no larger magnitude, 8 blocks to a 128-element row."""
    rng = np.random.default_rng(seed)
    amax = np.arange(0, 0x7F80, dtype=np.uint32)
    n = amax.size
    rest = (rng.integers(0, 1 << 16, size=(n, 15), dtype=np.uint32) & 0x7FFF) % (amax[:, None] + 1)
    rest |= rng.integers(0, 2, size=(n, 15), dtype=np.uint32) << 15
    blocks = np.concatenate([(amax | ((np.arange(n, dtype=np.uint32) & 1) << 15))[:, None], rest], axis=1)
    pad = (-n) % 8
    blocks = np.concatenate([blocks, np.zeros((pad, 16), dtype=np.uint32)])
    return blocks.astype(np.uint16).reshape(-1, 128)


@pytest.mark.parametrize("amax_prev,headroom", [(3.5, 32.0), (1.0e-38, 1.0), (1.0e-30, 3.0), (3.0e38, 1.0),
                                                (2.0e-8, 0.75), (0.0, 32.0)])
def test_dual_nvfp4_every_block_amax(amax_prev, headroom):
    """The NVFP4 block scale byte and element codes of every finite bf16
    magnitude as a block amax, under delayed tensor scales from zero and
    fp32-subnormal up to about 10^35: both copies byte for byte against the
    oracle (the row copy holds the 16-element blocks as built; the column
    copy re-blocks them down the columns)."""
    bits = every_block_amax(seed=int(headroom * 1000) % 9973)
    compare_dual(bits, "nvfp4", amax_prev, headroom)


E2M1_MIDPOINTS = (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0)


def near_midpoint_tiles(width_tiles: int = 4) -> np.ndarray:
    """16 x 16 tiles stacked down and across, so that every row block and
    every column block of 16 holds its tile's amax (on the tile's
    diagonal). Tile i has amax 6 (block scale byte 1.0 at s_t near 1) or
    6 x an E4M3 rounding midpoint (the block scale rounds up or down by a
    hair); its other entries are the E2M1 midpoints times the E4M3 values
    around amax / 6, both signs, and their bf16 neighbours. At s_t = 1 +
    delta the quotients x / S then sit within about delta of E2M1 midpoints,
    and the block scale quotients within delta of E4M3 midpoints."""
    amaxes = [6.0] + [(51 + 6 * k) / 8 for k in range(8)] + [(51 + 6 * k) / 16 for k in range(0, 8, 2)] + [6.0 * 2 ** -5, 6.0 * 2 ** 4]
    tiles = []
    for a in amaxes:
        q = a / 6.0
        e = np.floor(np.log2(q))
        k = np.floor(q / 2.0 ** e * 8) - 8                   # E4M3 values (8 + k) 2^(e-3) and (9 + k) 2^(e-3)
        vals = [m * (8 + k + d) * 2.0 ** (e - 3) for m in E2M1_MIDPOINTS for d in (0, 1)]
        vals += [-v for v in vals]
        exact = W.to_bf16_bits(np.array(vals))
        assert np.array_equal(F.bf16_to_f64(exact), np.array(vals)), "tile values must be bf16-exact"
        body = np.concatenate([exact, exact + 1, exact - 1]).astype(np.uint16)
        for t in range(width_tiles):
            tile = np.zeros((16, 16), dtype=np.uint16)
            off = [(r, c) for r in range(16) for c in range(16) if r != c]
            for n, (r, c) in enumerate(off):
                tile[r, c] = body[(n + 7 * t) % len(body)]
            np.fill_diagonal(tile, W.to_bf16_bits(np.array([a]))[0])
            tiles.append(tile)
    rows = [np.concatenate(tiles[i:i + width_tiles], axis=1) for i in range(0, len(tiles), width_tiles)]
    return np.concatenate(rows, axis=0)


# s_t = fp32(A / 2688) for A = 2688 + j 2^-12 (fp32-exact): s_t - 1 runs from
# 0 through about +-2^-23 .. 2^-15
NEAR_MIDPOINT_J = [-300, -40, -7, -3, -1, 0, 1, 2, 5, 33, 257]


@pytest.mark.parametrize("j", NEAR_MIDPOINT_J)
def test_dual_nvfp4_near_midpoints(j):
    """Element quotients and block-scale quotients at and within 2^-23 ..
    2^-15 of their rounding midpoints (ties, and near ties on both sides):
    both copies byte for byte against the oracle's exact rounding."""
    amax_prev = 2688.0 + j * 2.0 ** -12
    assert float(np.float32(amax_prev)) == amax_prev
    compare_dual(near_midpoint_tiles(), "nvfp4", amax_prev, 1.0)


@pytest.mark.parametrize("j", [-7, 0, 1, 33])
def test_dual_sr_near_midpoints(j):
    """Stochastic rounding of the same tiles: block scales next to E4M3
    midpoints, quotients on and next to E2M1 grid points and midpoints."""
    compare_dual_sr(near_midpoint_tiles(), SR_SEED, 2688.0 + j * 2.0 ** -12, 1.0)


def test_dual_nvfp4_headroom_one_equals_plain_quantize():
    bits = W.np_gelu_activation((257, 333), seed=32)
    x = to_device_bf16(bits)
    plain_row = api.mx_quantize(x, "nvfp4", "row")
    plain_col = api.mx_quantize(x, "nvfp4", "col")
    row, col = api.mx_quantize_dual(x, "nvfp4", api.amax_field(plain_row.scales).clone(), 1.0)
    assert np.array_equal(bytes_of(row.codes), bytes_of(plain_row.codes))
    assert np.array_equal(bytes_of(row.scales), bytes_of(plain_row.scales))
    assert np.array_equal(bytes_of(col.codes), bytes_of(plain_col.codes))
    assert np.array_equal(bytes_of(col.scales), bytes_of(plain_col.scales))


def test_dual_nvfp4_delayed_amax_from_own_trailer():
    """Two steps on the same buffers: step 2 reads its delayed amax from the
    trailer it rewrites (step 1's amax), as a training loop would."""
    b1 = W.np_normal((140, 260), seed=33, std=1e-3)
    b2 = W.np_normal((140, 260), seed=34, std=2e-3)
    out = api.mx_quantize_dual(to_device_bf16(b1), "nvfp4")
    r1, c1 = Q.quantize_dual(b1, "nvfp4")
    check_copy(out[0], r1, "step 1 row")
    row, col = api.mx_quantize_dual(to_device_bf16(b2), "nvfp4", api.amax_field(out[0].scales), 32.0, out=out)
    r2, c2 = Q.quantize_dual(b2, "nvfp4", float(r1.amax), 32.0)
    check_copy(row, r2, "step 2 row")
    check_copy(col, c2, "step 2 col")


@pytest.mark.parametrize("fmt,shape,kind,delayed", [
    ("nvfp4", (11235, 4096), "gelu", False),     # H: fprop fc2 and wgrad fc2 copies
    ("nvfp4", (11235, 1024), "grad", True),      # dY2 with a delayed scale
    ("nvfp4", (4096, 1024), "weight", False),    # W1: fprop and dgrad copies
    ("mxfp8", (11235, 1024), "act", False),
    ("mxfp8", (11235, 4096), "gelu", False),     # H of the MXFP8 training pair
    ("mxfp8", (1024, 4096), "weight", False),    # W2: fprop and dgrad copies
])
def test_dual_full_size(fmt, shape, kind, delayed):
    seed = W.seed(9, 1, hash((fmt, shape)) % 97)
    if kind == "act":
        bits = W.np_activation(shape, seed)
    elif kind == "gelu":
        bits = W.np_gelu_activation(shape, seed)
    elif kind == "grad":
        bits = W.np_normal(shape, seed, W.GRAD_STD)
    else:
        bits = W.np_normal(shape, seed, W.W_STD)
    compare_dual(bits, fmt, 2.5e-3 if delayed else None, 32.0)



# ------------------------------------------------------------------ stochastic rounding

SR_SEED = (0x0123456789ABCDEF, 0xFEDCBA9876543210)


def compare_dual_sr(bits, seed, amax_prev=None, headroom=32.0):
    rows, cols = bits.shape
    log(f"dual sr shape={rows}x{cols} seed={seed[0]:#x} delayed={amax_prev is not None}")
    prev = None
    if amax_prev is not None:
        prev = torch.tensor([amax_prev], dtype=torch.float32, device="cuda")
    out, guards = guarded_pair(rows, cols, "nvfp4")
    row, col = api.mx_quantize_dual_sr(to_device_bf16(bits), seed, prev, headroom, out=out)
    check_guards(guards)
    r_ref, c_ref = Q.quantize_dual_sr(bits, seed, amax_prev, headroom)
    check_copy(row, r_ref, "row")
    check_copy(col, c_ref, "col")
    return row, col


@pytest.mark.parametrize("shape", [(1, 8), (16, 64), (37, 96), (129, 264), (300, 1024)])
def test_dual_sr_random(shape):
    compare_dual_sr(W.np_normal(shape, W.seed(9, 2, shape[0] % 97), W.GRAD_STD), SR_SEED)


def test_dual_sr_special_values():
    bits = special(130, 256, seed=17)
    compare_dual_sr(bits, (7, 11))


def test_dual_sr_delayed_scale():
    """Delayed s_t: blocks past 2688 s_t saturate; the trailers record this
    tensor's amax."""
    compare_dual_sr(W.np_normal((200, 512), 77, W.GRAD_STD), SR_SEED, 1.5e-4, 32.0)


def test_dual_sr_seed_determines_the_codes():
    bits = W.np_normal((256, 512), 5, W.GRAD_STD)
    x = to_device_bf16(bits)
    a = api.mx_quantize_dual_sr(x, SR_SEED)
    b = api.mx_quantize_dual_sr(x, SR_SEED)
    c = api.mx_quantize_dual_sr(x, (SR_SEED[0] + 1, SR_SEED[1]))
    for u, v in zip(a, b):
        assert torch.equal(u.codes, v.codes) and torch.equal(u.scales, v.scales)
    assert torch.equal(a[0].scales, c[0].scales)
    changed = (a[0].codes != c[0].codes).float().mean().item()
    assert 0.05 < changed < 0.9, changed


def test_dual_sr_full_size_grad():
    """dY2 of the NVFP4 training pair (11235 x 1024), both copies."""
    tp = W.TRAIN_PAIR
    bits = W.np_normal((tp.m, tp.hidden), W.seed(tp.wid, 0, tp.DY2), W.GRAD_STD)
    compare_dual_sr(bits, SR_SEED)
