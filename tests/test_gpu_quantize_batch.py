"""GPU parity of mx_quantize_batch: one launch quantizes several tensors,
and every item's codes and scale bytes must equal the oracle's row
quantization of that tensor byte for byte (the same bytes mx_quantize
writes). Items differ in shape, ragged tails, leading dimension and value
range, so a workgroup that picks the wrong item or offset shows up."""
import numpy as np
import pytest
import torch

from block_scaled_precision_mx_amd import api
from block_scaled_precision_mx_amd import workloads as W
from oracle import quantize as Q
from gpu_util import bytes_of, guarded_quantized, log, to_device_bf16
from test_gpu_quantize import special

pytestmark = pytest.mark.gpu


def check_items(bits_list, got, fmt):
    for i, (bits, q) in enumerate(zip(bits_list, got)):
        ref = Q.quantize(bits, fmt, "row")
        codes = bytes_of(q.codes).reshape(ref.rows, -1)
        bad = np.argwhere(codes != ref.packed_codes())
        assert bad.size == 0, f"item {i} {bits.shape}: {len(bad)} code mismatches, first {bad[:5].tolist()}"
        scales = bytes_of(q.scales)
        assert np.array_equal(scales, ref.scale_buffer()), f"item {i} {bits.shape}: scale bytes differ"


@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp4"])
def test_batch_mixed_shapes(fmt):
    shapes = [(1, 1), (3, 32), (37, 300), (130, 99), (256, 768), (300, 1030), (7, 64), (129, 257)]
    bits_list = [special(*s, seed=11 + i) if i % 2 else W.np_activation(s, seed=11 + i) for i, s in enumerate(shapes)]
    log(f"quantize batch fmt={fmt} items={len(shapes)}")
    guards = [guarded_quantized(*b.shape, fmt, "row") for b in bits_list]
    outs = [api.Quantized(gc.view, gs.view, fmt, *b.shape) for (gc, gs), b in zip(guards, bits_list)]
    got = api.mx_quantize_batch([to_device_bf16(b) for b in bits_list], fmt, out=outs)
    for i, (gc, gs) in enumerate(guards):
        gc.check(f"item {i} codes")
        gs.check(f"item {i} scales")
    check_items(bits_list, got, fmt)


@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp4"])
def test_batch_strided_and_reused(fmt):
    """Row-strided sources (ld > cols), then a second call into the same
    buffers with other data: every byte is rewritten."""
    big = [W.np_normal((200, 700), seed=31, std=W.W_STD), W.np_activation((64, 1100), seed=32)]
    views = [to_device_bf16(b)[:, : b.shape[1] - 37] for b in big]
    bits_list = [np.ascontiguousarray(b[:, : b.shape[1] - 37]) for b in big]
    log(f"quantize batch strided fmt={fmt}")
    got = api.mx_quantize_batch(views, fmt)
    check_items(bits_list, got, fmt)
    bits2 = [special(200, 663, seed=33), W.np_activation((64, 1063), seed=34)]
    got2 = api.mx_quantize_batch([to_device_bf16(b) for b in bits2], fmt, out=got)
    check_items(bits2, got2, fmt)


def test_batch_matches_single_calls_full_size():
    """The four ViT-L weight matrices of one block in one MXFP8 launch, as the
    benchmark issues them, equal four mx_quantize calls and the oracle."""
    wl = W.VITL_MXFP8
    bits_list = [W.np_normal((l.n, l.k), W.seed(wl.wid, 0, l.w_id), W.W_STD) for l in wl.linears]
    xs = [to_device_bf16(b) for b in bits_list]
    log("quantize batch ViT-L weights")
    got = api.mx_quantize_batch(xs, "mxfp8")
    for x, q in zip(xs, got):
        single = api.mx_quantize(x, "mxfp8", "row")
        assert torch.equal(single.codes, q.codes) and torch.equal(single.scales, q.scales)
    check_items(bits_list, got, "mxfp8")


def test_batch_max_items():
    """MX_QUANT_BATCH_MAX items of different sizes in one call."""
    shapes = [(1 + 13 * i, 32 + 61 * i) for i in range(32)]
    bits_list = [W.np_activation(s, seed=100 + i) for i, s in enumerate(shapes)]
    log("quantize batch 32 items mxfp4")
    got = api.mx_quantize_batch([to_device_bf16(b) for b in bits_list], "mxfp4")
    check_items(bits_list, got, "mxfp4")
