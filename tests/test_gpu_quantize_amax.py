"""GPU parity of mx_quantize_batch_amax and mx_quantize_amax (the P3 recipe:
the MXFP8 forward quantization of a tensor also finds its amax, and the
NVFP4 backward copy takes that amax instead of a pass of its own).

- The batch's codes and scales equal mx_quantize_batch's byte for byte, and
  the largest of an item's accumulator words is the tensor's amax (the
  largest bf16 magnitude, exactly), also when the accumulators held a
  larger earlier value.
- mx_quantize_amax with those words writes mx_quantize's bytes, both axes.
- With another amax given (larger: coarser blocks; smaller: saturating
  blocks) the codes and scales are the oracle's at s_t from that amax, and
  the trailer records it.
- The full ViT-L sizes of the P3 block, in the launch configuration the
  benchmark uses."""
import numpy as np
import pytest
import torch

from block_scaled_precision_mx_amd import api
from block_scaled_precision_mx_amd import workloads as W
from oracle import formats as F
from oracle import quantize as Q
from gpu_util import bytes_of, log, to_device_bf16
from test_gpu_quantize import special

pytestmark = pytest.mark.gpu
SLOTS = 256


def tensor_amax(bits: np.ndarray) -> np.float32:
    """The largest |x| of a bf16 tensor, as fp32."""
    return np.float32(np.abs(F.bf16_to_f64(bits)).max())


def reduced(amax: torch.Tensor, i: int) -> np.float32:
    return np.float32(amax[i * SLOTS:(i + 1) * SLOTS].abs().max().item())


def assert_same_bytes(a: api.Quantized, b: api.Quantized, what: str):
    assert np.array_equal(bytes_of(a.codes), bytes_of(b.codes)), f"{what}: codes differ"
    assert np.array_equal(bytes_of(a.scales), bytes_of(b.scales)), f"{what}: scales differ"


INPUTS = [
    ("act", (300, 1030)), ("weight", (96, 640)), ("special", (64, 1100)), ("act", (1, 7)), ("gelu", (257, 333)),
]


def make(kind, shape, seed):
    if kind == "act":
        return W.np_activation(shape, seed)
    if kind == "gelu":
        return W.np_gelu_activation(shape, seed)
    if kind == "weight":
        return W.np_normal(shape, seed, W.W_STD)
    return special(*shape, seed=seed)


@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp4"])
def test_batch_amax_codes_and_amax(fmt):
    bits = [make(k, s, 40 + i) for i, (k, s) in enumerate(INPUTS)]
    xs = [to_device_bf16(b) for b in bits]
    log(f"batch amax fmt={fmt} shapes={[b.shape for b in bits]}")
    # the accumulators hold a large stale value: the call must zero them first
    amax = torch.full((len(xs) * SLOTS,), 1.0e30, dtype=torch.float32, device="cuda")
    got = api.mx_quantize_batch(xs, fmt, amax=amax)
    want = api.mx_quantize_batch(xs, fmt)
    for i, (g, w) in enumerate(zip(got, want)):
        assert_same_bytes(g, w, f"item {i}")
        assert reduced(amax, i) == tensor_amax(bits[i]), f"item {i}: amax {reduced(amax, i)} vs {tensor_amax(bits[i])}"
    # a second, smaller call on the same accumulators
    small = [xs[1], xs[3]]
    api.mx_quantize_batch(small, fmt, amax=amax)
    assert reduced(amax, 0) == tensor_amax(bits[1]) and reduced(amax, 1) == tensor_amax(bits[3])


@pytest.mark.parametrize("axis", ["row", "col"])
def test_quantize_amax_from_batch_equals_quantize(axis):
    bits = [make(k, s, 60 + i) for i, (k, s) in enumerate(INPUTS)]
    xs = [to_device_bf16(b) for b in bits]
    log(f"quantize_amax from batch, axis={axis}")
    amax = torch.empty(len(xs) * SLOTS, dtype=torch.float32, device="cuda")
    api.mx_quantize_batch(xs, "mxfp8", amax=amax)
    for i, x in enumerate(xs):
        got = api.mx_quantize_amax(x, "nvfp4", axis, amax[i * SLOTS:(i + 1) * SLOTS])
        assert_same_bytes(got, api.mx_quantize(x, "nvfp4", axis), f"item {i}")
        ref = Q.quantize(bits[i], "nvfp4", axis)
        assert np.array_equal(bytes_of(got.scales), ref.scale_buffer())


@pytest.mark.parametrize("factor", [4.0, 1.0, 0.25, 1.0e-30])
@pytest.mark.parametrize("axis", ["row", "col"])
def test_quantize_amax_given_value(axis, factor):
    """An amax other than the tensor's own, given as one word: blocks use s_t
    from it (saturating where it is too small) and the trailer records it."""
    bits = W.np_activation((130, 300), seed=71)
    given = np.float32(tensor_amax(bits) * np.float32(factor))
    log(f"quantize_amax given={given} axis={axis}")
    amax = torch.tensor([given], dtype=torch.float32, device="cuda")
    got = api.mx_quantize_amax(to_device_bf16(bits), "nvfp4", axis, amax)
    ref = Q.quantize(bits, "nvfp4", axis, s_t=Q.nvfp4_tensor_scale(float(given)))
    ref.amax = given
    assert np.array_equal(bytes_of(got.codes).reshape(ref.rows, -1), ref.packed_codes())
    assert np.array_equal(bytes_of(got.scales), ref.scale_buffer())


def test_quantize_amax_largest_of_the_words():
    """The amax is the largest magnitude among the words, in any position."""
    bits = W.np_normal((64, 256), 72, W.GRAD_STD)
    own = tensor_amax(bits)
    words = np.zeros(13, dtype=np.float32)
    words[[2, 5, 11]] = [own * np.float32(0.5), own, own * np.float32(0.25)]
    got = api.mx_quantize_amax(to_device_bf16(bits), "nvfp4", "col", torch.tensor(words, device="cuda"))
    assert_same_bytes(got, api.mx_quantize(to_device_bf16(bits), "nvfp4", "col"), "13 words")


def test_p3_block_tensors_full_size():
    """The P3 block's forward batch (activation 11235x1024 and the qkv weight
    3072x1024, MXFP8, with amax) and the backward NVFP4 copies of both from
    the found amax: equal to mx_quantize_batch and mx_quantize."""
    m = 11235
    x = to_device_bf16(W.np_activation((m, 1024), W.seed(9, 3, 1)))
    w = to_device_bf16(W.np_normal((3072, 1024), W.seed(9, 3, 2), W.W_STD))
    amax = torch.empty(2 * SLOTS, dtype=torch.float32, device="cuda")
    log("p3 full-size batch amax")
    got = api.mx_quantize_batch([x, w], "mxfp8", amax=amax)
    for g, want in zip(got, api.mx_quantize_batch([x, w], "mxfp8")):
        assert_same_bytes(g, want, "batch")
    for i, t in enumerate((x, w)):
        got_col = api.mx_quantize_amax(t, "nvfp4", "col", amax[i * SLOTS:(i + 1) * SLOTS])
        assert_same_bytes(got_col, api.mx_quantize(t, "nvfp4", "col"), f"col copy {i}")
    torch.cuda.synchronize()
