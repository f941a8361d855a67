"""Seeded synthetic inputs and the workload shapes (no quantization arithmetic).

The pages measure on a private video, dataset and checkpoints of a DINOv3
ViT + EoMT segmenter (lightly-train README "DINOv3 + EoMT on RTX 5090",
section 1). None of that is available, so every input here is a seeded
synthetic bf16 tensor with the shapes of the ViT linear layers named in the
README's section 4.3 (qkv, proj, fc1, fc2 per block) and these values:

  activations  N(0, 1), each element independently (p = 1e-3) multiplied by
               50 to model the "massive activations" of README section 5.5
  fc2 input    GELU (exact erf) of such an activation
  weights      N(0, 0.02)        bias  N(0, 0.01)        grad_out  N(0, 1e-3)

(the second parameter is a standard deviation). Two generators produce the
same recipe:
  * ``np_*``: numpy PCG64 samples in float64, rounded once to bf16 (round to
    nearest, ties to even). Used by tests, so the oracle sees exactly the
    bits the GPU sees.
  * ``torch_*``: torch's device generator in float32, rounded once to bf16
    (RNE). Used by the benchmark to fill gigabytes of HBM quickly; same
    distributions, different random stream.

Seeds: seed = 100000 * workload_id + 100 * block + tensor_id.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

OUTLIER_P = 1e-3
OUTLIER_GAIN = 50.0
W_STD = 0.02
BIAS_STD = 0.01
GRAD_STD = 1e-3


# ------------------------------------------------------------- bf16 bits

def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float64 -> bf16 bit patterns, one round to nearest with ties to even
    (finite inputs; magnitudes that round past the largest bf16 give Inf).

    A bf16 value is m * 2^q with an integer m < 256 and q >= -133: for
    |x| >= 2^-126, q = floor(log2 |x|) - 7, and below that q = -133
    (subnormals). Scaling by 2^-q is exact in float64 and np.rint rounds
    half to even, so m = rint(|x| 2^-q) is the single correctly rounded
    significand; m = 256 carries into the next binade."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    sign = np.signbit(x).astype(np.uint32) << 15
    _, e2 = np.frexp(a)                             # a = f 2^e2, f in [0.5, 1)
    q = np.maximum(e2.astype(np.int64) - 8, -133)
    m = np.rint(np.ldexp(a, -q)).astype(np.int64)   # 0 .. 256
    carry = m >= 256
    m = np.where(carry, m // 2, m)
    q = q + carry
    # biased exponent: subnormals (m < 128 at q = -133) keep field 0
    normal = m >= 128
    field = np.where(normal, q + 7 + 127, 0)
    bits = np.where(normal, (field << 7) | (m - 128), m)
    bits = np.where(field >= 255, 0x7F80, bits)     # overflow to Inf
    return (sign | bits.astype(np.uint32)).astype(np.uint16)


# ------------------------------------------------------------- numpy recipe

def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def _activation_f64(shape, seed: int) -> np.ndarray:
    rng = _rng(seed)
    z = rng.standard_normal(shape)
    hit = rng.random(shape) < OUTLIER_P
    z[hit] *= OUTLIER_GAIN
    return z


def np_activation(shape, seed: int) -> np.ndarray:
    return to_bf16_bits(_activation_f64(shape, seed))


def np_gelu_activation(shape, seed: int) -> np.ndarray:
    from scipy.special import erf
    z = _activation_f64(shape, seed)
    return to_bf16_bits(0.5 * z * (1.0 + erf(z / np.sqrt(2.0))))


def np_normal(shape, seed: int, std: float) -> np.ndarray:
    return to_bf16_bits(_rng(seed).standard_normal(shape) * std)


# ------------------------------------------------------------- torch recipe

def torch_activation(shape, seed: int, device="cuda", gelu=False):
    import torch
    g = torch.Generator(device=device).manual_seed(seed)
    z = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    hit = torch.rand(shape, generator=g, device=device) < OUTLIER_P
    z = torch.where(hit, z * OUTLIER_GAIN, z)
    if gelu:
        z = torch.nn.functional.gelu(z)
    return z.to(torch.bfloat16)


# LayerNorm inputs (the fp32 residual stream and the affine parameters)
LN_EPS = 1e-6
LN_GAMMA_STD = 0.1
LN_BETA_STD = 0.02


def torch_residual(shape, seed: int, device="cuda"):
    """The fp32 residual stream entering a LayerNorm: the activation recipe
    (N(0, 1), 0.1% of the entries times 50) kept in fp32."""
    import torch
    g = torch.Generator(device=device).manual_seed(seed)
    z = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    hit = torch.rand(shape, generator=g, device=device) < OUTLIER_P
    return torch.where(hit, z * OUTLIER_GAIN, z)


def torch_ln_params(n: int, seed: int, device="cuda"):
    """(gamma, beta) fp32: 1 + N(0, LN_GAMMA_STD) and N(0, LN_BETA_STD)."""
    import torch
    g = torch.Generator(device=device).manual_seed(seed)
    gamma = 1.0 + LN_GAMMA_STD * torch.randn(n, generator=g, device=device, dtype=torch.float32)
    beta = LN_BETA_STD * torch.randn(n, generator=g, device=device, dtype=torch.float32)
    return gamma, beta


def torch_normal(shape, seed: int, std: float, device="cuda"):
    import torch
    g = torch.Generator(device=device).manual_seed(seed)
    return (torch.randn(shape, generator=g, device=device, dtype=torch.float32) * std).to(torch.bfloat16)


# ------------------------------------------------------------- workloads

@dataclass(frozen=True)
class Linear:
    """One quantized GEMM C[M, N] = A[M, K] * W[N, K]^T + bias."""
    name: str
    n: int
    k: int
    a_kind: str          # "act" or "gelu"
    a_id: int            # tensor ids for seeds
    w_id: int
    bias_id: int


@dataclass(frozen=True)
class Stack:
    """A forward linear stack: `blocks` ViT blocks of qkv/proj/fc1/fc2."""
    wid: int
    name: str
    fmt: str
    m: int
    hidden: int
    mlp: int
    blocks: int
    linears: tuple = field(default=())
    # fc1's epilogue applies GELU and writes fc2's quantized operand, so fc2's
    # input is GELU(fc1's output) instead of a separate synthetic tensor
    fuse_fc1_gelu: bool = False
    # qkv's and fc1's inputs are the LayerNorm of an fp32 residual stream,
    # computed and quantized in one launch (mx_layernorm_quantize)
    ln_quant: bool = False

    def gemm_flops(self) -> int:
        return 2 * self.m * sum(l.n * l.k for l in self.linears) * self.blocks


def _vit_linears(hidden: int, mlp: int):
    return (
        Linear("qkv", 3 * hidden, hidden, "act", 0, 1, 2),
        Linear("proj", hidden, hidden, "act", 3, 4, 5),
        Linear("fc1", mlp, hidden, "act", 6, 7, 8),
        Linear("fc2", hidden, mlp, "gelu", 9, 10, 11),
    )


TOKENS = 1605                  # 40 x 40 patches of a 640 x 640 image + cls + 4 registers

SINGLE_LAYER = Stack(1, "single_mxfp8_256x768x768", "mxfp8", 256, 768, 768, 1,
                     (Linear("linear", 768, 768, "act", 0, 1, 2),))
VITB_MXFP8 = Stack(2, "vitb16_mxfp8_fwd_stack", "mxfp8", 14 * TOKENS, 768, 3072, 12,
                   _vit_linears(768, 3072))
VITL_MXFP8 = Stack(3, "vitl16_mxfp8_fwd_stack", "mxfp8", 7 * TOKENS, 1024, 4096, 24,
                   _vit_linears(1024, 4096))
VITL_MXFP4 = Stack(4, "vitl16_mxfp4_fwd_stack", "mxfp4", 7 * TOKENS, 1024, 4096, 24,
                   _vit_linears(1024, 4096))

VITL_MXFP8_FUSED = Stack(3, "vitl16_mxfp8_fwd_stack_fc1gelu", "mxfp8", 7 * TOKENS, 1024, 4096, 24,
                         _vit_linears(1024, 4096), fuse_fc1_gelu=True)
VITL_MXFP4_FUSED = Stack(4, "vitl16_mxfp4_fwd_stack_fc1gelu", "mxfp4", 7 * TOKENS, 1024, 4096, 24,
                         _vit_linears(1024, 4096), fuse_fc1_gelu=True)

# the layer structure of the pages' MXFP8 stack: LayerNorm fused with the
# quantization of qkv's and fc1's inputs, fc1's epilogue writing fc2's operand
VITL_MXFP8_LAYER = Stack(3, "vitl16_mxfp8_fwd_stack_lnq_fc1gelu", "mxfp8", 7 * TOKENS, 1024, 4096, 24,
                         _vit_linears(1024, 4096), fuse_fc1_gelu=True, ln_quant=True)
VITL_MXFP4_LAYER = Stack(4, "vitl16_mxfp4_fwd_stack_lnq_fc1gelu", "mxfp4", 7 * TOKENS, 1024, 4096, 24,
                         _vit_linears(1024, 4096), fuse_fc1_gelu=True, ln_quant=True)

STACKS = {s.name: s for s in (SINGLE_LAYER, VITB_MXFP8, VITL_MXFP8, VITL_MXFP4, VITL_MXFP8_FUSED, VITL_MXFP4_FUSED,
                              VITL_MXFP8_LAYER, VITL_MXFP4_LAYER)}


@dataclass(frozen=True)
class TrainPair:
    """fc1/fc2 of one ViT-L block: fprop, dgrad and wgrad GEMMs, every
    operand quantized in `fmt` (its row copy and its transposed copy)."""
    wid: int = 5
    name: str = "vitl16_nvfp4_fc1fc2_train"
    fmt: str = "nvfp4"
    m: int = 7 * TOKENS
    hidden: int = 1024
    mlp: int = 4096
    # tensor ids
    X: int = 20
    H: int = 21
    DY1: int = 22
    DY2: int = 23
    W1: int = 24
    W2: int = 25
    B1: int = 26
    B2: int = 27
    # gradients (dY1, dY2) rounded stochastically (NVFP4 only), with this seed
    sr_grads: bool = False
    sr_seed: tuple = (0x5EED0001, 0x5EED0002)

    def gemm_flops(self) -> int:
        return 6 * 2 * self.m * self.hidden * self.mlp


TRAIN_PAIR = TrainPair()
# the same pair in MXFP8: the MXFP8 training stack's dgrad / wgrad GEMMs
TRAIN_PAIR_MXFP8 = TrainPair(wid=6, name="vitl16_mxfp8_fc1fc2_train", fmt="mxfp8")
# the NVFP4 pair with stochastically rounded gradients (same tensors as TRAIN_PAIR)
TRAIN_PAIR_SR = TrainPair(name="vitl16_nvfp4_fc1fc2_train_srgrad", sr_grads=True)
TRAIN_PAIRS = {tp.name: tp for tp in (TRAIN_PAIR, TRAIN_PAIR_MXFP8, TRAIN_PAIR_SR)}


def seed(wid: int, block: int, tensor_id: int) -> int:
    return 100000 * wid + 100 * block + tensor_id


@dataclass(frozen=True)
class BlockTrain:
    """The twelve GEMMs of one ViT block's training step (README section 5.4
    measures them per ViT-L block): for each linear L of qkv / proj / fc1 /
    fc2, fprop Y = X W^T + b, dgrad dX = dY W and wgrad dW = dY^T X, with
    every operand quantized along its own K axis. `fwd_fmt` is the format of
    the four fprop GEMMs, `bwd_fmt` that of the eight dgrad / wgrad GEMMs
    (README section 5.3's format maps: FINAL runs all three GEMMs of a
    Linear in MXFP8; P3 moves dgrad / wgrad to NVFP4 with the gradient
    rounded stochastically). `blocks` blocks with their own tensors make one
    step, so that no launch is served from the Infinity Cache."""
    wid: int
    name: str
    fwd_fmt: str
    bwd_fmt: str
    sr_grads: bool = False
    m: int = 7 * TOKENS
    hidden: int = 1024
    mlp: int = 4096
    blocks: int = 4
    sr_seed: tuple = (0x5EED0011, 0x5EED0012)

    def linears(self):
        return _vit_linears(self.hidden, self.mlp)

    # tensor ids of linear i (0 qkv, 1 proj, 2 fc1, 3 fc2): X, W, bias, dY
    @staticmethod
    def ids(i: int):
        return 10 * i, 10 * i + 1, 10 * i + 2, 10 * i + 3

    def gemm_flops(self) -> int:
        return 3 * 2 * self.m * sum(l.n * l.k for l in self.linears()) * self.blocks


# FINAL: every GEMM of the block in MXFP8 (the page keeps qkv's fprop in BF16;
# its section 5.4 measures all twelve GEMMs of a ViT-L block in MXFP8)
BLOCK_TRAIN_MXFP8 = BlockTrain(7, "vitl16_mxfp8_block_train", "mxfp8", "mxfp8")
# P3: fprop MXFP8, dgrad / wgrad NVFP4 with stochastically rounded gradients
BLOCK_TRAIN_P3 = BlockTrain(8, "vitl16_p3_block_train", "mxfp8", "nvfp4", sr_grads=True)
BLOCK_TRAINS = {bt.name: bt for bt in (BLOCK_TRAIN_MXFP8, BLOCK_TRAIN_P3)}
