"""Helpers shared by the GPU parity tests: move seeded bf16 bit arrays to the
device, run the HIP path through the binding, read bytes back, and guard
every output with canary bytes before and after it."""
import sys

import numpy as np
import torch

from block_scaled_precision_mx_amd import api

# every output buffer a test hands to the library sits between two guard
# regions filled with this byte; the library must leave them untouched
CANARY = 0xA5
GUARD = 256


def log(msg: str) -> None:
    """Name the case before each GPU step (flushed, so a fault still shows it)."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def to_device_bf16(bits: np.ndarray) -> torch.Tensor:
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return torch.from_numpy(bits.view(np.int16)).to("cuda").view(torch.bfloat16)


def bytes_of(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.detach().cpu().numpy().view(np.uint8).copy()


def f64_of(out: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    if out.dtype == torch.bfloat16:
        bits = out.detach().cpu().view(torch.int16).numpy().view(np.uint16)
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return out.detach().cpu().numpy().astype(np.float64)


class Guarded:
    """`nbytes` of device memory (16-byte aligned) with GUARD canary bytes on
    each side, and the slack up to the next multiple of 16 canary-filled too."""

    def __init__(self, nbytes: int):
        self.n = int(nbytes)
        total = GUARD + (self.n + 15) // 16 * 16 + GUARD
        self.raw = torch.full((total,), CANARY, dtype=torch.uint8, device="cuda")
        self.view = self.raw[GUARD:GUARD + self.n]
        assert self.view.data_ptr() % 16 == 0

    def typed(self, dtype, shape):
        return self.view.view(dtype).reshape(shape)

    def check(self, what: str = "output") -> None:
        torch.cuda.synchronize()
        raw = self.raw.cpu().numpy()
        head, tail = raw[:GUARD], raw[GUARD + self.n:]
        bad_head = np.flatnonzero(head != CANARY)
        bad_tail = np.flatnonzero(tail != CANARY)
        assert bad_head.size == 0, f"{what}: {bad_head.size} guard bytes before the buffer written, at {bad_head[:8] - GUARD}"
        assert bad_tail.size == 0, f"{what}: {bad_tail.size} guard bytes after the buffer written, at +{bad_tail[:8]}"


def guarded_quantized(rows: int, cols: int, fmt: str, axis: str):
    """Empty guarded code and scale buffers for quantizing [rows, cols] along axis."""
    return Guarded(api.codes_bytes(rows, cols, fmt, axis)), Guarded(api.scales_bytes(rows, cols, fmt, axis))


def quantize_guarded(x: torch.Tensor, fmt: str, axis: str = "row") -> "api.Quantized":
    """api.mx_quantize into guarded buffers; the guards are checked after the call."""
    rows, cols = x.shape
    gc, gs = guarded_quantized(rows, cols, fmt, axis)
    q = api.mx_quantize(x, fmt, axis, gc.view, gs.view)
    gc.check(f"{fmt} {axis} codes")
    gs.check(f"{fmt} {axis} scales")
    return q


def gemm_guarded(qa, qb, bias, out_dtype: str) -> torch.Tensor:
    """api.mx_gemm into a guarded C buffer; the guards are checked after the call."""
    M, N = qa.rows, qb.rows
    dt = torch.bfloat16 if out_dtype == "bf16" else torch.float32
    g = Guarded(M * N * (2 if out_dtype == "bf16" else 4))
    out = g.typed(dt, (M, N))
    api.mx_gemm(qa, qb, bias, out_dtype, out)
    g.check(f"C [{M}, {N}] {out_dtype}")
    return out
