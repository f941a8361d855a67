"""Helpers shared by the GPU parity tests: move seeded bf16 bit arrays to the
device, run the HIP path through the binding, read bytes back."""
import sys

import numpy as np
import torch


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
