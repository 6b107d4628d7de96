"""Seeded draws and dtype rounding (no retention arithmetic here)."""

from dataclasses import dataclass

import numpy as np


def f64_to_bf16_bits(x):
    """Round fp64 values to bf16 bit patterns (uint16): first to fp32 with
    numpy's round-to-nearest-even, then fp32 -> bf16 round-to-nearest-even on
    the bit pattern. Inputs here are finite normals, so no NaN handling."""
    f32 = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = f32.view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


def bf16_bits_to_f64(bits):
    """Exact upcast of bf16 bit patterns to fp64."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


@dataclass
class Tensor:
    """One synthetic tensor: ``bits`` is what goes to the device (float32
    array, or uint16 bf16 bit patterns), ``f64`` the same values in fp64."""

    bits: np.ndarray
    f64: np.ndarray
    dtype: str  # "f32" or "bf16"

    def torch(self, device="cpu"):
        """The stored bits as a torch tensor of the storage dtype."""
        import torch

        if self.dtype == "f32":
            t = torch.from_numpy(np.ascontiguousarray(self.bits))
        else:
            t = torch.from_numpy(np.ascontiguousarray(self.bits).view(np.int16)).view(torch.bfloat16)
        return t.to(device)


def round_to(x, dtype):
    """Round an fp64 array to ``dtype`` ("f32" or "bf16") -> Tensor."""
    if dtype == "f32":
        bits = np.asarray(x, dtype=np.float32)
        return Tensor(bits, bits.astype(np.float64), "f32")
    if dtype == "bf16":
        bits = f64_to_bf16_bits(x)
        return Tensor(bits, bf16_bits_to_f64(bits), "bf16")
    raise ValueError(f"unknown dtype {dtype!r}")


def draw(seed, specs, dtype):
    """Draw standard normals in order. ``specs`` is a list of (shape, scale);
    returns a list of Tensor, one per spec, in the same order."""
    rng = np.random.default_rng(seed)
    out = []
    for shape, scale in specs:
        x = rng.standard_normal(size=shape) * scale
        out.append(round_to(x, dtype))
    return out
