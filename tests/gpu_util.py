"""Helpers for the GPU parity tests (host <-> device marshalling, guard bands)."""
from __future__ import annotations

import numpy as np
import torch

from ulysses_head_sharded_amd import binding, synth

POISON = 0x5A


def dev():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    binding.load()  # fail loudly if the HIP library is missing
    return torch.device("cuda:0")


def to_dev(a: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:  # bf16 bit patterns
        return torch.from_numpy(a.view(np.int16)).to(dev()).view(torch.bfloat16)
    if a.dtype == np.float32:
        return torch.from_numpy(a).to(dev())
    raise TypeError(a.dtype)


def from_dev(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return t.contiguous().cpu().numpy()


def as_f64(a: np.ndarray) -> np.ndarray:
    return synth.bf16_bits_to_f32(a).astype(np.float64) if a.dtype == np.uint16 else \
        a.astype(np.float64)


class Guarded:
    """A device buffer with poison-filled guard bands on both sides."""

    GUARD = 4096

    def __init__(self, shape, dtype):
        elt = torch.tensor([], dtype=dtype).element_size()
        n = int(np.prod(shape))
        self.raw = torch.full((n * elt + 2 * self.GUARD,), POISON, dtype=torch.uint8,
                              device=dev())
        self.tensor = self.raw[self.GUARD:self.GUARD + n * elt].view(dtype).view(*shape)

    def guards_intact(self) -> bool:
        g = self.GUARD
        head = self.raw[:g]
        tail = self.raw[self.raw.numel() - g:]
        return bool((head == POISON).all().item() and (tail == POISON).all().item())


def share_inputs(c: int, s: int, b: int, hp: int, hkvp: int, d: int, dtype: str):
    """Seeded Q, K, V of one share (host arrays)."""
    q = synth.tensor(100 * c + 1, (s, b, hp, d), dtype)
    k = synth.tensor(100 * c + 2, (s, b, hkvp, d), dtype)
    v = synth.tensor(100 * c + 3, (s, b, hkvp, d), dtype)
    return q, k, v
