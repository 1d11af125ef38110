"""Seeded synthetic inputs, shared by the tests, the bench and the smoke check.

This module holds no arithmetic of the method: it only draws numbers.  Both
the HIP path and the CPU oracle receive the identical host arrays it makes.

* SplitMix64 (Steele, Lea & Flood, "Fast Splittable Pseudorandom Number
  Generators", OOPSLA 2014), used counter-style: draw ``i`` of stream ``seed``
  is ``mix(seed + (i + 1) * GAMMA)`` with ``GAMMA = 0x9E3779B97F4A7C15`` and
  ``mix`` the published 64-bit finaliser (xor-shift 30, multiply, xor-shift 27,
  multiply, xor-shift 31).
* A uniform in [0, 1) is the top 53 bits of a draw times 2^-53.
* Box & Muller (1958): from uniforms (u1, u2) of draws 2p and 2p+1,
  ``r = sqrt(-2 ln(1 - u1))`` and the pair ``(r cos 2 pi u2, r sin 2 pi u2)``
  fill elements 2p and 2p+1; computed in float64, then rounded to float32.
* bf16 values are float32 rounded to nearest-even on the top 16 bits and are
  carried as their raw uint16 bit patterns.

Seeds per workload c (1-based): Q = 100c+1, K = 100c+2, V = 100c+3, random
bit patterns for layout tests 100c+9, row samples 100c+7.

For tensors of gigabytes, which the host draws too slowly for a test,
``device_normal_bf16`` and ``device_bits`` draw on the GPU with torch's
seeded counter-based (Philox) generator; the oracle then receives the very
same values copied back to the host.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_CHUNK = 1 << 22


def _mix(z: np.ndarray) -> np.ndarray:
    z = (z ^ (z >> np.uint64(30))) * _M1
    z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def splitmix64(seed: int, n: int, start: int = 0) -> np.ndarray:
    """Draws start .. start+n-1 of the SplitMix64 stream seeded with ``seed``."""
    out = np.empty(n, dtype=np.uint64)
    base = np.uint64(seed % (1 << 64))
    with np.errstate(over="ignore"):
        for c0 in range(0, n, _CHUNK):
            c1 = min(n, c0 + _CHUNK)
            idx = np.arange(start + c0 + 1, start + c1 + 1, dtype=np.uint64)
            out[c0:c1] = _mix(base + idx * GAMMA)
    return out


def uniform01(seed: int, n: int, start: int = 0) -> np.ndarray:
    """float64 uniforms in [0, 1) from the top 53 bits of each draw."""
    return (splitmix64(seed, n, start) >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)


def _normal_chunk(seed: int, out: np.ndarray, p0: int, p1: int, n: int) -> None:
    u = uniform01(seed, 2 * (p1 - p0), start=2 * p0)
    u1, u2 = u[0::2], u[1::2]
    r = np.sqrt(-2.0 * np.log1p(-u1))
    ang = 2.0 * np.pi * u2
    z = np.empty(2 * (p1 - p0), dtype=np.float64)
    z[0::2] = r * np.cos(ang)
    z[1::2] = r * np.sin(ang)
    e0 = 2 * p0
    e1 = min(n, 2 * p1)
    out[e0:e1] = z[: e1 - e0].astype(np.float32)


def normal_f32(seed: int, n: int) -> np.ndarray:
    """n N(0,1) samples (Box-Muller pairs), float64 math rounded to float32.

    Chunks are independent (counter-based draws), so they run on a few host
    threads; the result does not depend on the thread count."""
    out = np.empty(n, dtype=np.float32)
    npairs = (n + 1) // 2
    step = _CHUNK // 2
    spans = [(p0, min(npairs, p0 + step)) for p0 in range(0, npairs, step)]
    if len(spans) <= 1:
        for p0, p1 in spans:
            _normal_chunk(seed, out, p0, p1, n)
        return out
    workers = max(1, min(8, len(os.sched_getaffinity(0)), len(spans)))
    with ThreadPoolExecutor(max_workers=workers) as ex:
        list(ex.map(lambda sp: _normal_chunk(seed, out, sp[0], sp[1], n), spans))
    return out


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest, ties to even) and return the uint16 bits.

    NaNs keep a quiet-NaN pattern; the inputs here are finite."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    nan = (u & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)
    r[nan] = ((u[nan] >> np.uint32(16)) | np.uint32(0x0040)).astype(np.uint16)
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(
        np.float32)


def tensor(seed: int, shape, dtype: str) -> np.ndarray:
    """N(0,1) tensor of ``shape``: float32, or bf16 carried as uint16 bits."""
    n = int(np.prod(shape))
    f = normal_f32(seed, n)
    if dtype == "f32":
        return f.reshape(shape)
    if dtype == "bf16":
        return f32_to_bf16_bits(f).reshape(shape)
    raise ValueError(f"unknown dtype {dtype!r}")


def random_bits(seed: int, nbytes: int) -> np.ndarray:
    """nbytes of raw SplitMix64 output (every bit pattern, NaN payloads included)."""
    words = splitmix64(seed, (nbytes + 7) // 8)
    return words.view(np.uint8)[:nbytes].copy()


def row_sample(seed: int, s: int, b: int, hp: int, n_random: int = 1024,
               edge: int = 64, tile_bounds=(64, 128, 256)) -> np.ndarray:
    """Fixed, seeded sample of query rows (beta, head, t) for large shares.

    For every (beta, head): the first and last ``edge`` rows, rows t0-1, t0,
    t0+1 around eight tile boundaries spread through the sequence for each
    tile size in ``tile_bounds``, and ``n_random`` uniform rows."""
    ts = set(range(min(edge, s)))
    ts.update(range(max(0, s - edge), s))
    for tb in tile_bounds:
        nb = s // tb
        for k in range(1, 9):
            t0 = (nb * k // 9) * tb
            for t in (t0 - 1, t0, t0 + 1):
                if 0 <= t < s:
                    ts.add(t)
    if n_random:
        u = uniform01(seed, n_random)
        ts.update(int(x) for x in np.minimum((u * s).astype(np.int64), s - 1))
    t_arr = np.array(sorted(ts), dtype=np.int64)
    rows = []
    for be in range(b):
        for i in range(hp):
            blk = np.empty((t_arr.size, 3), dtype=np.int64)
            blk[:, 0] = be
            blk[:, 1] = i
            blk[:, 2] = t_arr
            rows.append(blk)
    return np.concatenate(rows, axis=0)


def device_normal_bf16(seed: int, shape, device="cuda", chunk: int = 1 << 26):
    """N(0,1) tensor of ``shape`` drawn on the device (torch's Philox generator
    seeded with ``seed``, float32 samples rounded to bf16, nearest-even), in
    chunks of ``chunk`` elements so no float32 copy of the whole tensor exists."""
    import torch

    n = int(np.prod(shape))
    out = torch.empty(n, dtype=torch.bfloat16, device=device)
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    for c0 in range(0, n, chunk):
        c1 = min(n, c0 + chunk)
        out[c0:c1] = torch.randn(c1 - c0, generator=g, dtype=torch.float32, device=device)
    return out.view(*shape)


def device_bits(seed: int, shape, device="cuda"):
    """int16 tensor of ``shape`` with uniformly drawn bit patterns, on the device."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.randint(-32768, 32768, tuple(shape), generator=g, dtype=torch.int16,
                         device=device)
