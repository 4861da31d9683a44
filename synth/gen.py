"""Counter-based synthetic input generator.

Every value is a pure function of (seed, stream, linear index), computed with integer torch ops
only. Integer arithmetic is exact on every device, so the same call gives the same bits on the CPU
and on the GPU, and any subset of a tensor (a few columns, a few rows) can be regenerated on the
host without materialising the rest. That is what lets the CPU oracle check sampled outputs of a
multi-gigabyte GPU run.

This module holds none of the conv-backward arithmetic: it only draws 16-bit patterns and mask
bytes.

Generator definition:
  mix32(v)         : 32-bit integer finaliser: v ^= v>>16; v *= 0x7feb352d; v ^= v>>15;
                     v *= 0x846ca68b; v ^= v>>16 (all mod 2^32; constants of the "lowbias32" hash
                     found by C. Wellons' hash-prospector search).
  key(seed,stream) : mix32(mix32(seed) ^ stream)
  draw(key, n)     : c = mix32(key ^ (n >> 32)); u = mix32(mix32((n & 0xffffffff) ^ c) ^ key)
  value            : TABLE[u >> 16], a 65536-entry table of 16-bit patterns holding the
                     distribution's quantiles at (q + 0.5) / 65536, rounded to the dtype.
"""
from __future__ import annotations

import functools
import statistics

import numpy as np
import torch

MASK32 = 0xFFFFFFFF
_C1 = 0x7FEB352D
_C2 = 0x846CA68B


# -- scalar (python int) versions, for keys -------------------------------------------------------
def _mix32_int(v: int) -> int:
    v &= MASK32
    v ^= v >> 16
    v = (v * _C1) & MASK32
    v ^= v >> 15
    v = (v * _C2) & MASK32
    v ^= v >> 16
    return v


def stream_key(seed: int, stream: int) -> int:
    return _mix32_int(_mix32_int(seed) ^ (stream & MASK32))


# -- tensor versions (int64 tensors holding values in [0, 2^32)) ----------------------------------
def _mul32(a: torch.Tensor, c: int) -> torch.Tensor:
    """(a * c) mod 2^32 without int64 overflow: split c into 16-bit halves."""
    lo = c & 0xFFFF
    hi = c >> 16
    return (a * lo + (((a * hi) & 0xFFFF) << 16)) & MASK32


def _mix32(v: torch.Tensor) -> torch.Tensor:
    v = v ^ (v >> 16)
    v = _mul32(v, _C1)
    v = v ^ (v >> 15)
    v = _mul32(v, _C2)
    v = v ^ (v >> 16)
    return v


def draw_u32(key: int, index: torch.Tensor) -> torch.Tensor:
    """32-bit uniform draws for the int64 linear indices in `index` (same device, same shape)."""
    hi = index >> 32
    lo = index & MASK32
    c = _mix32(hi ^ key)
    return _mix32(_mix32(lo ^ c) ^ key)


# -- value tables -----------------------------------------------------------------------------------
@functools.lru_cache(maxsize=None)
def _table_np(dtype: str, dist: tuple) -> np.ndarray:
    """65536 16-bit patterns (as int16) of the distribution's quantiles, rounded to `dtype`."""
    q = (np.arange(65536, dtype=np.float64) + 0.5) / 65536.0
    kind = dist[0]
    if kind == "normal":
        sigma = float(dist[1])
        nd = statistics.NormalDist(0.0, sigma)
        vals = np.array([nd.inv_cdf(float(p)) for p in q], dtype=np.float64)
    elif kind == "uniform":
        a, b = float(dist[1]), float(dist[2])
        vals = a + (b - a) * q
    elif kind == "const":
        vals = np.full(65536, float(dist[1]))
    else:
        raise ValueError(f"unknown distribution {dist}")
    if dtype == "fp16":
        bits = vals.astype(np.float16).view(np.uint16)
    elif dtype == "bf16":
        bits = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    else:
        raise ValueError(dtype)
    return bits.view(np.int16).copy()


def table(dtype: str, dist: tuple, device) -> torch.Tensor:
    return torch.from_numpy(_table_np(dtype, tuple(dist))).to(device)


TORCH_DTYPE = {"bf16": torch.bfloat16, "fp16": torch.float16}


def values_at(key: int, index: torch.Tensor, dtype: str, dist: tuple) -> torch.Tensor:
    """16-bit values (torch bf16/fp16) for the given int64 linear indices."""
    u = draw_u32(key, index)
    tab = table(dtype, dist, index.device)
    return tab[(u >> 16)].view(TORCH_DTYPE[dtype])


def fill_values(out: torch.Tensor, key: int, dtype: str, dist: tuple,
                chunk: int = 1 << 26) -> torch.Tensor:
    """Fill a contiguous bf16/fp16 tensor, element n getting the draw for linear index n."""
    flat = out.view(-1)
    n = flat.numel()
    tab = table(dtype, dist, out.device)
    for start in range(0, n, chunk):
        stop = min(n, start + chunk)
        idx = torch.arange(start, stop, dtype=torch.int64, device=out.device)
        u = draw_u32(key, idx)
        flat[start:stop].view(torch.int16).copy_(tab[(u >> 16)])
        del idx, u
    return out


def bernoulli_at(key: int, index: torch.Tensor, p: float) -> torch.Tensor:
    """Bool draws with P(true) = p (u < p * 2^32)."""
    thresh = int(round(p * 4294967296.0))
    return draw_u32(key, index) < thresh


def uniform_int_at(key: int, index: torch.Tensor, lo: int, hi: int) -> torch.Tensor:
    """Integers in [lo, hi] (inclusive); modulo bias is below 2^-32 * (hi - lo + 1)."""
    return lo + draw_u32(key, index) % (hi - lo + 1)
