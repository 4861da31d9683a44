"""The five synthetic workloads, and generators for whole tensors or column/row subsets of them.

Shapes and value distributions follow the operator's documented limits (the constraints section of
the "aclnnMaskedCausalConv1dBackward" page: B 1..32, B*S up to 512K = 524288, H 384..24576 in
multiples of 64, W = 3); the page names no dataset. Normal(0, s) takes s as the standard deviation.

Streams of one workload (seed = 1000 + workload index):
  0: gradY   1: x   2: weight   3: mask bits (Bernoulli)   4: mask prefix lengths
"""
from __future__ import annotations

import dataclasses

import torch

from . import gen

STREAM_GY, STREAM_X, STREAM_W, STREAM_MASK, STREAM_LEN = 0, 1, 2, 3, 4


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    S: int
    B: int
    H: int
    dtype: str  # "bf16" | "fp16"
    gy: tuple  # distribution of gradY
    x: tuple  # distribution of x
    w: tuple  # distribution of weight
    mask: tuple  # ("bernoulli", p) | ("prefix",) | ("all_true",) | ("null",)
    seed: int
    W: int = 3  # window taps: weight and gradWeight are [W,H]

    @property
    def N(self) -> int:
        return self.S * self.B * self.H

    @property
    def has_mask(self) -> bool:
        return self.mask[0] != "null"

    def algorithmic_bytes(self) -> int:
        """Bytes the method must move: read gradY and x, write gradX (2 bytes each per element),
        read the mask (1 byte per (j,i)) if present, read weight and write gradWeight [W,H]."""
        e = 2
        return 3 * self.N * e + (self.B * self.S if self.has_mask else 0) + 2 * self.W * self.H * e

    def describe(self) -> str:
        m = {"bernoulli": f"mask Bernoulli({self.mask[1] if len(self.mask) > 1 else ''})",
             "prefix": "mask per-batch valid prefix, length uniform in [S/2,S]",
             "all_true": "mask all-true", "null": "mask null (all-true)"}[self.mask[0]]
        return f"S={self.S} B={self.B} H={self.H} W={self.W} {self.dtype}, {m}"


def _w(i, name, S, B, H, dtype, gy, x, w, mask):
    return Workload(name, S, B, H, dtype, gy, x, w, mask, seed=1000 + i)


WORKLOADS = [
    _w(0, "S64_B1_H384_bf16", 64, 1, 384, "bf16",
       ("normal", 1.0), ("normal", 1.0), ("normal", 0.5), ("bernoulli", 0.8)),
    _w(1, "S4096_B4_H4096_bf16", 4096, 4, 4096, "bf16",
       ("normal", 1.0), ("normal", 1.0), ("normal", 0.5), ("all_true",)),
    _w(2, "S8192_B8_H8192_fp16", 8192, 8, 8192, "fp16",
       ("normal", 0.5), ("normal", 0.5), ("uniform", -1.0, 1.0), ("prefix",)),
    _w(3, "S16384_B32_H5120_bf16", 16384, 32, 5120, "bf16",
       ("normal", 1.0), ("normal", 1.0), ("normal", 0.5), ("bernoulli", 0.9)),
    _w(4, "S262144_B2_H24576_bf16", 262144, 2, 24576, "bf16",
       ("normal", 1.0), ("normal", 1.0), ("normal", 0.5), ("null",)),
]

HEADLINE = 3  # B*S = 512K, H = 5120


def custom(S: int, B: int, H: int, dtype: str = "bf16", mask: tuple = ("bernoulli", 0.8),
           seed: int = 7, gy=("normal", 1.0), x=("normal", 1.0), w=("normal", 0.5),
           W: int = 3) -> Workload:
    """An ad-hoc workload (edge shapes in the tests)."""
    name = f"S{S}_B{B}_H{H}_{dtype}" + ("" if W == 3 else f"_W{W}")
    return Workload(name, S, B, H, dtype, gy, x, w, mask, seed, W)


def with_taps(wl: Workload, W: int) -> Workload:
    """The same workload with a W-tap window (its weight stream extended or cut to [W,H])."""
    return dataclasses.replace(wl, name=f"{wl.name}_W{W}" if W != 3 else wl.name, W=W)


# -- generation -------------------------------------------------------------------------------------
def key(wl: Workload, stream: int) -> int:
    return gen.stream_key(wl.seed, stream)


def mask_tensor(wl: Workload, device="cpu") -> torch.Tensor | None:
    """[B,S] uint8 mask (1 = keep) or None for a null mask."""
    kind = wl.mask[0]
    if kind == "null":
        return None
    S, B = wl.S, wl.B
    if kind == "all_true":
        return torch.ones((B, S), dtype=torch.uint8, device=device)
    if kind == "bernoulli":
        idx = torch.arange(B * S, dtype=torch.int64)
        m = gen.bernoulli_at(key(wl, STREAM_MASK), idx, float(wl.mask[1])).view(B, S)
        return m.to(torch.uint8).to(device)
    if kind == "prefix":
        lens = prefix_lengths(wl)
        i = torch.arange(S, dtype=torch.int64)
        return (i[None, :] < lens[:, None]).to(torch.uint8).to(device)
    raise ValueError(kind)


def prefix_lengths(wl: Workload) -> torch.Tensor:
    """Per-batch valid lengths L_j, uniform integers in [S//2, S]."""
    return gen.uniform_int_at(key(wl, STREAM_LEN), torch.arange(wl.B, dtype=torch.int64),
                              wl.S // 2, wl.S)


def weight_tensor(wl: Workload, device="cpu") -> torch.Tensor:
    idx = torch.arange(wl.W * wl.H, dtype=torch.int64)
    return gen.values_at(key(wl, STREAM_W), idx, wl.dtype, wl.w).view(wl.W, wl.H).to(device)


def full_tensor(wl: Workload, stream: int, device) -> torch.Tensor:
    """Whole [S,B,H] gradY (stream 0) or x (stream 1), generated on `device`."""
    dist = wl.gy if stream == STREAM_GY else wl.x
    out = torch.empty((wl.S, wl.B, wl.H), dtype=gen.TORCH_DTYPE[wl.dtype], device=device)
    return gen.fill_values(out, key(wl, stream), wl.dtype, dist)


def column_tensor(wl: Workload, stream: int, hs: torch.Tensor) -> torch.Tensor:
    """[S,B,len(hs)] slice x[:, :, hs] (or gradY), regenerated on the CPU."""
    dist = wl.gy if stream == STREAM_GY else wl.x
    hs = hs.to(torch.int64)
    rows = torch.arange(wl.S * wl.B, dtype=torch.int64)
    idx = rows[:, None] * wl.H + hs[None, :]
    return gen.values_at(key(wl, stream), idx, wl.dtype, dist).view(wl.S, wl.B, len(hs))


def row_tensor(wl: Workload, stream: int, rows: torch.Tensor) -> torch.Tensor:
    """[len(rows),B,H] slice x[rows] (or gradY), regenerated on the CPU."""
    dist = wl.gy if stream == STREAM_GY else wl.x
    rows = rows.to(torch.int64)
    C = wl.B * wl.H
    idx = rows[:, None] * C + torch.arange(C, dtype=torch.int64)[None, :]
    return gen.values_at(key(wl, stream), idx, wl.dtype, dist).view(len(rows), wl.B, wl.H)


def host_inputs(wl: Workload) -> dict:
    """All inputs on the CPU (small workloads only): torch tensors gy, x, w, mask."""
    return {
        "gy": full_tensor(wl, STREAM_GY, "cpu"),
        "x": full_tensor(wl, STREAM_X, "cpu"),
        "w": weight_tensor(wl, "cpu"),
        "mask": mask_tensor(wl, "cpu"),
    }


def bits(t: torch.Tensor):
    """numpy uint16 view of a bf16/fp16 tensor's bit patterns (on the CPU)."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view("uint16")


# -- packed variable-length layout ---------------------------------------------------------------------
def varlen_lengths(wl: Workload) -> torch.Tensor:
    """Sequence lengths of the packed form of a workload: its batches' valid-prefix lengths
    (uniform integers in [S/2, S], as for the prefix mask)."""
    return prefix_lengths(wl)


def pack_index(lengths) -> tuple:
    """(row, batch) index tensors that gather a padded [S,B,...] tensor's valid tokens into the
    packed [T,...] order (batch-major: sequence 0's tokens first)."""
    lengths = torch.as_tensor(lengths, dtype=torch.int64)
    batch = torch.repeat_interleave(torch.arange(lengths.numel(), dtype=torch.int64), lengths)
    starts = torch.cumsum(lengths, 0) - lengths
    row = torch.arange(int(lengths.sum()), dtype=torch.int64) - torch.repeat_interleave(starts, lengths)
    return row, batch


def pack_tokens(t: torch.Tensor, lengths) -> torch.Tensor:
    """Packed [T,H] copy of the valid tokens of a padded [S,B,H] tensor (same device)."""
    row, batch = pack_index(lengths)
    return t[row.to(t.device), batch.to(t.device)].contiguous()


def cu_seqlens(lengths, device="cpu") -> torch.Tensor:
    """Cumulative sequence ends (int64), the packed layout's sequence description."""
    return torch.cumsum(torch.as_tensor(lengths, dtype=torch.int64), 0).to(device)
