"""Seeded synthetic inputs for the grouped tril mask softmax.

This module only draws inputs: it holds none of the operation's arithmetic, and both the
GPU path's tests and the oracle's tests take their inputs from it.

The workloads stand in for the ones measured on the pages (no dataset is involved there):
  - the README "Fused grouped tril mask softmax" (github aoxy/Attention-Mask-Optimization)
    times X of shape [B, 64, 1000, 1000] for B = 3 and 12 from randn, and prints a worked
    example at [3, 2, 5, 5] with lengths 3, 4, 5;
  - the ScaledMaskSoftmax article (section 3.2) times batch 32 at sequence length 4096
    with a scale factor, in half precision.
Scores are normal with mean 0; the valid lengths are uniform integers, inclusive at both
ends, or fixed lists.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

F32, F16, BF16 = 0, 1, 2
DTYPE_NAMES = {F32: "f32", F16: "f16", BF16: "bf16"}
ESIZE = {F32: 4, F16: 2, BF16: 2}


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    M: int
    S: int
    dtype: int
    sigma: float          # standard deviation of the normal scores
    scale: float
    len_lo: int = 0       # valid lengths ~ uniform integers in [len_lo, len_hi] ...
    len_hi: int = 0
    fixed_lens: tuple = field(default=())   # ... unless a fixed list is given
    x_seed: int = 0
    len_seed: int = 0

    @property
    def shape(self):
        return (self.B, self.M, self.S, self.S)

    @property
    def esize(self) -> int:
        return ESIZE[self.dtype]


WORKLOADS = {
    # the worked example of the README
    "example_f32_3x2x5": Workload("example_f32_3x2x5", 3, 2, 5, F32, 1.0, 1.0,
                                  fixed_lens=(3, 4, 5), x_seed=1001, len_seed=2001),
    # the README's timed shapes
    "readme_f32_3x64x1000": Workload("readme_f32_3x64x1000", 3, 64, 1000, F32, 1.0, 1.0,
                                     1, 1000, x_seed=1002, len_seed=2002),
    "readme_f32_12x64x1000": Workload("readme_f32_12x64x1000", 12, 64, 1000, F32, 1.0, 1.0,
                                      1, 1000, x_seed=1003, len_seed=2003),
    # batch 32 at sequence 4096, scaled, half precision (ScaledMaskSoftmax article)
    "scaled_f16_32x1x4096": Workload("scaled_f16_32x1x4096", 32, 1, 4096, F16, 2.0, 0.125,
                                     512, 4096, x_seed=1004, len_seed=2004),
    # long and skewed lengths in bfloat16
    "skewed_bf16_8x32x8192": Workload("skewed_bf16_8x32x8192", 8, 32, 8192, BF16, 1.0, 0.125,
                                      fixed_lens=(8192, 6000, 4096, 2048, 1024, 512, 128, 1),
                                      x_seed=1005, len_seed=2005),
    # rows of 128 KB (65536 bfloat16): the block path at its widest automatic layout, 16
    # wavefronts of eight 16-byte vectors per lane; 34 GB per tensor
    "long_bf16_2x2x65536": Workload("long_bf16_2x2x65536", 2, 2, 65536, BF16, 1.0, 0.125,
                                    fixed_lens=(65536, 40000), x_seed=1006, len_seed=2006),
    # rows of 200 KB (100000 bfloat16), beyond the block path's registers: the two-pass
    # paths (the row held on chip between the passes, or streamed twice); 20 GB per plane
    "long_bf16_2x1x100000": Workload("long_bf16_2x1x100000", 2, 1, 100000, BF16, 1.0, 0.125,
                                     fixed_lens=(100000, 70000), x_seed=1007, len_seed=2007),
}


@dataclass(frozen=True)
class AttnWorkload:
    """Inputs of the fused attention: q, k, v [B, M, S, D] normal, per-batch lengths."""
    name: str
    B: int
    M: int
    S: int
    D: int
    dtype: int
    len_lo: int = 0
    len_hi: int = 0
    fixed_lens: tuple = field(default=())
    x_seed: int = 0
    len_seed: int = 0

    @property
    def shape(self):
        return (self.B, self.M, self.S, self.D)

    @property
    def esize(self) -> int:
        return ESIZE[self.dtype]

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.D))


ATTN_WORKLOADS = {
    # batch 32 at sequence 4096 with head size 64 (ScaledMaskSoftmax article, test
    # conditions of its timing table) and 8 heads (the H of the README's configurations);
    # lengths as in scaled_f16_32x1x4096
    "attn_bf16_32x8x4096_d64": AttnWorkload("attn_bf16_32x8x4096_d64", 32, 8, 4096, 64, BF16,
                                            512, 4096, x_seed=1104, len_seed=2004),
    # the README's B = 3, M = 64, S = 1000, read as 64 heads of size 64; lengths as in
    # readme_f32_3x64x1000
    "attn_f16_3x64x1000_d64": AttnWorkload("attn_f16_3x64x1000_d64", 3, 64, 1000, 64, F16,
                                           1, 1000, x_seed=1102, len_seed=2002),
    # two sequences of the batch-32 shape above (a small batch of long rows): 512 (head, query
    # tile) pairs, two per compute unit, where each tile's keys are split over two groups of
    # wavefronts (flash_decoding.py's split-KV reduction)
    "attn_bf16_2x8x4096_d64": AttnWorkload("attn_bf16_2x8x4096_d64", 2, 8, 4096, 64, BF16,
                                           fixed_lens=(4096, 3001), x_seed=1105, len_seed=2005),
}


def seq_lens(w: Workload, seed: int | None = None) -> np.ndarray:
    """int32[B] valid lengths for a workload."""
    if w.fixed_lens:
        return np.asarray(w.fixed_lens, dtype=np.int32)
    rng = np.random.default_rng(w.len_seed if seed is None else seed)
    return rng.integers(w.len_lo, w.len_hi, size=w.B, endpoint=True).astype(np.int32)


def torch_dtype(dtype: int):
    import torch
    return {F32: torch.float32, F16: torch.float16, BF16: torch.bfloat16}[dtype]


def scores_cpu(shape, dtype: int, sigma: float = 1.0, seed: int = 0):
    """Normal scores on the host, drawn in fp32 and rounded into the element type."""
    import torch
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    x = torch.randn(*shape, generator=g, dtype=torch.float32)
    if sigma != 1.0:
        x.mul_(sigma)
    return x.to(torch_dtype(dtype))


def scores_device(shape, dtype: int, sigma: float = 1.0, seed: int = 0, device="cuda"):
    """Normal scores drawn on the device (used where the host draw would be too slow)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    x = torch.randn(*shape, generator=g, dtype=torch.float32 if dtype == F32 else
                    torch_dtype(dtype), device=device)
    if sigma != 1.0:
        x.mul_(sigma)
    return x


def random_lengths(B: int, S: int, seed: int, lo: int = -2, hi: int | None = None):
    """Lengths for edge-case sweeps, including values below 0 and above S."""
    rng = np.random.default_rng(seed)
    hi = S + 2 if hi is None else hi
    return rng.integers(lo, hi, size=B, endpoint=True).astype(np.int32)


def to_storage(t):
    """Raw element storage of a CPU torch tensor as numpy (float32, or uint16 bits)."""
    import torch
    t = t.contiguous()
    if t.dtype == torch.float32:
        return t.numpy()
    return t.view(torch.int16).numpy().view(np.uint16)


def from_storage(a: np.ndarray, dtype: int):
    """Inverse of to_storage: a CPU torch tensor of the element type."""
    import torch
    a = np.ascontiguousarray(a)
    if dtype == F32:
        return torch.from_numpy(a.astype(np.float32, copy=False))
    return torch.from_numpy(a.view(np.int16)).view(torch_dtype(dtype))
