"""Seeded synthetic workloads for three-tier activation-sparse decode.

This module only *generates inputs* and states the workload table. It holds
none of the method's arithmetic (no ranking, packing or products): both the
CPU oracle and the HIP library receive the arrays made here.

Shapes and distributions restate the five benchmark configurations (a single
1024x1024 layer, 7B-shaped attention and SwiGLU projections, a 32-layer 7B
projection stream and a 70B-shaped FFN layer), with weights ~ N(0, sigma)
rounded to fp16 and activations ~ Laplace(0, 1) rounded to fp16.

Storage convention (column-major): a matrix with R rows and n columns is held
as an array of shape [n, R]; row j of that array is column j of the matrix,
so one column is contiguous, as the SpAx page requires for reading a selected
column on its own (SpAx page, section 1, challenge 1).
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Tuple

import numpy as np

__all__ = [
    "CONFIGS", "TierSplit", "tier_counts", "rng", "weights_fp16", "laplace_fp16",
    "seed_of", "weights_fp16_torch", "laplace_fp16_torch",
]


@dataclasses.dataclass(frozen=True)
class TierSplit:
    """Integer percentages of the n input columns per tier (sum to 100)."""
    skip: int
    approx: int
    full: int

    def __post_init__(self):
        if self.skip + self.approx + self.full != 100:
            raise ValueError("tier percentages must sum to 100")


def tier_counts(n: int, split: TierSplit) -> Tuple[int, int]:
    """Column counts (k_full, k_approx) for n columns and integer percentages.

    The SpAx page calibrates integer tier sizes k_top and k_mid per group
    (section 5.2, steps 1-2); the workloads quote percentages instead, so the
    counts are taken cumulatively with round-half-up:
        k_full            = floor((p_full * n + 50) / 100)
        k_full + k_approx = floor(((p_full + p_approx) * n + 50) / 100)
    which keeps the three tiers summing to n.
    """
    kf = (split.full * n + 50) // 100
    kfa = ((split.full + split.approx) * n + 50) // 100
    return int(kf), int(kfa - kf)


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    description: str
    # (rows, cols) of every projection in one layer, keyed by matrix name
    shapes: Dict[str, Tuple[int, int]]
    splits: Tuple[TierSplit, ...]
    full_fmt: str            # "fp16" or "int4"
    approx_fmt: str          # "int4" or "int2"
    w_std: float
    layers: int = 1
    tokens: int = 1


_7B_ATTN = {"q": (4096, 4096), "k": (4096, 4096), "v": (4096, 4096), "o": (4096, 4096)}
_7B_FFN = {"gate": (11008, 4096), "up": (11008, 4096), "down": (4096, 11008)}
_70B_FFN = {"gate": (28672, 8192), "up": (28672, 8192), "down": (8192, 28672)}

CONFIGS: Dict[int, Config] = {
    1: Config("linear-1024", "single 1024x1024 linear layer, 50/25/25 skip/approx/full",
              {"w": (1024, 1024)}, (TierSplit(50, 25, 25),), "fp16", "int4", 0.02),
    2: Config("llama2-7b-attn", "q,k,v,o 4096x4096, 40/30/30, 32 tokens",
              _7B_ATTN, (TierSplit(40, 30, 30),), "fp16", "int4", 0.02, tokens=32),
    3: Config("llama2-7b-swiglu", "gate/up 11008x4096, down 4096x11008, skip 30/50/70, approx 20",
              _7B_FFN, (TierSplit(30, 20, 50), TierSplit(50, 20, 30), TierSplit(70, 20, 10)),
              "fp16", "int4", 0.02),
    4: Config("llama2-7b-stream", "32 layers x (4 attn + 3 FFN), 64 tokens, 50/25/25",
              {**_7B_ATTN, **_7B_FFN}, (TierSplit(50, 25, 25),), "fp16", "int4", 0.02,
              layers=32, tokens=64),
    5: Config("70b-ffn", "gate/up 28672x8192, down 8192x28672, int4 full + int2 approx, 50/30/20",
              _70B_FFN, (TierSplit(50, 30, 20),), "int4", "int2", 0.015),
}

# Matrix ids used in seeds (stable across configs).
MATRIX_ID = {"w": 0, "q": 1, "k": 2, "v": 3, "o": 4, "gate": 5, "up": 6, "down": 7,
             "h": 10, "z": 11, "x": 12, "codebook": 13}


def seed_of(config: int, layer: int, matrix: str, token: int = 0) -> np.random.SeedSequence:
    """SeedSequence([config, layer, matrix id, token]) -- one stream per input."""
    return np.random.SeedSequence([config, layer, MATRIX_ID[matrix], token])


def rng(config: int, layer: int, matrix: str, token: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed_of(config, layer, matrix, token)))


def weights_fp16(config: int, layer: int, matrix: str, rows: int, cols: int,
                 std: float) -> np.ndarray:
    """W ~ N(0, std) rounded to fp16, column-major: shape [cols, rows].

    Draws float32 standard normals, scales by std in float32 and rounds to
    fp16 (round to nearest even)."""
    g = rng(config, layer, matrix)
    w = g.standard_normal((cols, rows), dtype=np.float32)
    w *= np.float32(std)
    return w.astype(np.float16)


def laplace_fp16(config: int, layer: int, name: str, token: int, n: int,
                 scale: float = 1.0) -> np.ndarray:
    """x ~ Laplace(0, scale) rounded to fp16 (round to nearest even), shape [n]."""
    g = rng(config, layer, name, token)
    return g.laplace(0.0, scale, n).astype(np.float16)


def _torch_seed(seq: np.random.SeedSequence) -> int:
    return int(seq.generate_state(1, dtype=np.uint64)[0] & ((1 << 63) - 1))


def weights_fp16_torch(config: int, layer: int, matrix: str, rows: int, cols: int,
                       std: float, device):
    """Bulk weights for GPU-resident sets too large to draw on the host.

    W ~ N(0, std) from torch's generator on `device`, seeded from the same
    SeedSequence key, float32 then fp16 (round to nearest even); shape
    [cols, rows]. Values differ from weights_fp16 (a different generator), so
    a parity check on such a set copies the generated tensor to the host."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(_torch_seed(seed_of(config, layer, matrix)))
    w = torch.randn((cols, rows), generator=g, device=device, dtype=torch.float32)
    w.mul_(std)
    return w.to(torch.float16)


def laplace_fp16_torch(config: int, layer: int, name: str, token: int, n: int, device):
    """x ~ Laplace(0, 1) drawn on the host (laplace_fp16) and moved to device."""
    import torch
    return torch.from_numpy(laplace_fp16(config, layer, name, token, n)).to(device)


def trellis_codebook(config: int = 0) -> np.ndarray:
    """The trellis code's shared codebook: 2^16 draws of N(0, 1) rounded to
    fp16 (the method draws it once; both the library and the oracle take it
    as an input)."""
    g = rng(config, 0, "codebook")
    return g.standard_normal(65536).astype(np.float16)
