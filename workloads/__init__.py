"""Seeded synthetic inputs for the QLoRA linear layer.

This module is shared by the tests, the bench and the oracle's callers.  It
holds none of the layer's arithmetic: it only draws random tensors with the
shapes and distributions of the workloads and rounds the 16-bit ones with
torch's own float32 -> bfloat16 conversion.

Recipe (one linear):
  numpy ``Generator(PCG64(seed))``; tensors drawn in the order W, X, A, B, dY;
  W  float32 [d_out][d_in] ~ N(0, std 0.02)
  X  bf16    [T][d_in]     ~ N(0, 1)
  A  bf16    [r][d_in]     ~ N(0, std 1/r)
  B  bf16    [d_out][r]    ~ N(0, std 0.01)
  dY bf16    [T][d_out]    ~ N(0, 1)
Each tensor is drawn as float32 standard normals times its std; bf16 tensors
are then rounded to nearest even.  Single-linear workloads use seed 0;
multi-linear ones use seed 100*layer + projection index.

The weights stand in for the trained LLaMA-class projections the pages
discuss (7B/65B/70B scale); no model, dataset or checkpoint is read.
"""

from dataclasses import dataclass
from typing import Dict, List

import numpy as np

BF16_STD = {"X": 1.0, "dY": 1.0, "B": 0.01}
W_STD = 0.02


@dataclass(frozen=True)
class Linear:
    name: str
    d_out: int
    d_in: int
    T: int
    r: int
    alpha: float
    seed: int


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 values -> uint16 bf16 bit patterns (torch's round to nearest even)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def layer_inputs(d_out: int, d_in: int, T: int, r: int, seed: int, with_dy: bool = True) -> Dict[str, np.ndarray]:
    """Draw one linear's inputs.  bf16 tensors are returned as uint16 bits."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out = {}
    out["W"] = (rng.standard_normal((d_out, d_in), dtype=np.float32) * np.float32(W_STD)).astype(np.float32)
    out["X"] = bf16_bits(rng.standard_normal((T, d_in), dtype=np.float32))
    a_std = np.float32(1.0 / r) if r > 0 else np.float32(0.0)
    out["A"] = bf16_bits(rng.standard_normal((r, d_in), dtype=np.float32) * a_std)
    out["B"] = bf16_bits(rng.standard_normal((d_out, r), dtype=np.float32) * np.float32(0.01))
    if with_dy:
        out["dY"] = bf16_bits(rng.standard_normal((T, d_out), dtype=np.float32))
    return out


def dropout_keep_bits(T: int, d_in: int, p: float, seed: int) -> np.ndarray:
    """Seeded LoRA-dropout keep mask: each element kept with probability 1 - p,
    packed 8 per byte ([T][d_in / 8] uint8, bit j of byte i keeps element 8i + j)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    keep = rng.random((T, d_in)) >= p
    return np.packbits(keep, axis=1, bitorder="little")


def bf16_bits_to_float(bits: np.ndarray) -> np.ndarray:
    """uint16 bf16 bit patterns -> float32 values (exact widening)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


# The workloads: shapes, ranks, alpha.
def parity_256() -> List[Linear]:
    """Single linear, W 256x256, 16 tokens, r=8, alpha=16, seed 0."""
    return [Linear("parity_256", 256, 256, 16, 8, 16.0, 0)]


def attn_4096() -> List[Linear]:
    """Attention-projection-shaped linear: W 4096x4096, 2048 tokens, r=16, alpha=32."""
    return [Linear("attn_4096", 4096, 4096, 2048, 16, 32.0, 0)]


def mlp_llama7b() -> List[Linear]:
    """MLP set: gate/up 4096->11008, down 11008->4096, 4096 tokens, r=64, alpha=16."""
    return [Linear("gate", 11008, 4096, 4096, 64, 16.0, 0),
            Linear("up", 11008, 4096, 4096, 64, 16.0, 1),
            Linear("down", 4096, 11008, 4096, 64, 16.0, 2)]


def decode_70b(T: int) -> List[Linear]:
    """Decode-shaped forward: 8192->28672 and 28672->8192 at T tokens, r=64, alpha=16."""
    return [Linear(f"up_T{T}", 28672, 8192, T, 64, 16.0, 0),
            Linear(f"down_T{T}", 8192, 28672, T, 64, 16.0, 1)]


def stack_65b(layers: int = 8) -> List[Linear]:
    """65B-class share: per layer q,k,v,o 8192x8192, gate/up 8192->22016, down 22016->8192."""
    out = []
    projs = [("q", 8192, 8192), ("k", 8192, 8192), ("v", 8192, 8192), ("o", 8192, 8192),
             ("gate", 22016, 8192), ("up", 22016, 8192), ("down", 8192, 22016)]
    for layer in range(layers):
        for p, (name, d_out, d_in) in enumerate(projs):
            out.append(Linear(f"L{layer}.{name}", d_out, d_in, 4096, 64, 16.0, 100 * layer + p))
    return out
