"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This module only draws random numbers and rounds them to bf16; it holds none
of the attention arithmetic. Both the HIP library's callers and the oracle get
their inputs from here, and from nothing else.

Recipe (one numpy ``Generator(PCG64(seed))`` per workload):

1. draw float32 standard normals for Q, K, V (and dO when asked), in that
   order, each C-ordered ``[B, H, N, d]``;
2. optionally (the fp8 workload) multiply, for Q, K and V independently and in
   that order, ``round(0.001 * numel)`` distinct flat positions, chosen with
   ``Generator.choice(numel, size, replace=False)`` from the same generator, by
   20 in float32;
3. round each tensor to bf16 (round to nearest even, via torch's CPU cast).

Grouped heads (``grouped_inputs``): the same recipe without outliers, with K and
V drawn ``[B, H_kv, N, d]``.

Arrays are returned as float32 holding exact bf16 values. Hadamard signs are
128 Rademacher draws (int8 +-1) from ``Generator(PCG64(1105))``.
"""

from __future__ import annotations

import numpy as np
import torch

HADAMARD_SEED = 1105

# Workloads the tests and the bench use: (B, H, N, d, causal, seed).
WORKLOADS = {
    "fwd_small": (1, 2, 256, 64, False, 1),
    "fwd_n2k_d64": (4, 16, 2048, 64, None, 2),       # run non-causal and causal
    "fwd_n8k_d128_causal": (2, 16, 8192, 128, True, 3),
    "bwd_n4k_d128_causal": (2, 16, 4096, 128, True, 4),
    "fp8_n8k_d128_causal": (2, 16, 8192, 128, True, 5),
}


def sweep_seed(n: int) -> int:
    """Seed of a sequence-length sweep point: 100 + log2(N)."""
    return 100 + int(round(np.log2(n)))


def to_bf16_values(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (RNE) and widen back to float32 exactly."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def attention_inputs(B: int, H: int, N: int, d: int, seed: int, with_do: bool = False,
                     outliers: bool = False) -> dict:
    """Q, K, V (and dO) as float32 arrays of exact bf16 values."""
    rng = np.random.Generator(np.random.PCG64(seed))
    names = ["q", "k", "v"] + (["do"] if with_do else [])
    raw = {n: rng.standard_normal((B, H, N, d), dtype=np.float32) for n in names}
    if outliers:
        for n in ("q", "k", "v"):
            flat = raw[n].reshape(-1)
            count = int(round(0.001 * flat.size))
            pos = rng.choice(flat.size, size=count, replace=False)
            flat[pos] = flat[pos] * np.float32(20.0)
    return {n: to_bf16_values(raw[n]) for n in names}


def grouped_inputs(B: int, H: int, H_kv: int, N: int, d: int, seed: int, with_do: bool = False) -> dict:
    """Q (and dO) [B, H, N, d] with K, V [B, H_kv, N, d]; float32 exact bf16 values."""
    rng = np.random.Generator(np.random.PCG64(seed))
    heads = {"q": H, "k": H_kv, "v": H_kv, "do": H}
    names = ["q", "k", "v"] + (["do"] if with_do else [])
    return {n: to_bf16_values(rng.standard_normal((B, heads[n], N, d), dtype=np.float32)) for n in names}


def alibi_slopes(H: int) -> np.ndarray:
    """float32 [H] ALiBi slopes on the usual geometric schedule 2^(-8 (h + 1) / H)."""
    return (2.0 ** (-8.0 * (np.arange(H) + 1) / H)).astype(np.float32)


def hadamard_signs(seed: int = HADAMARD_SEED) -> np.ndarray:
    """128 random signs (int8, +-1)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return (rng.integers(0, 2, size=128) * 2 - 1).astype(np.int8)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """uint16 bit patterns of float32 arrays that hold exact bf16 values."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)
