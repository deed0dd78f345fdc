"""Seeded synthetic inputs for the masked dynamic-width path.

This module is shared by the oracle tests and the GPU path (tests, smoke, bench).
It holds only input generation: seeded normal draws, bf16 input rounding and the
three mask generators. None of the masked-execution arithmetic lives here.

Seeds: ``np.random.default_rng(zlib.crc32(f"{config}/{tensor}"))`` (PCG64), so
every tensor of every workload is reproducible by name on any host.

Conventions
-----------
* ``N(0, s)`` means standard deviation ``s``.
* Float tensors are drawn in float32, then rounded to bf16 (round to nearest
  even).  They are returned as float32 arrays that hold exactly bf16 values, so
  the oracle sees the same numbers the GPU path receives as bf16.
* Masks are ``uint8 [T, n_groups]``, nonzero = the token keeps the group.
"""
from __future__ import annotations

import zlib

import numpy as np

__all__ = [
    "seed_of", "rng", "bf16_round", "bf16_bits", "bits_to_f32", "normal",
    "topk_mask", "bernoulli_mask", "clustered_mask", "router_logits",
]


def seed_of(config: str, tensor: str) -> int:
    return zlib.crc32(f"{config}/{tensor}".encode())


def rng(config: str, tensor: str) -> np.random.Generator:
    return np.random.default_rng(seed_of(config, tensor))


def bf16_round(a) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns float32."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return (u.astype(np.uint32) << 16).view(np.float32).reshape(a.shape)


def bf16_bits(a) -> np.ndarray:
    """bf16 bit patterns (uint16) of float32 values that are already bf16-exact."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    if np.any(u & 0xFFFF):
        raise ValueError("bf16_bits: input holds values that are not bf16-exact")
    return (u >> 16).astype(np.uint16)


def bits_to_f32(b) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def normal(config: str, tensor: str, shape, std: float = 1.0, *, round_bf16: bool = True) -> np.ndarray:
    x = rng(config, tensor).standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return bf16_round(x) if round_bf16 else x


# ---------------------------------------------------------------- masks


def topk_mask(logits: np.ndarray, k: int) -> np.ndarray:
    """Keep the k largest logits per row; ties go to the lower group index."""
    logits = np.asarray(logits)
    T, n = logits.shape
    if not 0 <= k <= n:
        raise ValueError("topk_mask: k out of range")
    order = np.argsort(-logits, axis=1, kind="stable")[:, :k]
    m = np.zeros((T, n), np.uint8)
    np.put_along_axis(m, order, 1, axis=1)
    return m


def router_logits(x: np.ndarray, config: str, tensor: str, n_groups: int, std: float) -> np.ndarray:
    """Input-correlated router logits x @ R with a seeded R [d, n_groups] ~ N(0, std).

    The stand-in for a trained router: masks then depend on the token's content.
    The product is taken in float32 on the bf16-rounded x.
    """
    d = x.shape[1]
    R = normal(config, tensor, (d, n_groups), std, round_bf16=False)
    return np.asarray(x, np.float32) @ R


def bernoulli_mask(config: str, tensor: str, T: int, n: int, p: float) -> np.ndarray:
    u = rng(config, tensor).random((T, n))
    return (u < p).astype(np.uint8)


def clustered_mask(config: str, tensor: str, T: int, n: int, keep: float,
                   n_proto: int = 8, flip: float = 0.05) -> np.ndarray:
    """n_proto prototype patterns with exactly round(keep*n) ones each; every token
    takes one prototype uniformly and flips each bit with probability ``flip``."""
    g = rng(config, tensor)
    k = int(round(keep * n))
    protos = np.zeros((n_proto, n), np.uint8)
    for i in range(n_proto):
        protos[i, g.choice(n, size=k, replace=False)] = 1
    pick = g.integers(0, n_proto, size=T)
    flips = (g.random((T, n)) < flip).astype(np.uint8)
    return protos[pick] ^ flips
