"""Counter-based normal generator used for the seeded weight init (oracle side).

The pages fix only the seed value (PDS §4 optimisation paragraph: seed 1,337)
and the distribution N(0, 0.02) (PDS text around Fig. 1); no generator is
named.  This repository's generator, implemented independently here and in
the HIP library, is:

  * SplitMix64 (Steele, Lea & Flood, "Fast splittable pseudorandom number
    generators", OOPSLA 2014) used as a counter-based hash: the x-th output
    for seed s is mix64(s + (x + 1) * 0x9E3779B97F4A7C15) mod 2^64, where
    mix64(z): z ^= z >> 30; z *= 0xBF58476D1CE4E5B9; z ^= z >> 27;
              z *= 0x94D049BB133111EB; z ^= z >> 31.
  * element e of tensor number tau uses counters x1 = tau * 2^40 + 2e and
    x2 = x1 + 1; uniforms u = ((out >> 11) + 0.5) * 2^-53 lie in (0, 1).
  * Box-Muller (Box & Muller, 1958): z = sqrt(-2 ln u1) * cos(2 pi u2),
    evaluated in float64; the weight is float32(std * z) (round to nearest).
"""
from __future__ import annotations

import numpy as np

GAMMA = np.uint64(0x9E3779B97F4A7C15)
M1 = np.uint64(0xBF58476D1CE4E5B9)
M2 = np.uint64(0x94D049BB133111EB)
TENSOR_SHIFT = 40


def mix64(z: np.ndarray) -> np.ndarray:
    z = np.asarray(z, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = z ^ (z >> np.uint64(30))
        z = z * M1
        z = z ^ (z >> np.uint64(27))
        z = z * M2
        z = z ^ (z >> np.uint64(31))
    return z


def splitmix64(seed: int, counters: np.ndarray) -> np.ndarray:
    """Output number `counters` (0-based) of SplitMix64 started at `seed`."""
    c = np.asarray(counters, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = np.uint64(seed) + (c + np.uint64(1)) * GAMMA
    return mix64(z)


def uniform01(bits: np.ndarray) -> np.ndarray:
    return ((bits >> np.uint64(11)).astype(np.float64) + 0.5) * (2.0 ** -53)


def tensor_normal(seed: int, tensor_index: int, n: int, std: float) -> np.ndarray:
    """float32 N(0, std^2) draws for elements 0..n-1 of tensor `tensor_index`."""
    e = np.arange(n, dtype=np.uint64)
    base = np.uint64(tensor_index) << np.uint64(TENSOR_SHIFT)
    x1 = base + np.uint64(2) * e
    u1 = uniform01(splitmix64(seed, x1))
    u2 = uniform01(splitmix64(seed, x1 + np.uint64(1)))
    z = np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * np.pi * u2)
    return (std * z).astype(np.float32)
