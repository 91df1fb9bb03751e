"""Counter-based sketch matrix for the randomized SVD, from SplitMix64's published definition.

Test infrastructure only (see the package docstring).

The pages fix a seed for LoftQ's initialisation (loftq_config seed 42,
[LoftQ blog] §3.2) but nothing about how random numbers are drawn.  Reading:
the randomized range finder draws a Rademacher (+-1) test matrix; entry (i, j)
of the sketch for alternation t (1-based) of a k x l sketch takes counter
    c = ((t - 1) * k + i) * l + j
and the SplitMix64 output  z = mix(seed + (c + 1) * gamma)  (mod 2^64), with
gamma = 0x9E3779B97F4A7C15 and mix the SplitMix64 finalizer (Steele, Lea and
Flood, "Fast splittable pseudorandom number generators", OOPSLA 2014).  The
entry is +1 when the top bit of z is 0, else -1.  The HIP library implements the
same published generator independently; the values are exact integers, so the
two sides agree bit for bit.
"""
from __future__ import annotations

import numpy as np

__all__ = ["GAMMA", "splitmix64_stream", "rademacher_sketch"]

GAMMA = 0x9E3779B97F4A7C15
_M1 = 0xBF58476D1CE4E5B9
_M2 = 0x94D049BB133111EB


def _mix(z: np.ndarray) -> np.ndarray:
    z = np.asarray(z, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = (z ^ (z >> np.uint64(30))) * np.uint64(_M1)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(_M2)
    return z ^ (z >> np.uint64(31))


def splitmix64_stream(seed: int, counters: np.ndarray) -> np.ndarray:
    """Output number c (0-based) of the SplitMix64 sequence started at ``seed``."""
    c = np.asarray(counters, dtype=np.uint64)
    with np.errstate(over="ignore"):
        state = np.uint64(seed % (1 << 64)) + (c + np.uint64(1)) * np.uint64(GAMMA)
    return _mix(state)


def rademacher_sketch(seed: int, t: int, k: int, l: int) -> np.ndarray:
    """The k x l +-1 sketch matrix of alternation t (fp64)."""
    i = np.arange(k, dtype=np.uint64)[:, None]
    j = np.arange(l, dtype=np.uint64)[None, :]
    c = (np.uint64(t - 1) * np.uint64(k) + i) * np.uint64(l) + j
    z = splitmix64_stream(seed, c)
    top = (z >> np.uint64(63)).astype(np.int64)
    return np.where(top == 0, 1.0, -1.0)
