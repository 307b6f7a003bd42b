"""Block-extent checksum used to prove device slot bytes equal host bytes.

Test infrastructure (see the package docstring); not imported by the library.

The offload design keeps one authoritative host copy of each block and
requires the device slot to hold exactly that copy before the block runs
("CPU Offloading", section "Cross-strategy invariants"; "Distributed Layerwise
Offload", section "Startup and runtime sequence": tensors point at the ready
slot before the block executes).  The pages fix no checksum; this one is the
project's own choice:

    H(extent) = sum over 64-bit little-endian words w_i of
                SplitMix64(w_i XOR (i * 0x9E3779B97F4A7C15))   (mod 2^64)

where SplitMix64(s) is the first output of the SplitMix64 generator started
from state s, i.e. its finaliser applied to s + 0x9E3779B97F4A7C15 (Steele,
Lea and Flood, "Fast Splittable Pseudorandom Number Generators", OOPSLA 2014;
finaliser constants as in Vigna's public-domain splitmix64.c).  The sum is
order-independent, so a GPU can reduce it in any order and still match.
"""
from __future__ import annotations

import numpy as np

GOLDEN = np.uint64(0x9E3779B97F4A7C15)
M1 = np.uint64(0xBF58476D1CE4E5B9)
M2 = np.uint64(0x94D049BB133111EB)


def splitmix64_next(state: np.ndarray) -> np.ndarray:
    """First SplitMix64 output for each starting state (uint64, wrapping)."""
    z = np.asarray(state, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = z + GOLDEN
        z = (z ^ (z >> np.uint64(30))) * M1
        z = (z ^ (z >> np.uint64(27))) * M2
    return z ^ (z >> np.uint64(31))


def extent_checksum(buf) -> int:
    """H over a byte buffer whose length is a multiple of 8."""
    b = np.frombuffer(memoryview(buf).cast("B"), dtype=np.uint8)
    if b.size % 8:
        raise ValueError("extent length must be a multiple of 8 bytes")
    words = b.view("<u8").astype(np.uint64)
    total = np.uint64(0)
    chunk = 1 << 22
    with np.errstate(over="ignore"):
        for s in range(0, words.size, chunk):
            w = words[s:s + chunk]
            i = np.arange(s, s + w.size, dtype=np.uint64)
            h = splitmix64_next(w ^ (i * GOLDEN))
            total = total + np.sum(h, dtype=np.uint64)
    return int(total)
