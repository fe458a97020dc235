"""SplitMix64 and the seeded draws the cache format and allocator use.

SplitMix64 is the generator of Steele, Lea and Flood, "Fast Splittable
Pseudorandom Number Generators" (OOPSLA 2014), in the 64-bit form Vigna
publishes as ``splitmix64.c``: add the golden-gamma increment to the state,
then apply two xor-shift-multiply mixing rounds and a final xor-shift.

The pages say the block manager is deterministic (AX Engine page, "Core
Technical Architecture & Methods": the scheduler and KV manager are
deterministic and synchronous) but fix no allocation order; and they name a
rotation and a 1-bit QJL residual for the compressed cache (SwiftLM page,
TurboQuant KV-cache compression passage) without fixing how the random
rotation or projection is drawn.  The readings taken here:

* free list: seed 0 gives the identity order; any other seed gives a
  Fisher-Yates shuffle driven by SplitMix64 (i from n-1 down to 1,
  j = next() mod (i+1), swap).
* rotation signs D: the first d outputs of SplitMix64 seeded with the codec
  seed; D_i = -1 when the top bit of output i is set, else +1.
* QJL matrix S (d x d, row-major): the following outputs, taken in pairs
  (x1, x2): u1 = ((x1 >> 11) + 1) * 2^-53 in (0, 1], u2 = (x2 >> 11) * 2^-53 in
  [0, 1); Box-Muller gives rho = sqrt(-2 ln u1), entries rho*cos(2 pi u2) and
  rho*sin(2 pi u2), each rounded to float32.

This module is written from those definitions alone; it is not shared with the
library, which carries its own implementation of the same definitions.
"""

import math

import numpy as np

MASK64 = (1 << 64) - 1
GOLDEN_GAMMA = 0x9E3779B97F4A7C15
MIX1 = 0xBF58476D1CE4E5B9
MIX2 = 0x94D049BB133111EB


class SplitMix64:
    """The SplitMix64 stream: one 64-bit state, one output per call."""

    def __init__(self, seed):
        self.state = int(seed) & MASK64

    def next(self):
        self.state = (self.state + GOLDEN_GAMMA) & MASK64
        z = self.state
        z = ((z ^ (z >> 30)) * MIX1) & MASK64
        z = ((z ^ (z >> 27)) * MIX2) & MASK64
        return z ^ (z >> 31)


def fisher_yates(n, draw):
    """Shuffle of [0, n): for i from n-1 down to 1, j = draw() mod (i+1),
    swap positions i and j.  ``draw`` returns 64-bit unsigned integers."""
    order = list(range(n))
    for i in range(n - 1, 0, -1):
        j = draw() % (i + 1)
        order[i], order[j] = order[j], order[i]
    return order


def free_list_order(num_blocks, alloc_seed):
    """Order in which a fresh pool hands out its blocks (first element first)."""
    if alloc_seed == 0:
        return list(range(num_blocks))
    return fisher_yates(num_blocks, SplitMix64(alloc_seed).next)


def box_muller(x1, x2):
    """Two N(0,1) values (float64) from two 64-bit outputs:
    u1 = ((x1 >> 11) + 1) 2^-53 in (0, 1], u2 = (x2 >> 11) 2^-53 in [0, 1),
    rho = sqrt(-2 ln u1); returns (rho cos 2 pi u2, rho sin 2 pi u2)."""
    u1 = ((x1 >> 11) + 1) * 2.0 ** -53
    u2 = (x2 >> 11) * 2.0 ** -53
    rho = math.sqrt(-2.0 * math.log(u1))
    return rho * math.cos(2.0 * math.pi * u2), rho * math.sin(2.0 * math.pi * u2)


def codec_draws_stream(d, draw):
    """Rotation signs D and QJL matrix S from a stream of 64-bit outputs: d
    outputs for the signs (top bit set -> -1), then pairs for S in row-major
    order, each Box-Muller value rounded to float32."""
    signs = np.empty(d, dtype=np.int8)
    for i in range(d):
        signs[i] = -1 if (draw() >> 63) else 1
    flat = np.empty(d * d, dtype=np.float32)
    for t in range(0, d * d, 2):
        x1 = draw()
        x2 = draw()
        a, b = box_muller(x1, x2)
        flat[t] = np.float32(a)
        flat[t + 1] = np.float32(b)
    return signs, flat.reshape(d, d)


def codec_draws(d, codec_seed):
    """Rotation signs D (int8 +-1, length d) and QJL matrix S (float32, d x d)
    from SplitMix64 seeded with the codec seed.

    Scalar ``math`` calls are used on purpose: one value at a time, as the
    definition reads.
    """
    return codec_draws_stream(d, SplitMix64(codec_seed).next)
