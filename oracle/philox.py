"""Philox4x32-10 and the uniform draws of the verifier (oracle side).

Philox4x32-10 is the counter-based generator of Salmon, Moraes, Dror and Shaw,
"Parallel random numbers: as easy as 1, 2, 3" (SC'11), section 4: ten rounds
of a multiply-based bijection on a 4x32-bit counter under a 2x32-bit key, the
key advanced by the Weyl constants between rounds.  The multipliers and Weyl
increments are the ones that paper publishes.  Written here with Python
integers so that every step is exact.

Draw layout (the verifier's contract, identical on the GPU side, which has its
own implementation):
  key     = (seed mod 2^32, seed >> 32)
  counter = (node, b, purpose + 2*(offset >> 32), offset mod 2^32)
  purpose 0 = accept test of node `node`, 1 = final draw at node `node`
  uniform = (word0 >> 8) * 2^-24, exactly representable in float32 and float64.
"""
from __future__ import annotations

MASK32 = 0xFFFFFFFF
PHILOX_M0 = 0xD2511F53  # multiplier applied to counter word 0
PHILOX_M1 = 0xCD9E8D57  # multiplier applied to counter word 2
PHILOX_W0 = 0x9E3779B9  # key schedule increment, key word 0
PHILOX_W1 = 0xBB67AE85  # key schedule increment, key word 1

PURPOSE_ACCEPT = 0
PURPOSE_FINAL = 1


def philox4x32_10(counter, key):
    """Return the 4 output words of Philox4x32 with 10 rounds."""
    c0, c1, c2, c3 = (int(w) & MASK32 for w in counter)
    k0, k1 = (int(w) & MASK32 for w in key)
    for rnd in range(10):
        if rnd:
            k0 = (k0 + PHILOX_W0) & MASK32
            k1 = (k1 + PHILOX_W1) & MASK32
        prod0 = PHILOX_M0 * c0
        prod1 = PHILOX_M1 * c2
        hi0, lo0 = prod0 >> 32, prod0 & MASK32
        hi1, lo1 = prod1 >> 32, prod1 & MASK32
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return c0, c1, c2, c3


def draw_counter(seed: int, offset: int, b: int, node: int, purpose: int):
    seed = int(seed) & 0xFFFFFFFFFFFFFFFF
    offset = int(offset) & 0xFFFFFFFFFFFFFFFF
    key = (seed & MASK32, seed >> 32)
    ctr = (int(node) & MASK32, int(b) & MASK32,
           (int(purpose) + 2 * (offset >> 32)) & MASK32, offset & MASK32)
    return ctr, key


def uniform_draw(seed: int, offset: int, b: int, node: int, purpose: int) -> float:
    """The uniform in [0, 1) that the verifier uses for (sequence b, node, purpose)."""
    ctr, key = draw_counter(seed, offset, b, node, purpose)
    w0 = philox4x32_10(ctr, key)[0]
    return (w0 >> 8) * (2.0 ** -24)
