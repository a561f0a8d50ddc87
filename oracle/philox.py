"""Philox4x32-10 counter-based generator (Salmon, Moraes, Dror, Shaw,
"Parallel random numbers: as easy as 1, 2, 3", SC'11), vectorised in numpy.

The method draws uniform random token ids for the canvas start and for every
re-noised position ([P3] step ② and ③; [P4] "uniform state diffusion").  The
pages fix no generator; a counter-based one lets every (seed, step, position)
be drawn independently and reproducibly.

Pins (tests/test_oracle_philox.py): rocRAND's Philox4x32-10 engine, compiled
for the host from the installed ROCm headers, on 10^5 counters; chi-square
uniformity of the token ids.
"""
from __future__ import annotations

import numpy as np

_M0 = np.uint64(0xD2511F53)
_M1 = np.uint64(0xCD9E8D57)
_W0 = np.uint64(0x9E3779B9)
_W1 = np.uint64(0xBB67AE85)
_MASK = np.uint64(0xFFFFFFFF)
_S32 = np.uint64(32)

TAG_CANVAS = 0
TAG_WEIGHTS = 1


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Return the four 32-bit output words for counters (c0..c3), key (k0,k1).

    Inputs broadcast; outputs are uint32 arrays.  One round: multiply c0 and c2
    by the two round constants into 64-bit products; the new words are
    (hi(M1*c2) ^ c1 ^ k0, lo(M1*c2), hi(M0*c0) ^ c3 ^ k1, lo(M0*c0)).  The key
    is bumped by the two Weyl constants between rounds; ten rounds in all.
    """
    c0, c1, c2, c3 = (np.asarray(x, dtype=np.uint64) & _MASK for x in (c0, c1, c2, c3))
    c0, c1, c2, c3 = np.broadcast_arrays(c0, c1, c2, c3)
    k0 = np.uint64(int(k0) & 0xFFFFFFFF)
    k1 = np.uint64(int(k1) & 0xFFFFFFFF)
    for r in range(10):
        if r:
            k0 = (k0 + _W0) & _MASK
            k1 = (k1 + _W1) & _MASK
        p0 = _M0 * c0
        p1 = _M1 * c2
        n0 = (p1 >> _S32) ^ c1 ^ k0
        n1 = p1 & _MASK
        n2 = (p0 >> _S32) ^ c3 ^ k1
        n3 = p0 & _MASK
        c0, c1, c2, c3 = n0, n1, n2, n3
    return tuple(x.astype(np.uint32) for x in (c0, c1, c2, c3))


def seed_key(seed: int):
    """Key words of a 64-bit seed: (low 32 bits, high 32 bits)."""
    seed = int(seed) & 0xFFFFFFFFFFFFFFFF
    return seed & 0xFFFFFFFF, seed >> 32


def token_draw(seed, pos, step, block, req, V):
    """Uniform token id in [0, V) for canvas position ``pos`` at ``step``.

    Counter = (pos, step, block, req | TAG_CANVAS << 24); the id is
    floor(r0 * V / 2^32), exactly uniform when V is a power of two.
    Step 0 is the canvas start; the re-noise after pass t uses step t.
    """
    k0, k1 = seed_key(seed)
    pos = np.asarray(pos, dtype=np.uint64)
    r0, _, _, _ = philox4x32_10(pos, step, block, (int(req) | (TAG_CANVAS << 24)), k0, k1)
    return ((r0.astype(np.uint64) * np.uint64(V)) >> _S32).astype(np.int64)
