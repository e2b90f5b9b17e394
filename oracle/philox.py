"""Philox4x32-10 counter-based generator, written out plainly in numpy.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

Published method: J. K. Salmon, M. A. Moraes, R. O. Dror, D. E. Shaw,
"Parallel Random Numbers: As Easy as 1, 2, 3", SC'11, the Philox-4x32 round.
A 128-bit counter (c0, c1, c2, c3) and a 64-bit key (k0, k1) go through ten
rounds.  One round multiplies c0 by 0xD2511F53 and c2 by 0xCD9E8D57 as full
32x32 -> 64-bit products and emits

    (hi(c2*M1) ^ c1 ^ k0,  lo(c2*M1),  hi(c0*M0) ^ c3 ^ k1,  lo(c0*M0))

and between rounds the key is bumped by the Weyl constants (0x9E3779B9,
0xBB67AE85) modulo 2^32.  The first round uses the key as given.

The pages only ask for "random signs" and "stochastic rounding"; which
generator draws them is an engineering choice (UFP4 summary page, "Method":
random sign diagonal S_n; 2D-block page, "2D square-block quantization":
stochastic rounding).  Philox is chosen because it is counter-based, so the
draw for any element is a pure function of (seed, element index).
"""
import numpy as np

MASK32 = np.uint64(0xFFFFFFFF)
M0 = np.uint64(0xD2511F53)
M1 = np.uint64(0xCD9E8D57)
W0 = np.uint64(0x9E3779B9)
W1 = np.uint64(0xBB67AE85)


def philox4x32_10(counters, key):
    """Philox4x32-10 of every counter under one key.

    counters: uint32 array of shape (N, 4) -- (c0, c1, c2, c3) per row.
    key:      pair of uint32 (k0, k1).
    Returns a uint32 array of shape (N, 4).
    """
    ctr = np.asarray(counters, dtype=np.uint64).reshape(-1, 4)
    c0, c1, c2, c3 = (ctr[:, i].copy() for i in range(4))
    k0 = np.uint64(int(key[0]) & 0xFFFFFFFF)
    k1 = np.uint64(int(key[1]) & 0xFFFFFFFF)
    for rnd in range(10):
        if rnd > 0:
            k0 = (k0 + W0) & MASK32
            k1 = (k1 + W1) & MASK32
        p0 = c0 * M0          # exact: both factors < 2^32, product < 2^64
        p1 = c2 * M1
        hi0, lo0 = p0 >> np.uint64(32), p0 & MASK32
        hi1, lo1 = p1 >> np.uint64(32), p1 & MASK32
        c0, c1, c2, c3 = (hi1 ^ c1 ^ k0), lo1, (hi0 ^ c3 ^ k1), lo0
    return np.stack([c0, c1, c2, c3], axis=1).astype(np.uint32)


def split_seed(seed):
    """64-bit seed -> Philox key (low word, high word)."""
    seed = int(seed) & 0xFFFFFFFFFFFFFFFF
    return (seed & 0xFFFFFFFF, seed >> 32)
