"""Philox4x32-10 counter-based generator (CPU oracle; test only).

R9.  The pages ask for stochastic rounding "per the recipe" in the combine
backward (P1, PR description) and say nothing about the generator; the
generator is fixed here as Philox4x32 with 10 rounds, as published by Salmon,
Moraes, Dror and Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3" (SC'11):

* state: a 128-bit counter (c0, c1, c2, c3) and a 64-bit key (k0, k1);
* one round: (hi0, lo0) = M0 * c0 and (hi1, lo1) = M1 * c2 as full 64-bit
  products, then (c0, c1, c2, c3) <- (hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0),
  with M0 = 0xD2511F53 and M1 = 0xCD9E8D57;
* between consecutive rounds the key advances by the Weyl constants
  (k0 += 0x9E3779B9, k1 += 0xBB67AE85, modulo 2^32);
* the output block is the counter after the tenth round.
"""

import numpy as np

M0 = 0xD2511F53
M1 = 0xCD9E8D57
W0 = 0x9E3779B9
W1 = 0xBB67AE85
_MASK = np.uint64(0xFFFFFFFF)


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Vectorised Philox4x32-10.  All arguments broadcast; returns 4 uint32 arrays."""
    c = [np.asarray(v, dtype=np.uint64) & _MASK for v in (c0, c1, c2, c3)]
    k0 = np.asarray(k0, dtype=np.uint64) & _MASK
    k1 = np.asarray(k1, dtype=np.uint64) & _MASK
    c = list(np.broadcast_arrays(*c, k0, k1))
    k0, k1 = c[4].copy(), c[5].copy()
    c = [v.copy() for v in c[:4]]
    for rnd in range(10):
        if rnd > 0:
            k0 = (k0 + np.uint64(W0)) & _MASK
            k1 = (k1 + np.uint64(W1)) & _MASK
        p0 = np.uint64(M0) * c[0]          # < 2^64, exact in uint64
        p1 = np.uint64(M1) * c[2]
        hi0, lo0 = p0 >> np.uint64(32), p0 & _MASK
        hi1, lo1 = p1 >> np.uint64(32), p1 & _MASK
        c = [hi1 ^ c[1] ^ k0, lo1, hi0 ^ c[3] ^ k1, lo0]
    return tuple(v.astype(np.uint32) for v in c)


def sr_word(n, seed, mode="element"):
    """The 32-bit random word used by stochastic rounding of stream position n.

    R8.  key = (seed mod 2^32, seed >> 32).
    * mode "element" (the default, the literal reading of "counter =
      row*hidden + col"): counter = (n mod 2^32, n >> 32, 0, 0), word 0.
    * mode "stream": n indexes the stream of 32-bit outputs, four per block:
      counter = (b mod 2^32, b >> 32, 0, 0) with b = n >> 2, word n & 3.
    """
    n = np.asarray(n, dtype=np.uint64)
    seed = int(seed)
    k0, k1 = seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF
    if mode == "element":
        w = philox4x32_10(n & _MASK, n >> np.uint64(32), 0, 0, k0, k1)
        return w[0]
    if mode == "stream":
        b = n >> np.uint64(2)
        w = philox4x32_10(b & _MASK, b >> np.uint64(32), 0, 0, k0, k1)
        sel = (n & np.uint64(3)).astype(np.int64)
        return np.choose(sel, w).astype(np.uint32)
    raise ValueError(mode)
