"""16-point random Hadamard transform of the columnwise (wgrad) operand (CPU oracle; test only).

P1, PR description: the columnwise operand built at the receiver is an "RHT"
operand.  P4, description: after the transform the columnwise amax is bounded
by four times the rowwise amax, which is the bound for a 16-point transform
normalised by 1/4 (each output is a quarter of a signed sum of 16 inputs).

R15 (reading): y = (1/4) * H16 * D * z over 16 consecutive grouped rows of one
column, where H16 is the 16x16 Sylvester Hadamard matrix and D = diag(d) a
fixed pseudo-random sign vector.  Computed in float32 as:

1. z'_i = fl32(d_i * z_i / 4)   (exact unless below float32's normal range);
2. butterfly, strides h = 1, 2, 4, 8 in that order: for every i with
   (i & h) == 0, (z'_i, z'_{i+h}) <- (fl32(z'_i + z'_{i+h}), fl32(z'_i - z'_{i+h})).

The sign vector: d_i = -1 iff bit i of M is set, M = the low 16 bits of word 0
of Philox4x32-10 at key (0, 0), counter (0, 0, 0, 0).  M is a fixed constant
chosen by this reading (parity unpinned for the choice itself); the tests pin
that it is not a row of +-H16, which would collapse the transform.
"""

import numpy as np

from .philox import philox4x32_10


def sign_mask():
    w = philox4x32_10(0, 0, 0, 0, 0, 0)[0]
    return int(w) & 0xFFFF


def signs():
    m = sign_mask()
    return np.array([-1.0 if (m >> i) & 1 else 1.0 for i in range(16)], dtype=np.float64)


def rht16(z):
    """z [..., 16] (float32 values or exact float64 values) -> y [..., 16] float32."""
    z = np.asarray(z, dtype=np.float64)
    if z.shape[-1] != 16:
        raise ValueError("last axis must be 16")
    y = (z * (signs() * 0.25)).astype(np.float32)       # exact product, one rounding to float32
    for h in (1, 2, 4, 8):
        y = y.copy()
        for i in range(16):
            if i & h:
                continue
            a = y[..., i].copy()
            b = y[..., i + h].copy()
            y[..., i] = a + b                                # float32 + float32 -> float32 (RN)
            y[..., i + h] = a - b
    return y
