"""Sign-and-Hadamard rotations (oracle side).

exllamav3 #284 (API contract) says each projection carries suh/svh rotations
that residual stages reuse; TensorFold #837 (What this changes) applies the
input rotation before the decode-and-multiply and rotates each expert. The
pages do not give the transform's size or normalisation. This library reads
it as the orthonormal Sylvester Hadamard of order 128, H[i][j] =
(-1)^popcount(i & j) / sqrt(128), applied to each contiguous 128-block of a
vector; dimensions that are not multiples of 128 are rejected.
"""

import numpy as np

BLOCK = 128


def hadamard_matrix(n=BLOCK):
    """Orthonormal Sylvester Hadamard matrix of order n from its definition."""
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    v = np.bitwise_and(i, j)
    pc = np.zeros_like(v)
    while np.any(v):
        pc += v & 1
        v >>= 1
    return np.where(pc % 2 == 0, 1.0, -1.0) / np.sqrt(n)


_H = hadamard_matrix()


def rotate_blocks(v):
    """Apply H to every contiguous 128-block of the last axis (float64)."""
    v = np.asarray(v, dtype=np.float64)
    n = v.shape[-1]
    if n % BLOCK:
        raise ValueError("dimension %d is not a multiple of %d" % (n, BLOCK))
    blocks = v.reshape(v.shape[:-1] + (n // BLOCK, BLOCK))
    # H is symmetric, so row-vector times H is the transform of each block.
    return (blocks @ _H).reshape(v.shape)
