"""Random orthogonal rotation: Walsh-Hadamard transform after random signs.

The write path rotates each normalized vector before scalar quantization so
that every coordinate follows the same narrow law ("turbo4 post-mortem",
section 1: WHT-rotated vectors; section 9: FWHT; section 10: RHT, a
randomized Hadamard transform).  The pages fix neither the order of the sign
flip and the transform nor the normalization; the reading taken here is

    Pi = (1/sqrt(d)) * H_d * diag(s),      y = Pi u,      u = Pi^T y,

with H_d the Sylvester-ordered Hadamard matrix (H_1 = [1],
H_2n = [[H, H], [H, -H]]) and s the +-1 rotation signs.

The oracle materializes Pi as a dense float64 matrix and multiplies by it:
no fast transform, no blocking.
"""

import numpy as np


def hadamard(d):
    """Sylvester-ordered Hadamard matrix of order d (a power of two)."""
    if d < 1 or d & (d - 1):
        raise ValueError("d must be a power of two")
    h = np.ones((1, 1))
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h


def rotation_matrix(signs):
    """Pi = H diag(signs) / sqrt(d) as a dense float64 matrix."""
    signs = np.asarray(signs, dtype=np.float64)
    d = signs.shape[0]
    return hadamard(d) * signs[None, :] / np.sqrt(d)


def rotate(u, signs):
    """y = Pi u for each row u."""
    return np.asarray(u, dtype=np.float64) @ rotation_matrix(signs).T


def unrotate(y, signs):
    """u = Pi^T y for each row y (Pi is orthogonal)."""
    return np.asarray(y, dtype=np.float64) @ rotation_matrix(signs)
