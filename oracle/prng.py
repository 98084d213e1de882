"""Random state of the method: rotation signs and the QJL matrix S.

The pages only require that the sign pattern of the rotation and the QJL
projection come from independent random sources ("turbo4 post-mortem",
section 10: QJL only worked once its rotation used an independent seed).
They give no generator, so both are drawn from splitmix64 (Steele, Lea and
Flood, "Fast splittable pseudorandom number generators", OOPSLA 2014), which
is counter based: output i of the stream seeded with s is mix(s + (i+1)*G).

* sign j of the rotation is -1 when bit 63 of output j is set, else +1;
* S is d x d, row-major, N(0, 1) entries; entries 2t and 2t+1 come from the
  Box-Muller transform of outputs 2t and 2t+1, each mapped to a uniform in
  (0, 1) as ((x >> 11) + 0.5) * 2**-53, evaluated in double precision and
  rounded to fp32.

Written with Python integers and the ``math`` module, value by value.
"""

import math

import numpy as np

MASK64 = (1 << 64) - 1
GOLDEN_GAMMA = 0x9E3779B97F4A7C15


def splitmix64(seed, n):
    """First n outputs of the splitmix64 stream seeded with ``seed``."""
    out = []
    state = seed & MASK64
    for _ in range(n):
        state = (state + GOLDEN_GAMMA) & MASK64
        z = state
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK64
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK64
        out.append(z ^ (z >> 31))
    return out


def rotation_signs(seed, d):
    """float64 vector of +-1: -1 where bit 63 of output j is set."""
    return np.array([-1.0 if (x >> 63) else 1.0 for x in splitmix64(seed, d)])


def _unit(x):
    return ((x >> 11) + 0.5) * (2.0 ** -53)


def qjl_matrix(seed, d):
    """d x d matrix with N(0, 1) entries, fp32, row-major, via Box-Muller."""
    n = d * d
    xs = splitmix64(seed, n)
    vals = []
    for t in range(n // 2):
        u1 = _unit(xs[2 * t])
        u2 = _unit(xs[2 * t + 1])
        r = math.sqrt(-2.0 * math.log(u1))
        a = 2.0 * math.pi * u2
        vals.append(r * math.cos(a))
        vals.append(r * math.sin(a))
    return np.array(vals, dtype=np.float64).astype(np.float32).reshape(d, d)
