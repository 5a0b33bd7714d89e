"""QJL random projection: the Gaussian matrix S and the estimator scale.

Method ([C] "TurboQuantization", K-cache step 5; [A] "KVキャッシュ圧縮の内訳",
step 5): the key residual is projected by a random Johnson-Lindenstrauss
matrix and only the signs are kept.  The pages give neither the generator of
S nor the estimator that uses the signs; the readings taken are:

  * S is m x d with iid N(0, 1) entries, m = d = 128, one S shared by every
    head, rounded once to float32.  It is drawn from SplitMix64 (Steele, Lea
    and Flood, "Fast splittable pseudorandom number generators", OOPSLA 2014;
    the constants of Vigna's public-domain splitmix64.c) turned into normals
    by the Box-Muller transform (Box and Muller, 1958) in float64: output
    pair k uses uniforms u1 = U(2k), u2 = U(2k+1) and yields
    r*cos(2*pi*u2), r*sin(2*pi*u2) with r = sqrt(-2 ln u1); S is filled
    row-major from that stream.  Uniform U(n) = ((x_n >> 11) + 0.5) * 2^-53.
  * Estimator: for s ~ N(0, I), E[<s, q> sign(<s, r>)] = sqrt(2/pi) <q, r>/|r|,
    so <q, r> is estimated without bias by
        sqrt(pi/2)/m * |r| * sum_i (S q)_i * sign((S r)_i).
    ``qjl_alpha(m)`` returns sqrt(pi/2)/m.
  * sign(0) = +1.
"""

from __future__ import annotations

import math

import numpy as np

_MASK64 = (1 << 64) - 1
_GOLDEN_GAMMA = 0x9E3779B97F4A7C15


def splitmix64_stream(seed: int, n: int) -> list[int]:
    """First ``n`` outputs of SplitMix64 started at state ``seed``."""
    out = []
    state = seed & _MASK64
    for _ in range(n):
        state = (state + _GOLDEN_GAMMA) & _MASK64
        z = state
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _MASK64
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _MASK64
        z = z ^ (z >> 31)
        out.append(z)
    return out


def _uniform_open01(x: int) -> float:
    return ((x >> 11) + 0.5) * (2.0 ** -53)


def gaussian_matrix(seed: int, m: int = 128, d: int = 128) -> np.ndarray:
    """S (m x d, float32) from SplitMix64 + Box-Muller, row-major fill."""
    count = m * d
    pairs = (count + 1) // 2
    raw = splitmix64_stream(seed, 2 * pairs)
    vals = []
    for k in range(pairs):
        u1 = _uniform_open01(raw[2 * k])
        u2 = _uniform_open01(raw[2 * k + 1])
        r = math.sqrt(-2.0 * math.log(u1))
        th = 2.0 * math.pi * u2
        vals.append(r * math.cos(th))
        vals.append(r * math.sin(th))
    return np.array(vals[:count], dtype=np.float64).reshape(m, d).astype(np.float32)


def qjl_alpha(m: int = 128) -> float:
    """Scale of the sign estimator: sqrt(pi/2) / m."""
    return math.sqrt(math.pi / 2.0) / m
