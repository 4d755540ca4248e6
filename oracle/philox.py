"""Philox4x64-10 counter-based generator, written from its published definition.

Source: J. Salmon, M. Moraes, R. Dror, D. Shaw, "Parallel Random Numbers: As Easy as
1, 2, 3", SC'11 -- the Philox-4x64 bijection with 10 rounds: each round multiplies
words 0 and 2 by two fixed odd constants, keeps the 128-bit products' halves,
XORs the high halves with the other two words and the round key, and permutes;
the two key words are bumped by Weyl constants between rounds.

Test infrastructure (oracle side): the HIP library carries its own implementation.
Pinned in tests against ``numpy.random.Philox`` (the same bijection; numpy advances
its counter by one before producing each block of four words).
"""
from __future__ import annotations

import numpy as np

_M0 = np.uint64(0xD2E7470EE14C6C93)
_M1 = np.uint64(0xCA5A826395121157)
_W0 = np.uint64(0x9E3779B97F4A7C15)
_W1 = np.uint64(0xBB67AE8584CAA73B)
_LO32 = np.uint64(0xFFFFFFFF)
_S32 = np.uint64(32)

# Stream identifiers (second key word).
STREAM_DRAFT = 1
STREAM_ACCEPT = 2
STREAM_RESID = 3
STREAM_AR = 4


def _mulhilo(a: np.ndarray, m: np.uint64):
    """Full 64x64 -> 128-bit product of uint64 arrays by a constant, via 32-bit halves."""
    a0, a1 = a & _LO32, a >> _S32
    m0, m1 = m & _LO32, m >> _S32
    t = a0 * m0
    u = a1 * m0 + (t >> _S32)
    v = a0 * m1 + (u & _LO32)
    hi = a1 * m1 + (u >> _S32) + (v >> _S32)
    lo = a * m
    return hi, lo


def philox4x64(counter, key, rounds: int = 10) -> np.ndarray:
    """Apply the bijection to counters ``[..., 4]`` (uint64) under key ``[2]`` (or ``[..., 2]``).

    Returns ``[..., 4]`` uint64 output words.
    """
    with np.errstate(over="ignore"):
        c = np.array(counter, dtype=np.uint64, copy=True)
        k = np.array(key, dtype=np.uint64, copy=True)
        x0, x1, x2, x3 = c[..., 0], c[..., 1], c[..., 2], c[..., 3]
        k0, k1 = k[..., 0], k[..., 1]
        for r in range(rounds):
            if r > 0:
                k0 = k0 + _W0
                k1 = k1 + _W1
            hi0, lo0 = _mulhilo(x0, _M0)
            hi1, lo1 = _mulhilo(x2, _M1)
            x0, x1, x2, x3 = hi1 ^ x1 ^ k0, lo1, hi0 ^ x3 ^ k1, lo0
        return np.stack([x0, x1, x2, x3], axis=-1)


def words_to_uniform(w: np.ndarray) -> np.ndarray:
    """Top 23 bits -> u = (j + 1/2) * 2^-23 in (0, 1); exact in both FP32 and FP64."""
    j = (np.asarray(w, dtype=np.uint64) >> np.uint64(41)).astype(np.float64)
    return (j + 0.5) * (2.0 ** -23)


def uniforms(seed: int, stream: int, index, c1, c2, c3) -> np.ndarray:
    """Uniform for item ``index`` of a draw: counter (index // 4, c1, c2, c3), word index % 4.

    This is the one counter layout every randomised step uses.  All of ``index, c1, c2,
    c3`` broadcast against each other.  Draft sampling: index = block slot, c1 = vocabulary
    id; acceptance: index = slot, c1 = 0; residual: index = vocabulary id, c1 = 0; in all
    three c2 = the sequence's round counter and c3 = its sequence id.  The stream is the
    second key word, the seed the first.
    """
    index, c1, c2, c3 = np.broadcast_arrays(*(np.asarray(a, dtype=np.int64) for a in (index, c1, c2, c3)))
    ctr = np.stack([(index // 4), c1, c2, c3], axis=-1).astype(np.uint64)
    key = np.array([seed, stream], dtype=np.uint64)
    words = philox4x64(ctr, key)
    w = np.take_along_axis(words, (index % 4)[..., None], axis=-1)[..., 0]
    return words_to_uniform(w)
