"""Philox4x32-10 counter-based generator and the 53-bit uniform built from it (oracle side).

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import this module; only ``tests/``,
``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` use it.

The pages fix no generator: "Stochastic Sparse Attention for Memory-Bound Inference" only says
that kernels take a seed and draw offsets a0 ~ U(0,1) (Appendix O, Algorithm 4; Appendix P,
Algorithm 7). The reading taken here is Philox4x32 with 10 rounds, as published by Salmon, Moraes,
Dror and Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3" (SC'11): a 4x32-bit counter, a 2x32-bit
key, two 32x32->64 multiplies per round, and a Weyl-sequence key schedule.

Counter/key convention (shared by definition, not by code, with the GPU path):
    key     = (seed mod 2^32, seed >> 32)
    counter = (m, h, b, tag)
        tag 0: the m-th point of i.i.d. / stratified sampling of query head h, batch b
        tag 1: the single systematic offset of (b, h) (m = 0)
        tag 2 + 256*n: Bernoulli decision for query element m, Bernoulli sample n
    u53     = ((x0 << 32 | x1) >> 11) * 2^-53, an exact double in [0, 1)
"""

from __future__ import annotations

import numpy as np

# Round multipliers and key increments from the Philox publication (SC'11, Section 5).
PHILOX_M0 = 0xD2511F53
PHILOX_M1 = 0xCD9E8D57
PHILOX_W0 = 0x9E3779B9
PHILOX_W1 = 0xBB67AE85
ROUNDS = 10

TAG_POINT = 0
TAG_SYS = 1
TAG_BERNOULLI = 2

_MASK = np.uint64(0xFFFFFFFF)


def _u64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.uint64) & _MASK


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Philox4x32-10 bijection applied elementwise to broadcastable counter words.

    Each round: the products M0*c0 and M1*c2 are split into (hi, lo) halves, and the new counter is
    (hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0); the key advances by (W0, W1) between rounds.
    Returns four uint32 arrays.
    """
    c0, c1, c2, c3 = (_u64(c) for c in (c0, c1, c2, c3))
    c0, c1, c2, c3 = np.broadcast_arrays(c0, c1, c2, c3)
    k0 = _u64(k0)
    k1 = _u64(k1)
    m0 = np.uint64(PHILOX_M0)
    m1 = np.uint64(PHILOX_M1)
    for r in range(ROUNDS):
        if r:
            k0 = (k0 + np.uint64(PHILOX_W0)) & _MASK
            k1 = (k1 + np.uint64(PHILOX_W1)) & _MASK
        p0 = m0 * c0  # < 2^64: exact in uint64
        p1 = m1 * c2
        hi0, lo0 = p0 >> np.uint64(32), p0 & _MASK
        hi1, lo1 = p1 >> np.uint64(32), p1 & _MASK
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return tuple(x.astype(np.uint32) for x in (c0, c1, c2, c3))


def seed_key(seed: int):
    seed = int(seed) & 0xFFFFFFFFFFFFFFFF
    return seed & 0xFFFFFFFF, seed >> 32


def u53_from_words(x0, x1) -> np.ndarray:
    """53-bit uniform in [0, 1): top 53 bits of the 64-bit word (x0:x1), scaled by 2^-53 (exact)."""
    w = (np.asarray(x0, dtype=np.uint64) << np.uint64(32)) | np.asarray(x1, dtype=np.uint64)
    return (w >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)


def uniforms(seed: int, m, h: int, b: int, tag: int) -> np.ndarray:
    """u53 for counters (m, h, b, tag) under key(seed); m may be an array."""
    k0, k1 = seed_key(seed)
    x0, x1, _, _ = philox4x32_10(m, h, b, tag, k0, k1)
    return u53_from_words(x0, x1)
