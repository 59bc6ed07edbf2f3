"""Philox4x32-10 counter-based generator and the uniform mapping (CPU oracle).

TEST INFRASTRUCTURE: see the package docstring.

Algorithm and constants: Salmon, Moraes, Dror and Shaw, "Parallel Random
Numbers: As Easy as 1, 2, 3" (SC'11), the Philox-4x32 bijection with 10
rounds.  One round maps counter (c0, c1, c2, c3) and key (k0, k1) to

    (hi(M1*c2) ^ c1 ^ k0,  lo(M1*c2),  hi(M0*c0) ^ c3 ^ k1,  lo(M0*c0))

with M0 = 0xD2511F53, M1 = 0xCD9E8D57; between rounds the key is bumped by the
Weyl constants W0 = 0x9E3779B9, W1 = 0xBB67AE85 (mod 2**32).

Stream convention (the pages name a per-request Philox state whose offset picks
the request's own subsequence -- TensorRT-LLM speculative/interface.py,
``rejection_sampling_one_model`` docstring -- but give no word layout; this is
our reading):

    key     = (lo32(seed), hi32(seed))
    counter = (lo32(n), hi32(n), lo32(s), hi32(s))   n = block, s = subsequence
    word(seed, s, t) = block(seed, s, t // 4)[t % 4]

The uniform of a word w is u(w) = (2 * (w >> 9) + 1) * 2**-24, an odd multiple
of 2**-24 in [2**-24, 1 - 2**-24], exactly representable in float32.
"""
from __future__ import annotations

import numpy as np

M0 = 0xD2511F53
M1 = 0xCD9E8D57
W0 = 0x9E3779B9
W1 = 0xBB67AE85
_MASK32 = 0xFFFFFFFF
_MASK64 = (1 << 64) - 1


def philox4x32_10(counter, key):
    """One Philox4x32-10 block on Python ints: 4 counter words, 2 key words -> 4 words."""
    c0, c1, c2, c3 = (int(c) & _MASK32 for c in counter)
    k0, k1 = (int(k) & _MASK32 for k in key)
    for rnd in range(10):
        if rnd:
            k0 = (k0 + W0) & _MASK32
            k1 = (k1 + W1) & _MASK32
        prod0 = M0 * c0
        prod1 = M1 * c2
        c0, c1, c2, c3 = (
            ((prod1 >> 32) ^ c1 ^ k0) & _MASK32,
            prod1 & _MASK32,
            ((prod0 >> 32) ^ c3 ^ k1) & _MASK32,
            prod0 & _MASK32,
        )
    return c0, c1, c2, c3


def word(seed: int, subseq: int, t: int) -> int:
    """Word ``t`` of the stream (seed, subsequence), Python-int version."""
    seed &= _MASK64
    subseq &= _MASK64
    n = t // 4
    blk = philox4x32_10(
        (n & _MASK32, n >> 32, subseq & _MASK32, subseq >> 32),
        (seed & _MASK32, seed >> 32),
    )
    return blk[t % 4]


def words(seed: int, subseq: int, count: int, start: int = 0) -> np.ndarray:
    """Words ``start .. start+count-1`` of stream (seed, subsequence) as uint32 (numpy)."""
    seed = int(seed) & _MASK64
    subseq = int(subseq) & _MASK64
    if count <= 0:
        return np.zeros(0, np.uint32)
    first, last = start // 4, (start + count - 1) // 4
    n = np.arange(first, last + 1, dtype=np.uint64)
    m32 = np.uint64(_MASK32)
    c0 = n & m32
    c1 = n >> np.uint64(32)
    c2 = np.full_like(n, subseq & _MASK32)
    c3 = np.full_like(n, subseq >> 32)
    k0, k1 = seed & _MASK32, seed >> 32
    for rnd in range(10):
        if rnd:
            k0 = (k0 + W0) & _MASK32
            k1 = (k1 + W1) & _MASK32
        prod0 = np.uint64(M0) * c0
        prod1 = np.uint64(M1) * c2
        c0, c1, c2, c3 = (
            (prod1 >> np.uint64(32)) ^ c1 ^ np.uint64(k0),
            prod1 & m32,
            (prod0 >> np.uint64(32)) ^ c3 ^ np.uint64(k1),
            prod0 & m32,
        )
    blocks = np.stack([c0, c1, c2, c3], axis=1).reshape(-1).astype(np.uint32)
    off = start - first * 4
    return blocks[off:off + count]


def uniform(w) -> np.ndarray:
    """u(w) = (2 * (w >> 9) + 1) * 2**-24 as float64 (exact; also exact in float32)."""
    w = np.asarray(w, dtype=np.uint64)
    return ((w >> np.uint64(9)) * np.uint64(2) + np.uint64(1)).astype(np.float64) * 2.0 ** -24


def uniform_code(w) -> np.ndarray:
    """The odd integer 2 * (w >> 9) + 1, so that u = code * 2**-24 exactly."""
    w = np.asarray(w, dtype=np.uint64)
    return (w >> np.uint64(9)) * np.uint64(2) + np.uint64(1)
