"""Counter-based noise for the oracle: Philox4x32-10 and the uniform/Gumbel maps.

TEST INFRASTRUCTURE. This module belongs to the CPU oracle. Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it; the product path never does.

The pages say the Gumbel-Softmax relaxation draws noise for every coordinate
(GSQ paper page at agihunt.info, method paragraph; GSQ abstract on
thelatestinai.com) but name no generator. The generator used here is the
published counter-based Philox4x32 with 10 rounds (Salmon, Moraes, Dror, Shaw,
"Parallel random numbers: as easy as 1, 2, 3", SC'11), written from that
definition in NumPy 64-bit integer arithmetic:

* state: a 128-bit counter (four 32-bit words c0..c3) and a 64-bit key (k0, k1);
* one round: the two 32x32->64 products M0*c0 and M1*c2 give (hi0, lo0) and
  (hi1, lo1); the new counter is (hi1^c1^k0, lo1, hi0^c3^k1, lo0);
* between rounds the key is bumped by the Weyl constants (W0, W1);
* ten rounds give one block of four output words.

Noise stream layout (a convention of this implementation, the same one the
GPU library documents): element ``e`` of the stream for (seed, stream, step)
is word ``e & 3`` of the block whose counter is
``(lo32(e >> 2), hi32(e >> 2), step, stream)`` and whose key is
``(lo32(seed), hi32(seed))``.
"""

from __future__ import annotations

import numpy as np

PHILOX_M0 = 0xD2511F53
PHILOX_M1 = 0xCD9E8D57
PHILOX_W0 = 0x9E3779B9
PHILOX_W1 = 0xBB67AE85

_MASK32 = np.uint64(0xFFFFFFFF)


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Ten Philox4x32 rounds on arrays of 32-bit counters.

    Arguments are broadcastable integer arrays holding 32-bit values (the key
    may be Python ints). Returns four ``uint32`` arrays, the output block.
    """
    c0 = np.asarray(c0, dtype=np.uint64) & _MASK32
    c1 = np.asarray(c1, dtype=np.uint64) & _MASK32
    c2 = np.asarray(c2, dtype=np.uint64) & _MASK32
    c3 = np.asarray(c3, dtype=np.uint64) & _MASK32
    k0 = int(k0) & 0xFFFFFFFF
    k1 = int(k1) & 0xFFFFFFFF
    m0 = np.uint64(PHILOX_M0)
    m1 = np.uint64(PHILOX_M1)
    for _ in range(10):
        # 32x32 -> 64-bit products are exact in uint64.
        p0 = m0 * c0
        p1 = m1 * c2
        hi0, lo0 = p0 >> np.uint64(32), p0 & _MASK32
        hi1, lo1 = p1 >> np.uint64(32), p1 & _MASK32
        c0, c1, c2, c3 = (hi1 ^ c1 ^ np.uint64(k0), lo1,
                          hi0 ^ c3 ^ np.uint64(k1), lo0)
        k0 = (k0 + PHILOX_W0) & 0xFFFFFFFF
        k1 = (k1 + PHILOX_W1) & 0xFFFFFFFF
    return tuple(x.astype(np.uint32) for x in (c0, c1, c2, c3))


def noise_words(seed: int, stream: int, step: int, e) -> np.ndarray:
    """Raw 32-bit words of the noise stream at flat element indices ``e``."""
    e = np.asarray(e, dtype=np.uint64)
    blk = e >> np.uint64(2)
    word = (e & np.uint64(3)).astype(np.int64)
    seed = int(seed) & 0xFFFFFFFFFFFFFFFF
    out = philox4x32_10(blk & _MASK32, blk >> np.uint64(32),
                        np.uint64(int(step) & 0xFFFFFFFF),
                        np.uint64(int(stream) & 0xFFFFFFFF),
                        seed & 0xFFFFFFFF, seed >> 32)
    stacked = np.stack(np.broadcast_arrays(*out), axis=0)
    return np.take_along_axis(stacked, word[None, ...], axis=0)[0]


def uniform_from_word(x) -> np.ndarray:
    """Map a 32-bit word to a uniform in (0, 1).

    The top 24 bits, forced odd, times 2**-24: an odd multiple of 2**-24 in
    [2**-24, 1 - 2**-24]. Both u and 1 - u are exact in fp32 and fp64, and the
    value is never 0 or 1, so both logarithms below stay finite.
    """
    x = np.asarray(x, dtype=np.uint32)
    return ((x >> np.uint32(8)) | np.uint32(1)).astype(np.float64) * 2.0 ** -24


def gumbel(u) -> np.ndarray:
    """Standard Gumbel by inversion: -ln(-ln u), in fp64."""
    u = np.asarray(u, dtype=np.float64)
    return -np.log(-np.log(u))


def logistic(u) -> np.ndarray:
    """Standard logistic by inversion: ln u - ln(1 - u), in fp64.

    This is the law of the difference of two independent Gumbels, so a
    sigmoid of (l + n)/tau is exactly the two-way Gumbel-Softmax with logits
    (l, 0).
    """
    u = np.asarray(u, dtype=np.float64)
    return np.log(u) - np.log(1.0 - u)
