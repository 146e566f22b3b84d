"""Oracle: the Philox4x64-10 counter-based generator.

Published definition: J. K. Salmon, M. A. Moraes, R. O. Dror, D. E. Shaw,
"Parallel Random Numbers: As Easy as 1, 2, 3", SC'11, section 4 (Philox), with the
4x64 multipliers and Weyl key increments given there.  Waterfill samples the shared
expert's rank at random (Waterfill/LPLB blog, section "Waterfill算法执行步骤"); the
pages name no generator, so this counter-based one is the reading (one draw per
token, counter = (token, 0, 0, 0), key = (seed, layer)).  LPLB's dispatch-time copy
draw (blog section "从LP解决方案到Token调度") uses counter (token, slot, 1, 0), the
same key.

Pins: numpy.random.Philox (an independent implementation of the same generator)
at many counters and keys, and the scalar and vectorised forms against each other.
"""

import numpy as np

_M0 = 0xD2E7470EE14C6C93
_M1 = 0xCA5A826395121157
_W0 = 0x9E3779B97F4A7C15
_W1 = 0xBB67AE8584CAA73B
_MASK = (1 << 64) - 1


def philox4x64_10(counter, key):
    """Four 64-bit words for a 4-word counter and 2-word key (Python ints)."""
    c0, c1, c2, c3 = (int(v) & _MASK for v in counter)
    k0, k1 = (int(v) & _MASK for v in key)
    for _ in range(10):
        p0 = _M0 * c0
        p1 = _M1 * c2
        c0, c1, c2, c3 = ((p1 >> 64) ^ c1 ^ k0, p1 & _MASK, (p0 >> 64) ^ c3 ^ k1, p0 & _MASK)
        k0 = (k0 + _W0) & _MASK
        k1 = (k1 + _W1) & _MASK
    return c0, c1, c2, c3


def _mulhilo(a: np.ndarray, m: int):
    """64x64 -> 128-bit product of a uint64 array with a constant, as (hi, lo)."""
    lo32 = np.uint64(0xFFFFFFFF)
    s32 = np.uint64(32)
    a_lo, a_hi = a & lo32, a >> s32
    m_lo, m_hi = np.uint64(m & 0xFFFFFFFF), np.uint64(m >> 32)
    ll, lh, hl, hh = a_lo * m_lo, a_lo * m_hi, a_hi * m_lo, a_hi * m_hi
    mid = (ll >> s32) + (lh & lo32) + (hl & lo32)
    hi = hh + (lh >> s32) + (hl >> s32) + (mid >> s32)
    lo = (mid << s32) | (ll & lo32)
    return hi, lo


def philox4x64_10_np(c0: np.ndarray, key, c1=0, c2=0, c3=0) -> np.ndarray:
    """Word 0..3 for counters (c0[i], c1[i], c2[i], c3[i]) (c1..c3 arrays or scalars,
    default 0); returns uint64 [n][4]."""
    c0 = np.asarray(c0, dtype=np.uint64)
    c1 = np.broadcast_to(np.asarray(c1, dtype=np.uint64), c0.shape).copy()
    c2 = np.broadcast_to(np.asarray(c2, dtype=np.uint64), c0.shape).copy()
    c3 = np.broadcast_to(np.asarray(c3, dtype=np.uint64), c0.shape).copy()
    k0, k1 = int(key[0]) & _MASK, int(key[1]) & _MASK
    with np.errstate(over="ignore"):
        for _ in range(10):
            hi0, lo0 = _mulhilo(c0, _M0)
            hi1, lo1 = _mulhilo(c2, _M1)
            c0, c1, c2, c3 = hi1 ^ c1 ^ np.uint64(k0), lo1, hi0 ^ c3 ^ np.uint64(k1), lo0
            k0 = (k0 + _W0) & _MASK
            k1 = (k1 + _W1) & _MASK
    return np.stack([c0, c1, c2, c3], axis=1)
