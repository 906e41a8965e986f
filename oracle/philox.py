"""Philox4x64-10 counter-based generator (test infrastructure only).

Written from the published definition: J. K. Salmon, M. A. Moraes, R. O. Dror,
D. E. Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3", SC'11 - Philox with
N=4 words of W=64 bits, 10 rounds.  One round maps (x0,x1,x2,x3) with key
(k0,k1) to (hi(M1*x2) ^ x1 ^ k0, lo(M1*x2), hi(M0*x0) ^ x3 ^ k1, lo(M0*x0));
the key is bumped by the Weyl constants between rounds.

Uniforms.  The verifier draws u = (w0 >> 40) * 2^-24 from output word 0 of
counter (seq, node, event, 0) under key (seed, round): a value on the 2^-24
grid in [0, 1), exactly representable in fp32 and fp64.  event i < 64 is the
test of a node's i-th child; event 64 is the correction / bonus draw.
"""
from __future__ import annotations

import numpy as np

M0 = 0xD2E7470EE14C6C93
M1 = 0xCA5A826395121157
W0 = 0x9E3779B97F4A7C15
W1 = 0xBB67AE8584CAA73B
MASK64 = (1 << 64) - 1
EVENT_DRAW = 64


def philox4x64_10(counter, key):
    """Scalar reference on Python integers: returns 4 uint64 words."""
    x0, x1, x2, x3 = (int(c) & MASK64 for c in counter)
    k0, k1 = (int(k) & MASK64 for k in key)
    for rnd in range(10):
        if rnd:
            k0 = (k0 + W0) & MASK64
            k1 = (k1 + W1) & MASK64
        p0 = M0 * x0
        p1 = M1 * x2
        hi0, lo0 = p0 >> 64, p0 & MASK64
        hi1, lo1 = p1 >> 64, p1 & MASK64
        x0, x1, x2, x3 = hi1 ^ x1 ^ k0, lo1, hi0 ^ x3 ^ k1, lo0
    return x0, x1, x2, x3


def _mulhilo64(a: np.ndarray, b: int):
    """Full 128-bit product of uint64 arrays a and constant b, as (hi, lo)."""
    a = a.astype(np.uint64)
    mask32 = np.uint64(0xFFFFFFFF)
    a_lo, a_hi = a & mask32, a >> np.uint64(32)
    b_lo, b_hi = np.uint64(b & 0xFFFFFFFF), np.uint64(b >> 32)
    ll = a_lo * b_lo
    lh = a_lo * b_hi
    hl = a_hi * b_lo
    hh = a_hi * b_hi
    mid = (ll >> np.uint64(32)) + (lh & mask32) + (hl & mask32)
    lo = (ll & mask32) | ((mid & mask32) << np.uint64(32))
    hi = hh + (lh >> np.uint64(32)) + (hl >> np.uint64(32)) + (mid >> np.uint64(32))
    return hi, lo


def philox4x64_10_np(c0, c1, c2, c3, key):
    """Vectorised version over arrays of counters (same key)."""
    with np.errstate(over="ignore"):
        x0, x1, x2, x3 = (np.asarray(c, dtype=np.uint64).copy() for c in (c0, c1, c2, c3))
        x0, x1, x2, x3 = np.broadcast_arrays(x0, x1, x2, x3)
        k0, k1 = np.uint64(int(key[0]) & MASK64), np.uint64(int(key[1]) & MASK64)
        for rnd in range(10):
            if rnd:
                k0 = np.uint64((int(k0) + W0) & MASK64)
                k1 = np.uint64((int(k1) + W1) & MASK64)
            hi0, lo0 = _mulhilo64(x0, M0)
            hi1, lo1 = _mulhilo64(x2, M1)
            x0, x1, x2, x3 = hi1 ^ x1 ^ k0, lo1, hi0 ^ x3 ^ k1, lo0
    return x0, x1, x2, x3


def uniform(seed: int, rnd: int, seq: int, node: int, event: int) -> float:
    w0 = philox4x64_10((seq, node, event, 0), (seed, rnd))[0]
    return float(w0 >> 40) * 2.0 ** -24


def uniforms_np(seed: int, rnd: int, seq, node, event) -> np.ndarray:
    w0 = philox4x64_10_np(seq, node, event, 0, (seed, rnd))[0]
    return (w0 >> np.uint64(40)).astype(np.float64) * 2.0 ** -24
