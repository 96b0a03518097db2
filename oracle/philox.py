"""Philox4x32-10 counter-based generator and the dropout keep rule (oracle side).

TEST INFRASTRUCTURE: only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import this module.

The pages say dropout is fused into the attention kernel after the softmax and
before the product with V (FlashAttention explainer, azimuth.plus, "three ideas
in one kernel", kernel fusion; FlashAttention summary, xyznot.com, core ideas,
kernel fusion) but name no generator.  This oracle follows Philox-4xW-R from
Salmon, Moraes, Dror and Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3"
(SC'11), written from that paper's definition:

  one round on counter (c0, c1, c2, c3) with round key (k0, k1):
      (hi0, lo0) = M0 * c0          full 2W-bit product
      (hi1, lo1) = M1 * c2
      c <- (hi1 ^ c1 ^ k0,  lo1,  hi0 ^ c3 ^ k1,  lo0)
  after each round the key is bumped by the Weyl constants: k0 += W0, k1 += W1.

The Weyl constants are the golden ratio and sqrt(3) - 1 as W-bit fractions
(checked from those closed forms by the tests); M0 and M1 are the paper's
multipliers for each word width.

Counter layout and keep rule for attention element (b, h, i, j) -- a choice
of this library, which the FlashAttention explainer (kernel fusion, dropout)
leaves open.  One generator call decides a block of 4 keys x 2 query rows:
each of its four 32-bit output words holds two 16-bit uniforms, the low half
for the even row of the pair and the high half for the odd one:
  counter = (j >> 2, i >> 1, b*H + h, lo32(rng_offset)), key = (lo32(seed), hi32(seed))
  w = output word (j & 3),  u = (w >> 16) if i is odd else (w & 0xFFFF)
  keep iff u >= thr,  thr = min(floor(float32(p) * 2^16), 2^16 - 1)
so the drop probability is thr / 2^16, within 2^-16 of p.  Kept entries are
scaled by the inverse of the exact keep probability, 2^16 / (2^16 - thr),
whenever p > 0 (inverted dropout: each scaled keep bit has expectation 1, so
the expected dropped O equals the undropped one; the explainer names dropout
among the operations fused after the softmax but not its scaling).
"""

from __future__ import annotations

import numpy as np

PHILOX_M = {32: (0xD2511F53, 0xCD9E8D57),
            64: (0xD2E7470EE14C6C93, 0xCA5A826395121157)}
PHILOX_W = {32: (0x9E3779B9, 0xBB67AE85),
            64: (0x9E3779B97F4A7C15, 0xBB67AE8584CAA73B)}


def philox4_scalar(ctr, key, width=32, rounds=10):
    """Philox4xW-R on Python integers (exact 2W-bit products). Returns 4 words."""
    m0, m1 = PHILOX_M[width]
    w0, w1 = PHILOX_W[width]
    mask = (1 << width) - 1
    c0, c1, c2, c3 = (int(x) & mask for x in ctr)
    k0, k1 = (int(x) & mask for x in key)
    for _ in range(rounds):
        p0 = m0 * c0
        p1 = m1 * c2
        c0, c1, c2, c3 = ((p1 >> width) ^ c1 ^ k0, p1 & mask,
                          (p0 >> width) ^ c3 ^ k1, p0 & mask)
        k0 = (k0 + w0) & mask
        k1 = (k1 + w1) & mask
    return c0, c1, c2, c3


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Vectorised Philox4x32-10.  Counter and key words are broadcastable
    integer arrays (values < 2^32).  Returns four uint32 arrays."""
    u64 = np.uint64
    mask = u64(0xFFFFFFFF)
    m0, m1 = (u64(x) for x in PHILOX_M[32])
    w0, w1 = (u64(x) for x in PHILOX_W[32])
    shape = np.broadcast_shapes(np.shape(c0), np.shape(c1), np.shape(c2), np.shape(c3))
    c0, c1, c2, c3 = (np.broadcast_to(np.asarray(x, dtype=np.uint64), shape).copy()
                      for x in (c0, c1, c2, c3))
    k0 = np.asarray(k0, dtype=np.uint64)
    k1 = np.asarray(k1, dtype=np.uint64)
    for _ in range(10):
        p0 = m0 * c0                      # < 2^64: exact in uint64
        p1 = m1 * c2
        n0 = (p1 >> u64(32)) ^ c1 ^ k0
        n1 = p1 & mask
        n2 = (p0 >> u64(32)) ^ c3 ^ k1
        n3 = p0 & mask
        c0, c1, c2, c3 = n0, n1, n2, n3
        k0 = (k0 + w0) & mask
        k1 = (k1 + w1) & mask
    return tuple(x.astype(np.uint32) for x in (c0, c1, c2, c3))


def dropout_threshold(p: float) -> int:
    """Integer threshold on a uniform 16-bit value: drop iff u < thr.
    Computed from the float32 value of p, as the kernels receive it."""
    p32 = float(np.float32(p))
    return min(int(np.floor(p32 * 2.0 ** 16)), 2 ** 16 - 1)


def keep_scale(p: float) -> float:
    """Factor applied to kept entries: 1 / P(keep) = 2^16 / (2^16 - thr)
    for p > 0, else 1 (no dropout)."""
    if p <= 0:
        return 1.0
    return 2.0 ** 16 / (2.0 ** 16 - dropout_threshold(p))


def keep_mask(seed: int, rng_offset: int, p: float, b: int, h: int, H: int,
              rows, cols) -> np.ndarray:
    """bool [len(rows), len(cols)]: the keep bits of attention elements
    (b, h, i, j) for i in rows, j in cols."""
    rows = np.asarray(rows, dtype=np.uint64)
    cols = np.asarray(cols, dtype=np.uint64)
    thr = dropout_threshold(p)
    if thr == 0:
        return np.ones((len(rows), len(cols)), dtype=bool)
    seed = int(seed) & 0xFFFFFFFFFFFFFFFF
    k0, k1 = seed & 0xFFFFFFFF, seed >> 32
    c0 = (cols >> np.uint64(2))[None, :]
    c1 = (rows >> np.uint64(1))[:, None]
    c2 = np.uint64(b * H + h)
    c3 = np.uint64(int(rng_offset) & 0xFFFFFFFF)
    words = philox4x32_10(c0, c1, c2, c3, k0, k1)
    sel = (cols & np.uint64(3)).astype(np.int64)[None, :]
    w = np.choose(np.broadcast_to(sel, words[0].shape), words).astype(np.uint64)
    shift = ((rows & np.uint64(1)) * np.uint64(16))[:, None]
    u = (w >> shift) & np.uint64(0xFFFF)
    return u >= np.uint64(thr)
