"""Counter-based generator and the dropout multiplier matrix built from it.

TEST INFRASTRUCTURE ONLY (see the package docstring): the HIP library has its
own, separately written generator; the two share nothing.

Dropout replay.  "解析 FlashAttention（3）：FlashAttention-v1 反向传播", section
3.3 and the dropout lines of Algorithm 4 (section 4): the forward pass keeps
only the generator state, and the backward pass regenerates, block by block,
exactly the mask Z the forward pass used.  An element of Z is 1/(1 - p_drop)
with probability 1 - p_drop and 0 otherwise.  The pages fix no generator, so
this module states one:

Generator.  Philox-4xW-10 from J. K. Salmon, M. A. Moraes, R. O. Dror,
D. E. Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3" (SC'11), section 3
(the Philox family): a 4-word counter and a 2-word key; each of the 10 rounds
multiplies counter words 0 and 2 by the constants M0, M1 (keeping both halves
of the double-width products), mixes the high halves into words 1 and 3 with
the round key, and permutes the words; the key advances by the Weyl constants
(W0, W1) between rounds.  W = 32 is the instance used; W = 64 is kept so the
round structure can be checked against numpy's independent Philox4x64-10.

Element -> random bits (a choice the pages leave open; the kernels follow the
same statement, with code of their own).  For query head bh = b * H + h,
query row q and key k, one Philox4x32-10 call with
    counter = (k >> 1, q >> 2, bh, offset),  key = (seed mod 2^32, seed >> 32)
returns words x0..x3; the element's 16-bit value is u = half (k & 1) of word
(q & 3) (half 0 = low 16 bits).  One call covers a block of 4 query rows by 2
keys.  The element is kept iff u < t with t = floor((1 - p) 65536 + 1/2), so
its keep probability is t / 65536, within 2^-17 of 1 - p.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "PHILOX_M32",
    "PHILOX_W32",
    "PHILOX_M64",
    "PHILOX_W64",
    "philox4x32",
    "philox4x64",
    "keep_threshold",
    "dropout_bits",
    "dropout_multiplier",
]

# Multipliers and Weyl key increments (SC'11 paper, Philox parameters).  The
# Weyl constants are the fractional parts of the golden ratio and of sqrt(3)
# in fixed point.
PHILOX_M32 = (0xD2511F53, 0xCD9E8D57)
PHILOX_W32 = (0x9E3779B9, 0xBB67AE85)
PHILOX_M64 = (0xD2E7470EE14C6C93, 0xCA5A826395121157)
PHILOX_W64 = (0x9E3779B97F4A7C15, 0xBB67AE8584CAA73B)


def philox4x32(counter, key, rounds=10):
    """Philox-4x32-R on arrays: counter [..., 4], key [..., 2] -> [..., 4] uint64 words < 2^32.

    All arithmetic is exact in uint64: a 32 x 32-bit product fits in 64 bits.
    """
    x = np.asarray(counter, dtype=np.uint64)
    k = np.asarray(key, dtype=np.uint64)
    x0, x1, x2, x3 = (x[..., i].copy() for i in range(4))
    k0, k1 = k[..., 0].copy(), k[..., 1].copy()
    mask = np.uint64(0xFFFFFFFF)
    m0, m1 = np.uint64(PHILOX_M32[0]), np.uint64(PHILOX_M32[1])
    w0, w1 = np.uint64(PHILOX_W32[0]), np.uint64(PHILOX_W32[1])
    sh = np.uint64(32)
    for r in range(rounds):
        p0 = m0 * x0
        p1 = m1 * x2
        hi0, lo0 = p0 >> sh, p0 & mask
        hi1, lo1 = p1 >> sh, p1 & mask
        x0, x1, x2, x3 = hi1 ^ x1 ^ k0, lo1, hi0 ^ x3 ^ k1, lo0
        if r + 1 < rounds:
            k0 = (k0 + w0) & mask
            k1 = (k1 + w1) & mask
    return np.stack([x0, x1, x2, x3], axis=-1)


def philox4x64(counter, key, rounds=10):
    """Philox-4x64-R for one counter (4 Python ints < 2^64) and key (2 ints): 4 ints.

    Python integers hold the 128-bit products exactly.  Slow; used only to
    check the round structure against numpy's Philox bit generator.
    """
    mask = (1 << 64) - 1
    x0, x1, x2, x3 = (int(v) for v in counter)
    k0, k1 = (int(v) for v in key)
    for r in range(rounds):
        p0 = PHILOX_M64[0] * x0
        p1 = PHILOX_M64[1] * x2
        x0, x1, x2, x3 = (p1 >> 64) ^ x1 ^ k0, p1 & mask, (p0 >> 64) ^ x3 ^ k1, p0 & mask
        if r + 1 < rounds:
            k0 = (k0 + PHILOX_W64[0]) & mask
            k1 = (k1 + PHILOX_W64[1]) & mask
    return [x0, x1, x2, x3]


def keep_threshold(p):
    """t = floor((1 - p) 65536 + 1/2): an element is kept iff its 16-bit value is below t.

    p is the dropout probability as the float32 the interface carries.
    """
    p = float(np.float32(p))
    if not (0.0 <= p < 1.0):
        raise ValueError(f"dropout probability {p} outside [0, 1)")
    return min(65536, int(math.floor((1.0 - p) * 65536.0 + 0.5)))


def dropout_bits(seed, offset, bh, q_idx, k_idx):
    """16-bit random values u [len(q_idx), len(k_idx)] of query head bh.

    One Philox4x32-10 call per distinct (q >> 2, k >> 1) block, with counter
    (k >> 1, q >> 2, bh, offset) and key (seed low word, seed high word); the
    element takes half (k & 1) of word (q & 3).
    """
    q_idx = np.asarray(q_idx, dtype=np.int64)
    k_idx = np.asarray(k_idx, dtype=np.int64)
    seed = int(seed)
    if q_idx.size == 0 or k_idx.size == 0:
        return np.zeros((q_idx.size, k_idx.size), dtype=np.uint64)
    qb, q_inv = np.unique(q_idx >> 2, return_inverse=True)
    kb, k_inv = np.unique(k_idx >> 1, return_inverse=True)
    ctr = np.zeros((qb.size, kb.size, 4), dtype=np.uint64)
    ctr[..., 0] = kb[None, :]
    ctr[..., 1] = qb[:, None]
    ctr[..., 2] = int(bh)
    ctr[..., 3] = int(offset)
    key = np.array([seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF], dtype=np.uint64)
    words = philox4x32(ctr, key)  # [qb, kb, 4]
    w = words[q_inv[:, None], k_inv[None, :], (q_idx & 3)[:, None]]
    shift = (16 * (k_idx & 1)).astype(np.uint64)[None, :]
    return (w >> shift) & np.uint64(0xFFFF)


def dropout_multiplier(p, seed, offset, bh, q_idx, k_idx):
    """The replayed dropout matrix Z [len(q_idx), len(k_idx)] in float64.

    Z = 1 / (1 - p) where the element is kept and 0 where it is dropped (the
    FlashAttention-v1 page, section 4, the dropout-mask line of Algorithm 4).
    """
    p = float(np.float32(p))
    t = keep_threshold(p)
    u = dropout_bits(seed, offset, bh, q_idx, k_idx)
    return np.where(u < np.uint64(t), 1.0 / (1.0 - p), 0.0)
