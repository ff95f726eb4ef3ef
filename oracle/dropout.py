"""Attention dropout with counter-based random numbers (fp64 oracle side).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The digest page ("Fast and Exact Relative-Position Attention via
Structure-Aware Kernels", nanless.github.io), in its section on what a
reproduction must do first, lists dropout whose random numbers are recomputed
in the backward pass.  The page does not say which generator, which random
bits feed which score, or where in the formula the dropout sits.  Readings
adopted here:

* Dropout acts on the normalised attention weights: with keep mask K_ij and
  drop probability p, O = (P * K / (1 - p)) V.  The log-sum-exp is that of
  the undropped softmax.  The gradients follow by the chain rule:
      dV = (P * K / (1-p))^T dO,   dP = (dO V^T) * K / (1-p),
      D_i = sum_j P_ij dP_ij  (= dO_i . O_i),   dS = P * (dP - D).
* The generator is Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel
  Random Numbers: As Easy as 1, 2, 3", SC 2011): a 4 x 32-bit counter and a
  2 x 32-bit key, ten rounds of two 32 x 32 -> 64-bit products with the
  multipliers 0xD2511F53 and 0xCD9E8D57, the key bumped by the Weyl constants
  0x9E3779B9 and 0xBB67AE85 between rounds.
* The key is the 64-bit seed (low word first).  One call covers a 4 x 4
  block of scores: counter = (j // 4, i // 4, batch * H + head, offset), and
  byte (j % 4) of output word (i % 4) is the score's random byte u.
* The drop probability is a multiple of 1/256, p = t / 256 with an integer
  threshold t in [0, 255]; a score is kept iff u >= t.
"""

import numpy as np

PHILOX_M = (0xD2511F53, 0xCD9E8D57)
PHILOX_W = (0x9E3779B9, 0xBB67AE85)
_U32 = np.uint64(0xFFFFFFFF)


def philox4x32_10(ctr, key):
    """Philox4x32-10 of counters ``ctr`` ([..., 4] integers < 2^32) under
    ``key`` = (k0, k1); returns [..., 4] uint64 holding 32-bit words."""
    c = np.asarray(ctr, dtype=np.uint64)
    c0, c1, c2, c3 = (c[..., n].copy() for n in range(4))
    k0, k1 = int(key[0]) & 0xFFFFFFFF, int(key[1]) & 0xFFFFFFFF
    m0, m1 = np.uint64(PHILOX_M[0]), np.uint64(PHILOX_M[1])
    for _ in range(10):
        p0 = m0 * c0  # < 2^64: exact in uint64
        p1 = m1 * c2
        c0, c1, c2, c3 = ((p1 >> np.uint64(32)) ^ c1 ^ np.uint64(k0), p1 & _U32,
                          (p0 >> np.uint64(32)) ^ c3 ^ np.uint64(k1), p0 & _U32)
        k0 = (k0 + PHILOX_W[0]) & 0xFFFFFFFF
        k1 = (k1 + PHILOX_W[1]) & 0xFFFFFFFF
    return np.stack([c0, c1, c2, c3], axis=-1)


def random_bytes(seed, offset, bh_index, rows, N):
    """The random byte u_ij of every score (i in ``rows``, 0 <= j < N) of the
    (batch, head) pair with flat index ``bh_index``; uint8 [len(rows), N]."""
    rows = np.asarray(rows, dtype=np.int64)
    ig = np.unique(rows // 4)
    jg = np.arange((N + 3) // 4, dtype=np.int64)
    ctr = np.zeros((ig.size, jg.size, 4), dtype=np.uint64)
    ctr[..., 0] = jg[None, :]
    ctr[..., 1] = ig[:, None]
    ctr[..., 2] = bh_index
    ctr[..., 3] = offset
    words = philox4x32_10(ctr, (seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF))
    gi = np.searchsorted(ig, rows // 4)
    w = words[gi][:, :, :]                       # [rows, jg, 4 words]
    w = np.take_along_axis(w, (rows % 4)[:, None, None], axis=2)[:, :, 0]  # word i % 4
    jj = np.arange(N, dtype=np.int64)
    byte = (w[:, jj // 4] >> (np.uint64(8) * (jj % 4).astype(np.uint64))) & np.uint64(0xFF)
    return byte.astype(np.uint8)


def keep_mask(dropout, bh_index, rows, N):
    """Boolean keep mask K_ij for ``dropout`` = (t, seed, offset)."""
    t, seed, offset = dropout
    if not 0 <= t <= 255:
        raise ValueError("dropout threshold must be in [0, 255]")
    return random_bytes(seed, offset, bh_index, rows, N) >= t


def keep_scale(dropout):
    """1 / (1 - p) with p = t / 256."""
    return 256.0 / (256.0 - dropout[0])
