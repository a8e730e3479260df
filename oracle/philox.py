"""Philox4x32-10 counter-based generator and the dropout keep mask.

TEST INFRASTRUCTURE ONLY (part of the oracle; the HIP library never imports
it and shares no code with it).

Generator: Philox4x32 with 10 rounds, as defined by Salmon, Moraes, Dror and
Shaw, "Parallel random numbers: as easy as 1, 2, 3" (SC'11), section 4.2
(the Philox S-box: two 32 x 32 -> 64-bit products per round, the high
halves XORed with the other two counter words and the round key, a fixed
word permutation, and a Weyl-sequence key schedule). Multipliers
0xD2511F53, 0xCD9E8D57; key increments 0x9E3779B9 (golden ratio) and
0xBB67AE85 (sqrt(3) - 1), applied between rounds. Written here from that
definition with numpy uint64 arithmetic; pinned by the generator's published
known-answer vectors (tests/golden/philox4x32_10_kat.txt).

Dropout keep mask (the pages say only that dropout is applied inside the
fused kernel on chip and never materialised -- the zako-mio report, section
3.2, "single-kernel fusion"; they fix no generator, so the plainest
counter-based reading is taken and stated here):

* element (b, h, i, j) of a problem with Hq query heads draws the 16-bit
  uniform  u = half (j mod 2) of word ((j div 2) mod 4) of
  Philox4x32-10(counter = (j div 8, i, b * Hq + h, offset),
                key = (seed mod 2^32, seed div 2^32)),
  half 0 being the low 16 bits; one generator call serves 8 consecutive keys
  of one query row;
* the element is kept iff u < T, T = round((1 - p) * 65536) in double
  precision (ties away from zero), so the realised keep probability is
  q = T / 65536 (p is honoured to within 2^-17); T = 0 is rejected;
* kept entries of P are scaled by 1 / q (which makes E[O] the undropped O).
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

M0 = 0xD2511F53
M1 = 0xCD9E8D57
W0 = 0x9E3779B9
W1 = 0xBB67AE85
ROUNDS = 10
_MASK32 = np.uint64(0xFFFFFFFF)


def philox4x32(counter: np.ndarray, key, rounds: int = ROUNDS) -> np.ndarray:
    """Philox4x32-``rounds`` of every counter in ``counter`` ([..., 4] uint32)
    under key (k0, k1). Returns [..., 4] uint32."""
    c = np.asarray(counter, dtype=np.uint64) & _MASK32
    x0, x1, x2, x3 = c[..., 0], c[..., 1], c[..., 2], c[..., 3]
    k0 = int(key[0]) & 0xFFFFFFFF
    k1 = int(key[1]) & 0xFFFFFFFF
    for _ in range(rounds):
        p0 = x0 * np.uint64(M0)  # exact: both factors < 2^32
        p1 = x2 * np.uint64(M1)
        hi0, lo0 = p0 >> np.uint64(32), p0 & _MASK32
        hi1, lo1 = p1 >> np.uint64(32), p1 & _MASK32
        x0, x1, x2, x3 = (hi1 ^ x1 ^ np.uint64(k0), lo1,
                          hi0 ^ x3 ^ np.uint64(k1), lo0)
        k0 = (k0 + W0) & 0xFFFFFFFF
        k1 = (k1 + W1) & 0xFFFFFFFF
    return np.stack([x0, x1, x2, x3], axis=-1).astype(np.uint32)


def keep_threshold(p: float) -> int:
    """T = round((1 - p) * 65536), ties away from zero, for 0 < p < 1."""
    if not (0.0 < p < 1.0):
        raise ValueError("dropout probability must lie in (0, 1)")
    t = int(math.floor((1.0 - float(p)) * 65536.0 + 0.5))
    if t <= 0:
        raise ValueError("dropout probability rounds to dropping everything")
    return min(t, 65536)


@dataclasses.dataclass(frozen=True)
class Dropout:
    """Dropout of a whole problem: probability p, 64-bit seed, 32-bit offset."""

    p: float
    seed: int = 0
    offset: int = 0

    @property
    def threshold(self) -> int:
        return keep_threshold(self.p)

    @property
    def scale(self) -> float:
        """1 / q with q = T / 65536 the realised keep probability."""
        return 65536.0 / self.threshold

    def uniforms(self, bh: int, rows, cols) -> np.ndarray:
        """uint32 [len(rows), len(cols)] 16-bit uniforms of head bh = b*Hq+h."""
        i = np.asarray(rows, dtype=np.int64)[:, None]
        j = np.asarray(cols, dtype=np.int64)[None, :]
        shape = np.broadcast_shapes(i.shape, j.shape)
        ctr = np.empty(shape + (4,), dtype=np.uint64)
        ctr[..., 0] = j >> 3
        ctr[..., 1] = i
        ctr[..., 2] = bh
        ctr[..., 3] = self.offset
        key = (self.seed & 0xFFFFFFFF, (self.seed >> 32) & 0xFFFFFFFF)
        words = philox4x32(ctr, key).astype(np.uint64)
        jw = np.broadcast_to((j >> 1) & 3, shape)
        word = np.take_along_axis(words, jw[..., None], axis=-1)[..., 0]
        half = np.broadcast_to(j & 1, shape).astype(np.uint64)
        return ((word >> (np.uint64(16) * half)) & np.uint64(0xFFFF)).astype(np.uint32)

    def keep(self, bh: int, rows, cols) -> np.ndarray:
        """Boolean keep mask [len(rows), len(cols)] of head bh = b*Hq+h."""
        return self.uniforms(bh, rows, cols) < self.threshold

    def head(self, bh: int) -> "HeadDropout":
        return HeadDropout(self, bh)


@dataclasses.dataclass(frozen=True)
class HeadDropout:
    """The keep mask of one (batch, query head): what a head function needs."""

    spec: Dropout
    bh: int

    @property
    def scale(self) -> float:
        return self.spec.scale

    def keep(self, rows, cols) -> np.ndarray:
        return self.spec.keep(self.bh, rows, cols)
