"""Error bound of the FP8 (e4m3) forward, derived from its arithmetic.

The kernel computes S from the exact e4m3 inputs (products of two e4m3
values are exact in fp32; fp32 accumulation error is far below what follows),
P~ = 2^(S c - m) with a running reference m that trails the row maximum by at
most 8 (so 1 <= max P~ <= 256 < 448, the largest e4m3), the row sum l from the
fp32 P~, and the numerator from P~ rounded to e4m3. One e4m3 rounding moves a
value x by at most one unit in the last place: 2^-3 x in the normal range
(3 mantissa bits) and 2^-9 below it (the subnormal spacing), whatever the
rounding mode. With P = P~ / l and l >= max P~ >= 1:

  |dP_ij| <= 2^-3 P_ij + 2^-9 / l <= 2^-3 P_ij + 2^-9 max_j P_ij

so per output element

  |O_ic - O_ref_ic| <= sum_j (2^-3 P_ij + 2^-9 max_j P_ij [j allowed]) |V_jc|

(V the logical, descaled values) plus the rounding of O to its output type
and a small relative slack for fp32 arithmetic.
"""
from __future__ import annotations

import numpy as np


def fp8_o_bound(p: np.ndarray, v: np.ndarray, allowed: np.ndarray) -> np.ndarray:
    """Per-element bound [rows, d] from the exact probabilities p [rows, N],
    logical values v [N, d] and the boolean allowed mask [rows, N]."""
    av = np.abs(v)
    pmax = p.max(axis=1, keepdims=True)
    return 2.0 ** -3 * (p @ av) + 2.0 ** -9 * pmax * (allowed.astype(np.float64) @ av)
