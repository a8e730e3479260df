"""Work and traffic accounting for attention problems (host-side arithmetic).

FLOP convention (algorithmic work, not executed work):
* forward  = 2 matrix products (S = Q K^T and O = P V) over the allowed
  (query, key) pairs: 4 * d flops per pair;
* backward = 5 matrix products (S rebuilt, dP = dO V^T, dV = P^T dO,
  dQ = dS K, dK = dS^T Q): 10 * d flops per pair -- the five-product
  structure the zhaifeiyue.github.io cross-paper synthesis (section 5, item 5)
  contrasts with the forward's two.
Masked pairs count nothing. Work the implementation repeats beyond that
(the dQ kernel rebuilding S and dP) is not counted.

Per-kernel shares used for roofline reporting: the forward kernel carries
4 d per pair; the dK/dV kernel carries S, dP, dV and dK (8 d per pair); the
dQ kernel carries dQ (2 d per pair).

HBM byte models (eb = bytes per element):
* compulsory: every input read once and every output written once;
* tile model: Q read and O written once, plus one K tile and one V tile
  (128 x d each) per visited 128 x 128 tile -- the Theta(N^2 d^2 / M) traffic
  of the tiled algorithm with no cache reuse (deep-reading report, section
  3.4 table);
* Algorithm 0: compulsory plus writing and reading back S and P
  (N x N each) -- the Theta(N d + N^2) standard implementation of the
  report's section 3.1.
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np

MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X published dense bf16 / fp16 matrix peak
MFMA_FP32_PEAK_TFLOPS = 157.3   # MI355X published fp32 matrix/vector peak
MFMA_FP8_PEAK_TFLOPS = 5000.0   # MI355X published dense fp8 matrix peak
HBM_PEAK_GBS = 8000.0           # MI355X published HBM3E bandwidth


def allowed_pairs_per_row(N: int, *, causal=False, seqlen_k: Optional[int] = None,
                          block_mask: Optional[np.ndarray] = None, block=128,
                          window=None) -> np.ndarray:
    """int64 [N]: number of allowed keys of each query row of one sequence.

    Row i's allowed keys (before the block mask) are the interval
    [lo_i, cap_i): lo_i = max(0, i - left) under a (left, right) window, and
    cap_i the least of L, i + 1 (causal) and i + right + 1 (window)."""
    i = np.arange(N, dtype=np.int64)
    L = N if seqlen_k is None else int(min(max(seqlen_k, 0), N))
    cap = np.minimum(i + 1, L) if causal else np.full(N, L, dtype=np.int64)
    lo = np.zeros(N, dtype=np.int64)
    if window is not None:
        cap = np.minimum(cap, i + int(window[1]) + 1)
        lo = np.maximum(0, i - int(window[0]))
    if block_mask is None:
        return np.clip(cap - lo, 0, None)
    nb = -(-N // block)
    bm = np.asarray(block_mask)[:nb, :nb] != 0
    out = np.zeros(N, dtype=np.int64)
    for kb in range(nb):
        k0 = kb * block
        k1 = min(N, k0 + block)
        rows_on = bm[i // block, kb]
        cnt = np.clip(np.minimum(cap, k1) - np.maximum(lo, k0), 0, None)
        out += np.where(rows_on, cnt, 0)
    return out


def allowed_pairs(B: int, Hq: int, N: int, *, causal=False, seqlens=None, block_mask=None,
                  window=None) -> int:
    """Total allowed (query, key) pairs over all batches and query heads."""
    total = 0
    for b in range(B):
        L = None if seqlens is None else int(seqlens[b])
        total += int(allowed_pairs_per_row(N, causal=causal, seqlen_k=L,
                                           block_mask=block_mask, window=window).sum())
    return total * Hq


def tile_map(N: int, *, causal=False, seqlen_k: Optional[int] = None, block_mask=None,
             block=128, window=None) -> np.ndarray:
    """bool [nb, nb]: which block x block tiles of one sequence hold an
    allowed pair. Over the rows r0..r1 of a row block, the allowed keys
    (before the block mask) form one interval: from r0 - left to the least
    of L - 1, r1 (causal) and r1 + right."""
    nb = -(-N // block)
    r0 = np.arange(nb)[:, None] * block
    r1 = np.minimum(r0 + block, N) - 1
    c0 = np.arange(nb)[None, :] * block
    c1 = np.minimum(c0 + block, N) - 1
    L = N if seqlen_k is None else int(min(max(seqlen_k, 0), N))
    hi = np.full_like(r1, L - 1)
    if causal:
        hi = np.minimum(hi, r1)
    lo = np.zeros_like(r0)
    if window is not None:
        hi = np.minimum(hi, r1 + int(window[1]))
        lo = np.maximum(lo, r0 - int(window[0]))
    t = np.maximum(c0, lo) <= np.minimum(c1, hi)
    if block_mask is not None:
        t = t & (np.asarray(block_mask)[:nb, :nb] != 0)
    return t


def visited_tiles(B: int, Hq: int, N: int, *, causal=False, seqlens=None, block_mask=None,
                  block=128, window=None) -> int:
    """Number of 128 x 128 tiles with at least one allowed pair."""
    total = 0
    for b in range(B):
        L = None if seqlens is None else int(seqlens[b])
        total += int(tile_map(N, causal=causal, seqlen_k=L, block_mask=block_mask, block=block,
                              window=window).sum())
    return total * Hq


def decode_bytes(B: int, Hq: int, Hkv: int, d: int, cache_lens, eb: int = 2,
                 o_eb: int = 2) -> int:
    """Compulsory HBM bytes of one decode step: each sequence's cached K and
    V rows 0 .. L_b - 1 read once, the query rows read, the output rows and
    the float32 LSE written."""
    kv = sum(int(L) for L in cache_lens) * Hkv * d * eb * 2
    return kv + B * Hq * d * eb + B * Hq * d * o_eb + B * Hq * 4


def flops(pairs: int, d: int) -> dict:
    """Algorithmic flops of the forward, backward and per-kernel shares."""
    return {
        "fwd": 4 * d * pairs,
        "bwd": 10 * d * pairs,
        "fwd_bwd": 14 * d * pairs,
        "bwd_dkdv": 8 * d * pairs,
        "bwd_dq": 2 * d * pairs,
    }


def bytes_models(B, Hq, Hkv, N, d, eb, *, tiles, o_eb=None) -> dict:
    """Compulsory, tile-model and Algorithm-0 HBM bytes of forward and backward."""
    o_eb = eb if o_eb is None else o_eb
    q = B * Hq * N * d * eb
    kv = B * Hkv * N * d * eb
    o = B * Hq * N * d * o_eb
    lse = B * Hq * N * 4
    s_bytes = B * Hq * N * N * eb
    fwd_c = q + 2 * kv + o + lse
    bwd_c = q + 2 * kv + o + q + lse + q + 2 * kv + 2 * lse  # + dO in, dQ/dK/dV out, D out+in
    tile_kv = tiles * 2 * 128 * d * eb
    return {
        "fwd_compulsory": fwd_c,
        "fwd_tile_model": q + o + lse + tile_kv,
        "fwd_alg0": fwd_c + 4 * s_bytes,
        "bwd_compulsory": bwd_c,
        "bwd_tile_model": bwd_c - 2 * kv + 2 * tile_kv,
        "bwd_alg0": bwd_c + 7 * s_bytes,
    }


def score_matrix_bytes(heads: int, seqlen: int, eb: int) -> int:
    """Bytes of the full heads x N x N score matrix at eb bytes per element."""
    return heads * seqlen * seqlen * eb


def tflops(flop: float, seconds: float) -> float:
    return flop / seconds / 1e12 if seconds > 0 else math.nan
