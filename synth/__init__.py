"""Seeded synthetic inputs for the attention workloads.

This module only draws and packages inputs; it holds none of the attention
arithmetic. Both sides of a parity check (the fp64 CPU oracle and the HIP
library) consume exactly the arrays produced here, so a disagreement between
them can never come from the inputs.

Recipe (one generator per workload, numpy PCG64 seeded with the workload id):

* Q, K, V and the upstream gradient dO are drawn, in that order, as float32
  standard normals in the logical shape [batch, heads, seqlen, head_dim]
  (K and V with the key/value head count).
* bf16 workloads round those draws to bfloat16 with round-to-nearest-even;
  the oracle then reads the very same bf16 values widened to float64.
* Key-padding lengths, where a workload has them, are drawn last, as integers
  uniform over an inclusive range.
* The block-sparse "butterfly" pattern of the FlashAttention paper's
  block-sparse variant (deep-reading report, section 2.6 and section 3.5) is
  instantiated on a 2^k block grid as: block (i, j) is present iff i XOR j has
  at most one bit set (the diagonal plus one partner per bit).
* The softmax scale is 1/sqrt(head_dim), passed around as a float32 value.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

#: Granularity of block masks (rows and columns of one mask entry).
MASK_BLOCK = 128


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape and masking of one attention problem."""

    name: str
    batch: int
    heads_q: int
    heads_kv: int
    seqlen: int
    head_dim: int
    dtype: str  # "bf16" or "fp32"
    causal: bool = False
    pad_range: Optional[tuple] = None  # inclusive (lo, hi) for key lengths
    butterfly: bool = False
    backward: bool = True
    window: Optional[tuple] = None  # (left, right) sliding-window band
    decode: bool = False  # one query row per head against `seqlen` cached keys
    dropout: Optional[tuple] = None  # (p, seed, offset) of in-kernel dropout

    @property
    def group(self) -> int:
        return self.heads_q // self.heads_kv

    @property
    def scale(self) -> float:
        return float(np.float32(1.0 / math.sqrt(self.head_dim)))

    def describe(self) -> str:
        parts = [
            f"B{self.batch}",
            f"Hq{self.heads_q}",
            f"Hkv{self.heads_kv}",
            f"N{self.seqlen}",
            f"d{self.head_dim}",
            self.dtype,
        ]
        if self.causal:
            parts.append("causal")
        if self.pad_range:
            parts.append(f"keypad{self.pad_range[0]}-{self.pad_range[1]}")
        if self.butterfly:
            parts.append("butterfly128")
        if self.window is not None:
            parts.append(f"window{self.window[0]}-{self.window[1]}")
        if self.dropout is not None:
            parts.append(f"dropout{self.dropout[0]}")
        if self.decode:
            parts.append("decode")
            return " ".join(parts)
        parts.append("fwd+bwd" if self.backward else "fwd")
        return " ".join(parts)


#: The five workloads of the benchmark suite, keyed by id (also the seed).
WORKLOADS = {
    1: Workload("single-head-fp32", 1, 1, 1, 128, 64, "fp32", backward=False),
    2: Workload("gpt2-medium-attn", 64, 16, 16, 1024, 64, "bf16"),
    3: Workload("causal-keypad", 8, 16, 16, 4096, 128, "bf16", causal=True,
                pad_range=(2048, 4096)),
    4: Workload("long-causal-gqa", 1, 32, 8, 16384, 128, "bf16", causal=True),
    5: Workload("butterfly-64k", 1, 8, 8, 65536, 64, "bf16", butterfly=True),
    # Causal local attention: each query sees itself and the 1023 keys before
    # it (a sliding window; no such shape is fixed by the pages).
    6: Workload("sliding-window-8k", 4, 16, 16, 8192, 128, "bf16", causal=True,
                window=(1023, 0)),
    # Decoding: one new query row per head against a GQA key/value cache of
    # up to 32K positions per sequence (cache lengths uniform over
    # [16384, 32768]); the pages fix no such shape.
    7: Workload("decode-32k-gqa", 16, 32, 8, 32768, 128, "bf16", pad_range=(16384, 32768),
                backward=False, decode=True),
    # In-kernel dropout (p = 0.1, fixed seed and offset): the headline shape,
    # and the causal key-padded d = 128 shape -- dropout with a padding mask
    # is the setting of the pages' memory / runtime comparison.
    8: Workload("gpt2-medium-attn-dropout", 64, 16, 16, 1024, 64, "bf16",
                dropout=(0.1, 0x5EED, 0)),
    9: Workload("causal-keypad-dropout", 8, 16, 16, 4096, 128, "bf16", causal=True,
                pad_range=(2048, 4096), dropout=(0.1, 0x5EED, 0)),
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return bits.

    Inputs must be finite (normal draws always are).
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    rounded = u + np.uint32(0x7FFF) + lsb
    return (rounded >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns (uint16) to float64 exactly."""
    u = np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def butterfly_block_mask(nblocks: int) -> np.ndarray:
    """uint8 [nblocks, nblocks]: 1 where popcount(i XOR j) <= 1."""
    i = np.arange(nblocks, dtype=np.int64)[:, None]
    j = np.arange(nblocks, dtype=np.int64)[None, :]
    x = i ^ j
    # x has at most one bit set iff x & (x - 1) == 0 (covers x == 0).
    return ((x & (x - 1)) == 0).astype(np.uint8)


@dataclasses.dataclass
class Inputs:
    """One drawn problem. Tensors are in [B, H, N, d] order, C-contiguous.

    For bf16 workloads q/k/v/do hold uint16 bit patterns; for fp32 they hold
    float32 values. ``seqlens`` is int32 [B] or None; ``block_mask`` is uint8
    [ceil(N/128), ceil(N/128)] or None.
    """

    workload: Workload
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    do: Optional[np.ndarray]
    seqlens: Optional[np.ndarray]
    block_mask: Optional[np.ndarray]
    scale: float
    window: Optional[tuple] = None

    def as_f64(self, name: str, index=None) -> np.ndarray:
        """Exact float64 view of tensor ``name`` (optionally sliced first)."""
        a = getattr(self, name)
        if index is not None:
            a = a[index]
        if self.workload.dtype == "bf16":
            return bf16_bits_to_f64(a)
        return np.asarray(a, dtype=np.float64)


def draw(w: Workload, seed: int, *, with_do: Optional[bool] = None) -> Inputs:
    """Draw the inputs of workload ``w`` from ``numpy.random.default_rng(seed)``."""
    rng = np.random.default_rng(seed)
    with_do = w.backward if with_do is None else with_do
    qshape = (w.batch, w.heads_q, 1 if w.decode else w.seqlen, w.head_dim)
    kshape = (w.batch, w.heads_kv, w.seqlen, w.head_dim)

    def one(shape):
        x = rng.standard_normal(shape, dtype=np.float32)
        return f32_to_bf16_bits(x) if w.dtype == "bf16" else x

    q = one(qshape)
    k = one(kshape)
    v = one(kshape)
    do = one(qshape) if with_do else None
    seqlens = None
    if w.pad_range is not None:
        lo, hi = w.pad_range
        seqlens = rng.integers(lo, hi, endpoint=True, size=w.batch).astype(np.int32)
    block_mask = None
    if w.butterfly:
        nb = -(-w.seqlen // MASK_BLOCK)
        block_mask = butterfly_block_mask(nb)
    return Inputs(w, q, k, v, do, seqlens, block_mask, w.scale, w.window)


def draw_case(batch, heads_q, heads_kv, seqlen, head_dim, dtype="bf16", *,
              causal=False, seqlens=None, block_mask=None, seed=0,
              with_do=True, window=None) -> Inputs:
    """Draw an ad-hoc problem (used by the small parity cases).

    ``seqlens`` may be None, a sequence of ints, or "random" (uniform over
    [0, seqlen], inclusive, drawn after the tensors). ``block_mask`` may be
    None, an array, "butterfly" or "random" (each block on with prob. 1/2,
    the diagonal always on).
    """
    w = Workload("case", batch, heads_q, heads_kv, seqlen, head_dim, dtype,
                 causal=causal, backward=with_do)
    inp = draw(w, seed, with_do=with_do)
    rng = np.random.default_rng(seed + 7919)
    if isinstance(seqlens, str) and seqlens == "random":
        seqlens = rng.integers(0, seqlen, endpoint=True, size=batch)
    if seqlens is not None:
        inp.seqlens = np.asarray(seqlens, dtype=np.int32)
    nb = -(-seqlen // MASK_BLOCK)
    if isinstance(block_mask, str):
        if block_mask == "butterfly":
            block_mask = butterfly_block_mask(nb)
        elif block_mask == "random":
            bm = (rng.random((nb, nb)) < 0.5).astype(np.uint8)
            np.fill_diagonal(bm, 1)
            block_mask = bm
        else:
            raise ValueError(block_mask)
    if block_mask is not None:
        inp.block_mask = np.ascontiguousarray(block_mask, dtype=np.uint8)
    inp.window = None if window is None else (int(window[0]), int(window[1]))
    return inp
