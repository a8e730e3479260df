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
* fp8 workloads encode each draw x as the OCP e4m3 (E4M3FN) value nearest to
  x / descale (ties to even mantissa, saturating at +-448) with the
  workload's per-tensor descale factors; the logical input is then
  descale * decode(code), which is what the oracle reads. A power-of-two
  descale keeps that product exact.
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
    descale: tuple = (1.0, 1.0, 1.0)  # fp8: per-tensor (q, k, v) descale factors

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
        if self.dtype == "fp8" and tuple(self.descale) != (1.0, 1.0, 1.0):
            parts.append("descale" + "/".join(f"{x:g}" for x in self.descale))
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
    # FP8 (e4m3) forward: the headline shape and the causal key-padded d = 128
    # shape, inputs encoded at x * 16 with descale 1/16 (the pages fix no FP8
    # workload; these reuse the exact-attention shapes).
    10: Workload("gpt2-medium-attn-fp8", 64, 16, 16, 1024, 64, "fp8", backward=False,
                 descale=(0.0625, 0.0625, 0.0625)),
    11: Workload("causal-keypad-fp8", 8, 16, 16, 4096, 128, "fp8", causal=True,
                 pad_range=(2048, 4096), backward=False, descale=(0.0625, 0.0625, 0.0625)),
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


def f32_to_e4m3_bits(x: np.ndarray) -> np.ndarray:
    """Encode values as OCP e4m3 (E4M3FN: 1 sign, 4 exponent bits with bias
    7, 3 mantissa bits, subnormals below 2^-6, no infinities, NaN = S.1111.111,
    largest finite 448): the nearest representable value, ties to an even
    mantissa, magnitudes above 448 saturating to 448. Inputs must be finite.
    Returns uint8 codes."""
    x = np.asarray(x, dtype=np.float64)
    sign = (np.signbit(x)).astype(np.uint8) << 7
    a = np.minimum(np.abs(x), 448.0)
    # binade exponent, floored at the subnormal range (spacing 2^-9 there)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -6.0)
    quantum = np.exp2(e - 3)
    q = np.round(a / quantum) * quantum          # numpy rounds half to even
    q = np.minimum(q, 448.0)
    # re-derive the exponent of the rounded value (rounding may carry up)
    qe = np.floor(np.log2(np.where(q > 0, q, 1.0)))
    normal = q >= 2.0 ** -6
    E = np.where(normal, qe + 7, 0).astype(np.int64)
    M = np.where(normal, np.round((q / np.exp2(qe) - 1.0) * 8), np.round(q / 2.0 ** -9))
    M = M.astype(np.int64)
    code = (E << 3) | M
    return (sign | code.astype(np.uint8)).astype(np.uint8)


def e4m3_bits_to_f64(b: np.ndarray) -> np.ndarray:
    """Decode OCP e4m3 codes exactly (NaN for the two NaN codes)."""
    b = np.asarray(b, dtype=np.uint8).astype(np.int64)
    s = np.where(b & 0x80, -1.0, 1.0)
    E = (b >> 3) & 15
    M = b & 7
    v = np.where(E == 0, M * 2.0 ** -9, (1.0 + M / 8.0) * np.exp2(E - 7.0))
    v = np.where((E == 15) & (M == 7), np.nan, v)
    return s * v


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
    float32 values; for fp8 q/k/v hold uint8 e4m3 codes of value / descale.
    ``seqlens`` is int32 [B] or None; ``block_mask`` is uint8
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
    descale: tuple = (1.0, 1.0, 1.0)

    def as_f64(self, name: str, index=None) -> np.ndarray:
        """Exact float64 view of tensor ``name`` (optionally sliced first);
        for fp8 the logical value descale * decode(code)."""
        a = getattr(self, name)
        if index is not None:
            a = a[index]
        if self.workload.dtype == "bf16":
            return bf16_bits_to_f64(a)
        if self.workload.dtype == "fp8":
            ds = dict(q=self.descale[0], k=self.descale[1], v=self.descale[2])[name]
            return e4m3_bits_to_f64(a) * ds
        return np.asarray(a, dtype=np.float64)


def draw(w: Workload, seed: int, *, with_do: Optional[bool] = None) -> Inputs:
    """Draw the inputs of workload ``w`` from ``numpy.random.default_rng(seed)``."""
    rng = np.random.default_rng(seed)
    with_do = w.backward if with_do is None else with_do
    qshape = (w.batch, w.heads_q, 1 if w.decode else w.seqlen, w.head_dim)
    kshape = (w.batch, w.heads_kv, w.seqlen, w.head_dim)

    def one(shape, ds=1.0):
        x = rng.standard_normal(shape, dtype=np.float32)
        if w.dtype == "bf16":
            return f32_to_bf16_bits(x)
        if w.dtype == "fp8":
            return f32_to_e4m3_bits(x.astype(np.float64) / ds)
        return x

    q = one(qshape, w.descale[0])
    k = one(kshape, w.descale[1])
    v = one(kshape, w.descale[2])
    do = one(qshape) if with_do else None
    seqlens = None
    if w.pad_range is not None:
        lo, hi = w.pad_range
        seqlens = rng.integers(lo, hi, endpoint=True, size=w.batch).astype(np.int32)
    block_mask = None
    if w.butterfly:
        nb = -(-w.seqlen // MASK_BLOCK)
        block_mask = butterfly_block_mask(nb)
    return Inputs(w, q, k, v, do, seqlens, block_mask, w.scale, w.window,
                  tuple(float(x) for x in w.descale))


def draw_case(batch, heads_q, heads_kv, seqlen, head_dim, dtype="bf16", *,
              causal=False, seqlens=None, block_mask=None, seed=0,
              with_do=True, window=None, descale=(1.0, 1.0, 1.0)) -> Inputs:
    """Draw an ad-hoc problem (used by the small parity cases).

    ``seqlens`` may be None, a sequence of ints, or "random" (uniform over
    [0, seqlen], inclusive, drawn after the tensors). ``block_mask`` may be
    None, an array, "butterfly" or "random" (each block on with prob. 1/2,
    the diagonal always on).
    """
    w = Workload("case", batch, heads_q, heads_kv, seqlen, head_dim, dtype,
                 causal=causal, backward=with_do, descale=tuple(descale))
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
