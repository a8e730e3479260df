"""Plain fp64 CPU oracle for exact scaled-dot-product attention.

TEST INFRASTRUCTURE ONLY. This module is the reference that the HIP library
is checked against. Only the test-suite, the package smoke check and the
benchmark's CPU-baseline leg may import or run it; the library never does,
and it shares no code with the library.

What is computed (per batch b and query head h, with key/value head
g = floor(h / G), G = heads_q / heads_kv):

* Forward -- the standard attention of the FlashAttention deep-reading report
  (zako-mio), section 3.1 "Algorithm 0": the score matrix S = Q K^T is formed
  in full (here per block of query rows), then P = softmax(S) row by row, then
  O = P V. Scale and mask enter as the usual softmax(Q K^T * scale + mask):
  s_ij = scale * q_i . k_j, and s_ij = -inf where the key is not allowed.
  The softmax is computed in two passes (row max, then exp and sum), which is
  the textbook definition; the running-statistics form of the method is NOT
  used here, so that the GPU path's online softmax is checked against an
  independent formulation.
* The saved per-row statistic is the natural log-sum-exp
  LSE_i = m_i + ln(l_i), m_i = max_j s_ij, l_i = sum_j exp(s_ij - m_i)
  (the report, section 3.3, saves O and the row statistics (m, l); their
  combination m + ln l is the one number the recomputation needs).
  A row with no allowed key has O_i = 0 and LSE_i = -inf.
* Backward -- the analytic gradient of O = softmax(S) V with respect to
  Q, K, V (the report's section 3.3 and the "backward" paragraph of the
  bowenzhou.top tutorial name dP, dS and the gradient accumulation; the
  formulas are the softmax Jacobian):
      dP_ij = dO_i . v_j
      D_i   = sum_j P_ij dP_ij
      dS_ij = P_ij (dP_ij - D_i)
      dQ_i  = scale * sum_j dS_ij k_j
      dK_j  = scale * sum_{h in group g} sum_i dS_ij q_i
      dV_j  = sum_{h in group g} sum_i P_ij dO_i

Masks (all boolean, combined with AND):
* causal, top-left aligned: key j allowed for query i iff j <= i;
* key padding: key j allowed iff j < L_b (query rows past L_b are still
  computed and still attend to the first min(i + 1, L_b) keys under causal);
* block mask BM of granularity ``mask_block``: allowed iff
  BM[i // mask_block][j // mask_block] != 0 (the block-sparse variant of the
  report, section 2.6 / section 3.5);
* sliding window (left, right): allowed iff i - left <= j <= i + right.
  The pages name the sliding window only as an attention variant (the
  synthesis page, section 5 item 1) and as one of the sparse patterns that
  skip blocks of the score matrix (the tutorial page, "sparse attention");
  this two-sided band is the plain reading (right = 0 with causal is the
  usual causal local attention).

Dropout (optional): with keep mask Z of one head (``oracle.philox``) and
realised keep probability q, the forward is O = (P o Z / q) V with P the
undropped softmax (its LSE unchanged), and the backward differentiates that:
      dV_j  = sum_i (P_ij Z_ij / q) dO_i
      dP_ij = (Z_ij / q) dO_i . v_j
      D_i   = sum_j P_ij dP_ij        (= dO_i . O_i)
      dS_ij = P_ij (dP_ij - D_i),  dQ and dK as above.
The zako-mio report (section 3.2) places dropout inside the fused kernel,
applied on chip and regenerated rather than stored; where it enters (on the
normalised probabilities, before the product with V) is the standard reading.

Everything is float64; inputs are the exact values the GPU sees, widened.
"""
from __future__ import annotations

import dataclasses
from typing import Optional, Sequence, Tuple

import numpy as np

from .philox import Dropout, HeadDropout

ROW_CHUNK = 128  # rows of S materialised at once (softmax is row-independent)


@dataclasses.dataclass(frozen=True)
class MaskSpec:
    """Mask of one (batch, head) problem."""

    causal: bool = False
    seqlen_k: Optional[int] = None  # valid key count L_b, or None for all
    block_mask: Optional[np.ndarray] = None  # [nqb, nkb] 0/1
    mask_block: int = 128
    window: Optional[Tuple[int, int]] = None  # (left, right) band, or None

    def allowed(self, rows: np.ndarray, cols: np.ndarray) -> np.ndarray:
        """Boolean [len(rows), len(cols)]: may query ``rows[a]`` see key ``cols[c]``."""
        i = np.asarray(rows, dtype=np.int64)[:, None]
        j = np.asarray(cols, dtype=np.int64)[None, :]
        ok = np.ones((i.shape[0], j.shape[1]), dtype=bool)
        if self.causal:
            ok &= j <= i
        if self.seqlen_k is not None:
            ok &= j < self.seqlen_k
        if self.block_mask is not None:
            bm = np.asarray(self.block_mask) != 0
            ok &= bm[i // self.mask_block, j // self.mask_block]
        if self.window is not None:
            left, right = self.window
            ok &= (j >= i - left) & (j <= i + right)
        return ok


def mask_for(b: int, *, causal=False, seqlens=None, block_mask=None,
             mask_block=128, window=None) -> MaskSpec:
    """MaskSpec of batch entry ``b`` from whole-problem mask arguments."""
    L = None if seqlens is None else int(np.asarray(seqlens)[b])
    win = None if window is None else (int(window[0]), int(window[1]))
    return MaskSpec(bool(causal), L, block_mask, mask_block, win)


def _softmax_rows(s: np.ndarray):
    """Two-pass row softmax of ``s`` (entries may be -inf).

    Returns (P, LSE). Rows whose entries are all -inf get P = 0, LSE = -inf.
    """
    m = s.max(axis=1)
    empty = np.isneginf(m)
    m0 = np.where(empty, 0.0, m)
    e = np.exp(s - m0[:, None])  # exp(-inf) == 0 exactly
    l = e.sum(axis=1)
    p = e / np.where(empty, 1.0, l)[:, None]
    with np.errstate(divide="ignore"):
        lse = np.where(empty, -np.inf, m0 + np.log(np.where(empty, 1.0, l)))
    return p, lse


def _scores(q_rows: np.ndarray, k: np.ndarray, scale: float, mask: MaskSpec,
            rows: np.ndarray) -> np.ndarray:
    """S rows with the mask applied as -inf (dense over all keys)."""
    s = float(scale) * (q_rows @ k.T)
    ok = mask.allowed(rows, np.arange(k.shape[0]))
    return np.where(ok, s, -np.inf)


def _chunks(rows: np.ndarray):
    for a in range(0, len(rows), ROW_CHUNK):
        yield rows[a:a + ROW_CHUNK]


def probabilities(q: np.ndarray, k: np.ndarray, scale: float, mask: MaskSpec,
                  rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """P = softmax(S) for the given query rows of one head ([rows, N])."""
    rows = np.arange(q.shape[0]) if rows is None else np.asarray(rows)
    s = _scores(q[rows], k, scale, mask, rows)
    return _softmax_rows(s)[0]


def head_forward(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                 mask: MaskSpec, rows: Optional[Sequence[int]] = None,
                 drop: Optional[HeadDropout] = None):
    """Algorithm-0 forward of one head for the given query rows.

    q: [N, d] (only ``rows`` are read), k, v: [N, d]. Returns (O[rows], LSE[rows]).
    With ``drop``, O = (P o Z / q) V and LSE is that of the undropped P.
    """
    rows = np.arange(q.shape[0]) if rows is None else np.asarray(rows, dtype=np.int64)
    o = np.zeros((len(rows), v.shape[1]))
    lse = np.zeros(len(rows))
    at = 0
    for rc in _chunks(rows):
        s = _scores(q[rc], k, scale, mask, rc)  # S = Q K^T (materialised)
        p, l = _softmax_rows(s)                  # P = softmax(S)
        if drop is not None:                     # P <- P o Z / q
            p = p * (drop.keep(rc, np.arange(k.shape[0])) * drop.scale)
        o[at:at + len(rc)] = p @ v               # O = P V
        lse[at:at + len(rc)] = l
        at += len(rc)
    return o, lse


def head_backward(q: np.ndarray, k: np.ndarray, v: np.ndarray, do: np.ndarray,
                  scale: float, mask: MaskSpec,
                  q_rows: Optional[Sequence[int]] = None,
                  k_rows: Optional[Sequence[int]] = None,
                  drop: Optional[HeadDropout] = None):
    """Analytic backward of one query head.

    Returns (dQ[q_rows], dK[k_rows], dV[k_rows]) where dK/dV hold this head's
    contribution only (a GQA group sums its heads). With both row sets None,
    everything is computed. With only ``k_rows`` given, every query row that
    can see one of those keys is visited (each with its full softmax row).
    """
    n = q.shape[0]
    all_rows = np.arange(n)
    want_q = all_rows if (q_rows is None and k_rows is None) else (
        None if q_rows is None else np.asarray(q_rows, dtype=np.int64))
    want_k = all_rows if (q_rows is None and k_rows is None) else (
        None if k_rows is None else np.asarray(k_rows, dtype=np.int64))

    dq = None if want_q is None else np.zeros((len(want_q), q.shape[1]))
    dk = None if want_k is None else np.zeros((len(want_k), k.shape[1]))
    dv = None if want_k is None else np.zeros((len(want_k), v.shape[1]))

    def grads_of(rc):
        s = _scores(q[rc], k, scale, mask, rc)
        p, _ = _softmax_rows(s)
        dp = do[rc] @ v.T                                  # dP = dO V^T
        pv = p                                             # what multiplies V
        if drop is not None:
            z = drop.keep(rc, np.arange(n)) * drop.scale   # Z / q
            pv = p * z
            dp = dp * z                                    # dP = (Z / q) o dO V^T
        dsum = (p * dp).sum(axis=1)                        # D_i = sum_j P dP
        ds = p * (dp - dsum[:, None])                      # dS = P (dP - D)
        return pv, ds

    if want_q is not None:
        at = 0
        for rc in _chunks(want_q):
            _, ds = grads_of(rc)
            dq[at:at + len(rc)] = float(scale) * (ds @ k)  # dQ = scale dS K
            at += len(rc)
    if want_k is not None:
        for rc in _chunks(all_rows):
            if not mask.allowed(rc, want_k).any():
                continue  # no row here sees any wanted key: contributes 0
            p, ds = grads_of(rc)
            dv += p[:, want_k].T @ do[rc]                      # dV = P^T dO
            dk += float(scale) * (ds[:, want_k].T @ q[rc])      # dK = scale dS^T Q
    return dq, dk, dv


def attention_forward(q, k, v, scale, *, causal=False, seqlens=None,
                      block_mask=None, mask_block=128, window=None,
                      dropout: Optional[Dropout] = None):
    """Whole-tensor forward. q: [B, Hq, N, d], k/v: [B, Hkv, N, d] (float64).

    Returns O [B, Hq, N, d] and LSE [B, Hq, N].
    """
    B, Hq, N, d = q.shape
    G = Hq // k.shape[1]
    o = np.zeros((B, Hq, N, v.shape[3]))
    lse = np.zeros((B, Hq, N))
    for b in range(B):
        m = mask_for(b, causal=causal, seqlens=seqlens, block_mask=block_mask,
                     mask_block=mask_block, window=window)
        for h in range(Hq):
            o[b, h], lse[b, h] = head_forward(
                q[b, h], k[b, h // G], v[b, h // G], scale, m,
                drop=None if dropout is None else dropout.head(b * Hq + h))
    return o, lse


def attention_decode(q, k, v, scale, *, seqlens=None):
    """Decoding: one query row per head against a key/value cache.

    q: [B, Hq, d], k/v: [B, Hkv, N, d]. The query sees cached keys
    0 .. L_b - 1 (L_b = seqlens[b], or N). Returns O [B, Hq, d] and
    LSE [B, Hq]. This is the forward above for a single row (the synthesis
    page, section 3 item 4: in decoding the score matrix is one row per
    head); the split-and-merge of the GPU path is not reproduced here.
    """
    B, Hq, d = q.shape
    G = Hq // k.shape[1]
    o = np.zeros((B, Hq, v.shape[3]))
    lse = np.zeros((B, Hq))
    for b in range(B):
        m = mask_for(b, seqlens=seqlens)
        for h in range(Hq):
            ob, lb = head_forward(q[b, h][None, :], k[b, h // G], v[b, h // G], scale, m,
                                  rows=[0])
            o[b, h], lse[b, h] = ob[0], lb[0]
    return o, lse


def attention_backward(q, k, v, do, scale, *, causal=False, seqlens=None,
                       block_mask=None, mask_block=128, window=None,
                       dropout: Optional[Dropout] = None):
    """Whole-tensor backward. Returns dQ [B,Hq,N,d], dK, dV [B,Hkv,N,d]."""
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    dq = np.zeros_like(q, dtype=np.float64)
    dk = np.zeros(k.shape)
    dv = np.zeros(v.shape)
    for b in range(B):
        m = mask_for(b, causal=causal, seqlens=seqlens, block_mask=block_mask,
                     mask_block=mask_block, window=window)
        for h in range(Hq):
            g = h // G
            a, bk, bv = head_backward(
                q[b, h], k[b, g], v[b, g], do[b, h], scale, m,
                drop=None if dropout is None else dropout.head(b * Hq + h))
            dq[b, h] = a
            dk[b, g] += bk
            dv[b, g] += bv
    return dq, dk, dv
