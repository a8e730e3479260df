"""Helpers shared by the GPU parity tests: device copies, error metrics and
the expected tile-visit set."""
from __future__ import annotations

import numpy as np
import torch

import oracle
import oracle.attention as OA

# Tolerances (fp32 and bf16 bars of the parity contract).
TOL_FP32_O = 1e-5
TOL_FP32_LSE = 1e-5
TOL_BF16_O_ABS = 1e-2
TOL_BF16_O_RELF = 5e-3
TOL_BF16_LSE = 1e-4
TOL_BF16_GRAD_RELF = 1e-2
BF16_HALF_ULP_REL = 2.0 ** -8  # rounding one value to bf16 moves it by <= 2^-8 |x|


def dev(arr: np.ndarray, dtype: str) -> torch.Tensor:
    """numpy input (bf16 bits or fp32) -> contiguous CUDA tensor."""
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).cuda()


def host64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to(torch.float64).cpu().numpy()


def relf(x: np.ndarray, ref: np.ndarray) -> float:
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(x - ref) / (den if den > 0 else 1.0))


def check_o(o: np.ndarray, ref: np.ndarray, o_is_bf16: bool, what=""):
    """bf16 bar: max |O - O_ref| <= 1e-2 (plus the bf16 half-ULP of |O_ref| when
    O itself is stored in bf16) and relative Frobenius <= 5e-3."""
    err = np.abs(o - ref)
    bound = TOL_BF16_O_ABS + (BF16_HALF_ULP_REL * np.abs(ref) if o_is_bf16 else 0.0)
    worst = np.unravel_index(np.argmax(err - bound), err.shape)
    assert np.all(err <= bound), (
        f"{what} O max abs err {err.max():.3g} at {worst} (|ref| {abs(ref[worst]):.3g})")
    r = relf(o, ref)
    assert r <= TOL_BF16_O_RELF, f"{what} O relF {r:.3g}"
    return float(err.max()), r


def check_lse(lse: np.ndarray, ref: np.ndarray, tol: float, what=""):
    assert np.array_equal(np.isneginf(lse), np.isneginf(ref)), f"{what} LSE -inf pattern differs"
    fin = np.isfinite(ref)
    if fin.any():
        e = float(np.abs(lse[fin] - ref[fin]).max())
        assert e <= tol, f"{what} LSE abs err {e:.3g}"
        return e
    return 0.0


def check_grad(g: np.ndarray, ref: np.ndarray, name: str, what=""):
    r = relf(g, ref)
    assert r <= TOL_BF16_GRAD_RELF, f"{what} {name} relF {r:.3g}"
    return r


def expected_tiles(B, Hq, N, causal, seqlens, block_mask, window=None) -> np.ndarray:
    """bool [B, Hq, nlb, nlb]: 128 x 128 tiles holding at least one allowed
    (query, key) pair, derived from the mask definitions. With a sliding
    window (left, right), query row i allows keys i - left .. i + right, so
    the rows q0..q1 of a row block allow at most keys q0 - left .. q1 + right
    (and .. q1 under causal), every one of which some row of the block sees."""
    nlb = -(-N // 128)
    qb = np.arange(nlb)[:, None]
    kb = np.arange(nlb)[None, :]
    out = np.zeros((B, Hq, nlb, nlb), dtype=bool)
    for b in range(B):
        L = N if seqlens is None else int(min(max(seqlens[b], 0), N))
        t = kb * 128 < L
        if causal:
            t = t & (kb <= qb)
        if window is not None:
            first_row, last_row = qb * 128, np.minimum(qb * 128 + 127, N - 1)
            first_key, last_key = kb * 128, kb * 128 + 127
            t = t & (last_key >= first_row - window[0]) & (first_key <= last_row + window[1])
        if block_mask is not None:
            t = t & (np.asarray(block_mask)[:nlb, :nlb] != 0)
        out[b] = np.broadcast_to(t, (nlb, nlb))
    return out


def decode_log(words: torch.Tensor, B, Hq, N) -> np.ndarray:
    nlb = -(-N // 128)
    w = -(-nlb // 32)
    a = words.cpu().numpy().view(np.uint32).reshape(B, Hq, nlb, w)
    bits = np.zeros((B, Hq, nlb, nlb), dtype=bool)
    for kb in range(nlb):
        bits[..., kb] = (a[..., kb // 32] >> np.uint32(kb % 32)) & 1
    return bits


def oracle_heads(inp, heads, *, backward=True, q_rows=None, k_rows=None, dropout=None):
    """Oracle results for selected (b, h) query heads.

    Returns dict (b, h) -> dict(o, lse, dq) for q_rows (all rows if None),
    and (b, g) -> dict(dk, dv) summed over the whole GQA group for k_rows.
    ``dropout`` is an ``oracle.Dropout`` applied to every head.
    """
    w = inp.workload
    G = w.heads_q // w.heads_kv
    res = {}
    kv_done = set()
    for (b, h) in heads:
        m = OA.mask_for(b, causal=w.causal, seqlens=inp.seqlens, block_mask=inp.block_mask,
                        window=inp.window)
        g = h // G
        q = inp.as_f64("q", (b, h))
        k = inp.as_f64("k", (b, g))
        v = inp.as_f64("v", (b, g))
        drop = None if dropout is None else dropout.head(b * w.heads_q + h)
        o, lse = oracle.head_forward(q, k, v, inp.scale, m, rows=q_rows, drop=drop)
        ent = dict(o=o, lse=lse)
        if backward:
            do = inp.as_f64("do", (b, h))
            dq, _, _ = oracle.head_backward(q, k, v, do, inp.scale, m,
                                            q_rows=np.arange(w.seqlen) if q_rows is None else q_rows,
                                            drop=drop)
            ent["dq"] = dq
            if (b, g) not in kv_done:
                kv_done.add((b, g))
                kr = np.arange(w.seqlen) if k_rows is None else k_rows
                dk = np.zeros((len(kr), w.head_dim))
                dv = np.zeros((len(kr), w.head_dim))
                for hh in range(g * G, (g + 1) * G):
                    qh = inp.as_f64("q", (b, hh))
                    doh = inp.as_f64("do", (b, hh))
                    dh = None if dropout is None else dropout.head(b * w.heads_q + hh)
                    _, a, c = oracle.head_backward(qh, k, v, doh, inp.scale, m, k_rows=kr,
                                                   drop=dh)
                    dk += a
                    dv += c
                res[(b, g, "kv")] = dict(dk=dk, dv=dv)
        res[(b, h)] = ent
    return res
