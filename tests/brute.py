"""Scalar, loop-by-loop attention for tiny problems (pure Python floats).

Used only to pin the vectorised oracle. Nothing here uses numpy's matmul or
exp: each score is a Python sum of products, each exponential math.exp, and
the mask is re-derived from its plain-language rules:
causal (key index <= query index), key padding (key index < valid length),
block mask (the block of (query, key) is present), sliding window (the key
is at most `left` positions before and `right` positions after the query).
"""
import math


def allowed(i, j, causal=False, seqlen_k=None, block_mask=None, mask_block=128,
            window=None):
    if causal and j > i:
        return False
    if window is not None:
        left, right = window
        if i - j > left or j - i > right:
            return False
    if seqlen_k is not None and j >= seqlen_k:
        return False
    if block_mask is not None and not block_mask[i // mask_block][j // mask_block]:
        return False
    return True


def forward(q, k, v, scale, **mask):
    """q: list of N rows of d floats; k, v likewise. Returns (O rows, LSE list)."""
    n = len(q)
    o, lse = [], []
    for i in range(n):
        scores = {}
        for j in range(len(k)):
            if allowed(i, j, **mask):
                acc = 0.0
                for t in range(len(q[i])):
                    acc += q[i][t] * k[j][t]
                scores[j] = scale * acc
        if not scores:
            o.append([0.0] * len(v[0]))
            lse.append(-math.inf)
            continue
        m = max(scores.values())
        w = {j: math.exp(s - m) for j, s in scores.items()}
        total = sum(w.values())
        row = []
        for t in range(len(v[0])):
            row.append(sum(w[j] * v[j][t] for j in w) / total)
        o.append(row)
        lse.append(m + math.log(total))
    return o, lse
