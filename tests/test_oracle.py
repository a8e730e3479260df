"""Pins of the fp64 oracle against facts fixed by the pages and by mathematics.

Each test checks the oracle against something other than itself: a closed
form, an invariant, a textbook reduction, a brute-force scalar evaluation, or
finite differences. ``test_mutants_are_caught`` plants plausible mistakes in
the oracle (on the CPU) and checks that some pin fails for each.
"""
import math

import numpy as np
import pytest

import oracle
import oracle.attention as OA
from synth import bf16_bits_to_f64, butterfly_block_mask, draw_case
from tests import brute

RNG = np.random.default_rng(12345)


def rand(*shape, rng=RNG):
    return rng.standard_normal(shape)


MASKS = [
    dict(),
    dict(causal=True),
    dict(seqlen_k=5),
    dict(causal=True, seqlen_k=6),
    dict(block_mask=np.array([[1, 0, 1], [0, 1, 0], [1, 1, 1]]), mask_block=4),
    dict(causal=True, block_mask=np.array([[1, 0, 1], [1, 1, 0], [1, 1, 1]]), mask_block=4),
    dict(window=(2, 1)),
    dict(causal=True, window=(3, 0)),
    dict(seqlen_k=7, window=(1, 4)),
]
WINDOW_MASK = 6  # index of the first sliding-window entry


def _spec(m):
    return OA.MaskSpec(m.get("causal", False), m.get("seqlen_k"), m.get("block_mask"),
                       m.get("mask_block", 128), m.get("window"))


# ---------------------------------------------------------------- forward pins

@pytest.mark.parametrize("mi", range(len(MASKS)))
def test_brute_force_forward(mi):
    """Vectorised oracle == scalar triple loop (N = 12, d = 5)."""
    m = MASKS[mi]
    n, d = 12, 5
    q, k, v = rand(n, d), rand(n, d), rand(n, d)
    scale = 0.37
    o, lse = OA.head_forward(q, k, v, scale, _spec(m))
    bo, blse = brute.forward(q.tolist(), k.tolist(), v.tolist(), scale, **m)
    np.testing.assert_allclose(o, np.array(bo), rtol=0, atol=1e-13)
    bl = np.array(blse)
    assert np.array_equal(np.isneginf(lse), np.isneginf(bl))
    fin = np.isfinite(bl)
    np.testing.assert_allclose(lse[fin], bl[fin], rtol=0, atol=1e-13)


@pytest.mark.parametrize("mi", range(len(MASKS)))
def test_probability_rows_sum_to_one(mi):
    n, d = 12, 8
    q, k = rand(n, d) * 3, rand(n, d) * 3
    p = OA.probabilities(q, k, 0.5, _spec(MASKS[mi]))
    sums = p.sum(axis=1)
    nonempty = _spec(MASKS[mi]).allowed(np.arange(n), np.arange(n)).any(axis=1)
    np.testing.assert_allclose(sums[nonempty], 1.0, rtol=0, atol=1e-14)
    assert np.all(sums[~nonempty] == 0)
    assert np.all(p >= 0)


@pytest.mark.parametrize("mi", range(len(MASKS)))
def test_constant_v_returns_constant(mi):
    n, d = 12, 6
    c = rand(d)
    v = np.tile(c, (n, 1))
    o, _ = OA.head_forward(rand(n, d) * 4, rand(n, d) * 4, v, 0.8, _spec(MASKS[mi]))
    nonempty = _spec(MASKS[mi]).allowed(np.arange(n), np.arange(n)).any(axis=1)
    np.testing.assert_allclose(o[nonempty], np.tile(c, (nonempty.sum(), 1)), atol=1e-14)


def _allowed_counts_and_means(v, m, n):
    """Closed forms for Q = 0: mean of V over allowed keys, and their count."""
    counts, means = [], []
    for i in range(n):
        js = [j for j in range(n) if brute.allowed(i, j, **m)]
        counts.append(len(js))
        means.append(v[js].mean(axis=0) if js else np.zeros(v.shape[1]))
    return np.array(counts), np.array(means)


@pytest.mark.parametrize("mi", range(len(MASKS)))
def test_zero_query_gives_mean_and_log_count(mi):
    m = MASKS[mi]
    n, d = 12, 4
    v = rand(n, d)
    o, lse = OA.head_forward(np.zeros((n, d)), rand(n, d), v, 0.3, _spec(m))
    counts, means = _allowed_counts_and_means(v, m, n)
    np.testing.assert_allclose(o, means, atol=1e-14)
    fin = counts > 0
    np.testing.assert_allclose(lse[fin], np.log(counts[fin]), atol=1e-14)
    assert np.all(np.isneginf(lse[~fin]))


def test_zero_query_closed_forms_named_cases():
    """Q = 0: non-causal = column mean of V, LSE = ln N; causal = prefix mean,
    LSE = ln(i+1); butterfly on 16 blocks of 4 -> 5 blocks x 4 keys, ln 20."""
    n, d = 64, 3
    v = rand(n, d)
    z = np.zeros((n, d))
    o, lse = OA.head_forward(z, rand(n, d), v, 1.0, OA.MaskSpec())
    np.testing.assert_allclose(o, np.tile(v.mean(axis=0), (n, 1)), atol=1e-14)
    np.testing.assert_allclose(lse, math.log(n), atol=1e-14)
    o, lse = OA.head_forward(z, rand(n, d), v, 1.0, OA.MaskSpec(causal=True))
    prefix = np.cumsum(v, axis=0) / np.arange(1, n + 1)[:, None]
    np.testing.assert_allclose(o, prefix, atol=1e-13)
    np.testing.assert_allclose(lse, np.log(np.arange(1, n + 1)), atol=1e-14)
    bm = butterfly_block_mask(16)
    o, lse = OA.head_forward(z, rand(n, d), v, 1.0, OA.MaskSpec(block_mask=bm, mask_block=4))
    np.testing.assert_allclose(lse, math.log(20), atol=1e-14)
    # padding: count = min(i + 1, L) under causal
    L = 37
    o, lse = OA.head_forward(z, rand(n, d), v, 1.0, OA.MaskSpec(causal=True, seqlen_k=L))
    np.testing.assert_allclose(lse, np.log(np.minimum(np.arange(1, n + 1), L)), atol=1e-14)
    # sliding window (l, r): count = min(i, l) + min(n - 1 - i, r) + 1, and the
    # output is the mean of V over the band
    l, r = 5, 2
    o, lse = OA.head_forward(z, rand(n, d), v, 1.0, OA.MaskSpec(window=(l, r)))
    i = np.arange(n)
    cnt = np.minimum(i, l) + np.minimum(n - 1 - i, r) + 1
    np.testing.assert_allclose(lse, np.log(cnt), atol=1e-14)
    band = np.array([v[max(0, t - l):min(n, t + r + 1)].mean(axis=0) for t in range(n)])
    np.testing.assert_allclose(o, band, atol=1e-14)


def test_window_of_width_zero_is_the_diagonal():
    """Window (0, 0): each row sees only its own key, so O_i = V_i and
    LSE_i = scale * q_i . k_i exactly (a one-term softmax)."""
    n, d = 20, 7
    q, k, v = rand(n, d), rand(n, d), rand(n, d)
    o, lse = OA.head_forward(q, k, v, 0.6, OA.MaskSpec(window=(0, 0)))
    np.testing.assert_allclose(o, v, atol=1e-15)
    np.testing.assert_allclose(lse, 0.6 * (q * k).sum(axis=1), atol=1e-14)


def test_window_covering_everything_is_no_window():
    n, d = 24, 5
    q, k, v = rand(n, d), rand(n, d), rand(n, d)
    for causal in (False, True):
        o1, l1 = OA.head_forward(q, k, v, 0.4, OA.MaskSpec(causal=causal))
        o2, l2 = OA.head_forward(q, k, v, 0.4, OA.MaskSpec(causal=causal, window=(n, n)))
        np.testing.assert_array_equal(o1, o2)
        np.testing.assert_array_equal(l1, l2)


def _partial(q, k, v, scale, cols):
    """Unnormalised partial of one key block: (m, l, O~) over ``cols``."""
    s = scale * (q @ k[cols].T)
    m = s.max(axis=1)
    e = np.exp(s - m[:, None])
    return m, e.sum(axis=1), e @ v[cols]


def _merge(parts):
    """Merge rule for softmax partials (bowenzhou.top tutorial, exercise 2):
    m' = max m_k, l' = sum l_k e^{m_k - m'}, O~' = sum O~_k e^{m_k - m'}."""
    m = np.max([p[0] for p in parts], axis=0)
    l = sum(p[1] * np.exp(p[0] - m) for p in parts)
    ot = sum(p[2] * np.exp(p[0] - m)[:, None] for p in parts)
    return ot / l[:, None], m + np.log(l)


def test_two_block_merge_equals_full_softmax():
    n, d = 40, 16
    q, k, v = rand(n, d) * 2, rand(n, d) * 2, rand(n, d)
    o, lse = OA.head_forward(q, k, v, 0.25, OA.MaskSpec())
    mo, ml = _merge([_partial(q, k, v, 0.25, np.arange(0, 17)),
                     _partial(q, k, v, 0.25, np.arange(17, n))])
    np.testing.assert_allclose(o, mo, atol=1e-13)
    np.testing.assert_allclose(lse, ml, atol=1e-13)


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_k_way_merge_over_random_partition(seed):
    rng = np.random.default_rng(seed)
    n, d = 50, 8
    q, k, v = rand(n, d, rng=rng) * 3, rand(n, d, rng=rng) * 3, rand(n, d, rng=rng)
    perm = rng.permutation(n)
    cuts = np.sort(rng.choice(np.arange(1, n), size=4, replace=False))
    parts = [_partial(q, k, v, 0.6, c) for c in np.split(perm, cuts)]
    mo, ml = _merge(parts)
    o, lse = OA.head_forward(q, k, v, 0.6, OA.MaskSpec())
    np.testing.assert_allclose(o, mo, atol=1e-13)
    np.testing.assert_allclose(lse, ml, atol=1e-13)


def test_shift_invariance_of_keys():
    """K_j -> K_j + u leaves O unchanged and shifts LSE_i by scale * q_i . u,
    even for |u| = 1e3 (the max subtraction keeps exp in range)."""
    n, d = 20, 8
    q, k, v = rand(n, d), rand(n, d), rand(n, d)
    u = rand(d)
    u *= 1e3 / np.linalg.norm(u)
    scale = 0.35
    o, lse = OA.head_forward(q, k, v, scale, OA.MaskSpec())
    o2, lse2 = OA.head_forward(q, k + u, v, scale, OA.MaskSpec())
    assert np.all(np.isfinite(o2))
    np.testing.assert_allclose(o2, o, atol=1e-10)
    np.testing.assert_allclose(lse2 - lse, scale * q @ u, rtol=1e-12, atol=1e-9)


def test_single_key():
    n, d = 10, 4
    q, k, v = rand(n, d), rand(n, d), rand(n, d)
    o, lse = OA.head_forward(q, k, v, 0.5, OA.MaskSpec(seqlen_k=1))
    np.testing.assert_allclose(o, np.tile(v[0], (n, 1)), atol=1e-15)
    np.testing.assert_allclose(lse, 0.5 * q @ k[0], atol=1e-14)
    o, lse = OA.head_forward(q, k, v, 0.5, OA.MaskSpec(causal=True))
    np.testing.assert_allclose(o[0], v[0], atol=1e-15)
    np.testing.assert_allclose(lse[0], 0.5 * q[0] @ k[0], atol=1e-14)


def test_empty_rows():
    n, d = 8, 4
    q, k, v, do = rand(n, d), rand(n, d), rand(n, d), rand(n, d)
    bm = np.array([[0, 1], [1, 1]])
    m = OA.MaskSpec(causal=True, block_mask=bm, mask_block=4)
    o, lse = OA.head_forward(q, k, v, 0.5, m)
    assert np.all(o[:4] == 0) and np.all(np.isneginf(lse[:4]))
    dq, dk, dv = OA.head_backward(q, k, v, do, 0.5, m)
    assert np.all(dq[:4] == 0)
    m0 = OA.MaskSpec(seqlen_k=0)
    o, lse = OA.head_forward(q, k, v, 0.5, m0)
    assert np.all(o == 0) and np.all(np.isneginf(lse))
    dq, dk, dv = OA.head_backward(q, k, v, do, 0.5, m0)
    assert not dq.any() and not dk.any() and not dv.any()


def test_block_mask_reductions():
    n, d = 16, 4
    q, k, v = rand(n, d), rand(n, d), rand(n, d)
    full = OA.head_forward(q, k, v, 0.5, OA.MaskSpec())
    ones = OA.head_forward(q, k, v, 0.5, OA.MaskSpec(block_mask=np.ones((4, 4)), mask_block=4))
    np.testing.assert_array_equal(full[0], ones[0])
    np.testing.assert_array_equal(full[1], ones[1])
    diag = OA.head_forward(q, k, v, 0.5, OA.MaskSpec(block_mask=np.eye(4), mask_block=4))
    for b in range(4):
        sl = slice(4 * b, 4 * b + 4)
        ob, lb = OA.head_forward(q[sl], k[sl], v[sl], 0.5, OA.MaskSpec())
        np.testing.assert_allclose(diag[0][sl], ob, atol=1e-15)
        np.testing.assert_allclose(diag[1][sl], lb, atol=1e-15)


def test_row_subsets_match_full():
    n, d = 300, 8
    q, k, v, do = rand(n, d), rand(n, d), rand(n, d), rand(n, d)
    m = OA.MaskSpec(causal=True, seqlen_k=250)
    o, lse = OA.head_forward(q, k, v, 0.4, m)
    rows = np.array([0, 5, 127, 128, 129, 299])
    o2, lse2 = OA.head_forward(q, k, v, 0.4, m, rows=rows)
    np.testing.assert_array_equal(o[rows], o2)
    np.testing.assert_array_equal(lse[rows], lse2)
    dq, dk, dv = OA.head_backward(q, k, v, do, 0.4, m)
    kr = np.array([0, 1, 130, 249, 250, 299])
    dq2, _, _ = OA.head_backward(q, k, v, do, 0.4, m, q_rows=rows)
    _, dk2, dv2 = OA.head_backward(q, k, v, do, 0.4, m, k_rows=kr)
    np.testing.assert_allclose(dq[rows], dq2, atol=1e-14)
    np.testing.assert_allclose(dk[kr], dk2, atol=1e-14)
    np.testing.assert_allclose(dv[kr], dv2, atol=1e-14)


# ---------------------------------------------------------------- GQA

def test_gqa_equals_repeated_mha():
    B, Hq, Hkv, n, d = 2, 4, 2, 10, 4
    q, do = rand(B, Hq, n, d), rand(B, Hq, n, d)
    k, v = rand(B, Hkv, n, d), rand(B, Hkv, n, d)
    kr, vr = np.repeat(k, 2, axis=1), np.repeat(v, 2, axis=1)
    kw = dict(causal=True, seqlens=np.array([7, 10]))
    o, lse = oracle.attention_forward(q, k, v, 0.5, **kw)
    o2, lse2 = oracle.attention_forward(q, kr, vr, 0.5, **kw)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(lse, lse2)
    dq, dk, dv = oracle.attention_backward(q, k, v, do, 0.5, **kw)
    dq2, dk2, dv2 = oracle.attention_backward(q, kr, vr, do, 0.5, **kw)
    np.testing.assert_allclose(dq, dq2, atol=1e-15)
    np.testing.assert_allclose(dk, dk2[:, 0::2] + dk2[:, 1::2], atol=1e-14)
    np.testing.assert_allclose(dv, dv2[:, 0::2] + dv2[:, 1::2], atol=1e-14)


# ---------------------------------------------------------------- backward pins

def _loss(q, k, v, do, scale, kw):
    o, _ = oracle.attention_forward(q, k, v, scale, **kw)
    return float((o * do).sum())


FD_CASES = [
    dict(),
    dict(causal=True),
    dict(seqlens=np.array([5])),
    dict(causal=True, seqlens=np.array([4])),
    dict(block_mask=np.array([[1, 0], [1, 1]]), mask_block=4),
    dict(window=(2, 1)),
    dict(causal=True, window=(2, 0)),
]


@pytest.mark.parametrize("ci", range(len(FD_CASES)))
@pytest.mark.parametrize("G", [1, 2])
def test_finite_difference_gradients(ci, G):
    kw = FD_CASES[ci]
    rng = np.random.default_rng(100 + ci + 10 * G)
    B, Hkv, n, d = 1, 1, 8, 3
    Hq = Hkv * G
    q, do = rand(B, Hq, n, d, rng=rng), rand(B, Hq, n, d, rng=rng)
    k, v = rand(B, Hkv, n, d, rng=rng), rand(B, Hkv, n, d, rng=rng)
    scale = 0.7
    dq, dk, dv = oracle.attention_backward(q, k, v, do, scale, **kw)
    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            x0 = x[idx]
            x[idx] = x0 + h
            lp = _loss(q, k, v, do, scale, kw)
            x[idx] = x0 - h
            lm = _loss(q, k, v, do, scale, kw)
            x[idx] = x0
            num[idx] = (lp - lm) / (2 * h)
        np.testing.assert_allclose(g, num, atol=2e-7, err_msg=name)


def test_d_identity_and_gradient_sums():
    """D_i = dO_i . O_i; sum_j dK_j = 0 per kv head; sum_j dV_j = sum of dO
    over the rows that see at least one key."""
    B, Hq, Hkv, n, d = 1, 4, 2, 40, 8
    q, do = rand(B, Hq, n, d), rand(B, Hq, n, d)
    k, v = rand(B, Hkv, n, d), rand(B, Hkv, n, d)
    kw = dict(causal=True, seqlens=np.array([30]))
    o, _ = oracle.attention_forward(q, k, v, 0.5, **kw)
    m = OA.mask_for(0, **kw)
    p = OA.probabilities(q[0, 0], k[0, 0], 0.5, m)
    dp = do[0, 0] @ v[0, 0].T
    np.testing.assert_allclose((p * dp).sum(axis=1), (do[0, 0] * o[0, 0]).sum(axis=1),
                               atol=1e-13)
    dq, dk, dv = oracle.attention_backward(q, k, v, do, 0.5, **kw)
    np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-13)
    for g in range(Hkv):
        want = do[0, 2 * g:2 * g + 2].sum(axis=(0, 1))
        np.testing.assert_allclose(dv[0, g].sum(axis=0), want, atol=1e-12)


# ---------------------------------------------------------------- inputs

def test_bf16_inputs_widen_exactly():
    inp = draw_case(1, 2, 1, 33, 8, "bf16", seed=3)
    x = bf16_bits_to_f64(inp.q)
    # every value is exactly representable with an 8-bit significand
    mant, _ = np.frexp(x)
    assert np.all(mant * 2 ** 8 == np.round(mant * 2 ** 8))


# ---------------------------------------------------------------- decode pins

def test_decode_brute_force_and_closed_forms():
    """Decoding (one query row against a cache): the scalar brute force for
    several cache lengths; Q = 0 gives the mean of the first L values and
    LSE = ln L; an empty cache gives O = 0, LSE = -inf."""
    rng = np.random.default_rng(71)
    B, Hq, Hkv, n, d = 3, 4, 2, 11, 5
    q, k, v = rand(B, Hq, d, rng=rng), rand(B, Hkv, n, d, rng=rng), rand(B, Hkv, n, d, rng=rng)
    L = np.array([11, 4, 0])
    o, lse = oracle.attention_decode(q, k, v, 0.45, seqlens=L)
    for b in range(B):
        for h in range(Hq):
            g = h // 2
            bo, bl = brute.forward([q[b, h].tolist()], k[b, g].tolist(), v[b, g].tolist(), 0.45,
                                   seqlen_k=int(L[b]))
            np.testing.assert_allclose(o[b, h], bo[0], atol=1e-13)
            if L[b] == 0:
                assert np.isneginf(lse[b, h]) and not o[b, h].any()
            else:
                np.testing.assert_allclose(lse[b, h], bl[0], atol=1e-13)
    o0, l0 = oracle.attention_decode(np.zeros_like(q), k, v, 0.45, seqlens=L)
    for b in range(2):
        np.testing.assert_allclose(o0[b], np.repeat(v[b, :, :L[b]].mean(axis=1), 2, axis=0),
                                   atol=1e-14)
        np.testing.assert_allclose(l0[b], math.log(L[b]), atol=1e-14)


def test_decode_is_the_last_row_of_causal_attention():
    """With the whole cache visible, decoding the last position's query
    equals the last row of causal attention over the sequence."""
    rng = np.random.default_rng(72)
    B, Hq, Hkv, n, d = 2, 4, 1, 9, 6
    q, k, v = rand(B, Hq, n, d, rng=rng), rand(B, Hkv, n, d, rng=rng), rand(B, Hkv, n, d, rng=rng)
    of, lf = oracle.attention_forward(q, k, v, 0.3, causal=True)
    od, ld = oracle.attention_decode(q[:, :, -1], k, v, 0.3)
    np.testing.assert_allclose(od, of[:, :, -1], atol=1e-14)
    np.testing.assert_allclose(ld, lf[:, :, -1], atol=1e-14)


# ---------------------------------------------------------------- mutants

def _pins_pass():
    """Run a compact set of pins against the (possibly mutated) oracle."""
    try:
        test_brute_force_forward(1)
        test_brute_force_forward(2)
        test_brute_force_forward(4)
        test_brute_force_forward(WINDOW_MASK)
        test_zero_query_closed_forms_named_cases()
        test_gqa_equals_repeated_mha()
        test_finite_difference_gradients(1, 2)
        test_d_identity_and_gradient_sums()
    except (AssertionError, ValueError, IndexError):
        return False
    return True


def _mut_causal_flipped(self, rows, cols):
    """Causal mask with the inequality reversed (j >= i)."""
    i = np.asarray(rows, dtype=np.int64)[:, None]
    j = np.asarray(cols, dtype=np.int64)[None, :]
    ok = np.ones((i.shape[0], j.shape[1]), dtype=bool)
    if self.causal:
        ok &= j >= i
    if self.seqlen_k is not None:
        ok &= j < self.seqlen_k
    if self.block_mask is not None:
        ok &= np.asarray(self.block_mask)[i // self.mask_block, j // self.mask_block] != 0
    return ok


def _mut_no_scale(q_rows, k, scale, mask, rows):
    """Scores without the softmax scale."""
    s = q_rows @ k.T
    ok = mask.allowed(rows, np.arange(k.shape[0]))
    return np.where(ok, s, -np.inf)


def _mut_lse_without_max(s):
    """LSE that forgets to add back the row max (ln l only)."""
    p, lse = OA.__dict__["_orig_softmax"](s)
    m = s.max(axis=1)
    return p, np.where(np.isfinite(lse), lse - m, lse)


def _mut_window_swapped(self, rows, cols):
    """Sliding window with its left and right widths exchanged."""
    i = np.asarray(rows, dtype=np.int64)[:, None]
    j = np.asarray(cols, dtype=np.int64)[None, :]
    ok = np.ones((i.shape[0], j.shape[1]), dtype=bool)
    if self.causal:
        ok &= j <= i
    if self.seqlen_k is not None:
        ok &= j < self.seqlen_k
    if self.block_mask is not None:
        ok &= np.asarray(self.block_mask)[i // self.mask_block, j // self.mask_block] != 0
    if self.window is not None:
        right, left = self.window
        ok &= (j >= i - left) & (j <= i + right)
    return ok


@pytest.mark.parametrize("mutant", ["causal", "scale", "lse", "dq_scale", "ds_no_d",
                                    "gqa_index", "window_swapped"])
def test_mutants_are_caught(mutant, monkeypatch):
    assert _pins_pass()  # sanity: the real oracle passes
    if mutant == "causal":
        monkeypatch.setattr(OA.MaskSpec, "allowed", _mut_causal_flipped)
    elif mutant == "window_swapped":
        monkeypatch.setattr(OA.MaskSpec, "allowed", _mut_window_swapped)
    elif mutant == "scale":
        monkeypatch.setattr(OA, "_scores", _mut_no_scale)
    elif mutant == "lse":
        monkeypatch.setattr(OA, "_orig_softmax", OA._softmax_rows, raising=False)
        monkeypatch.setattr(OA, "_softmax_rows", _mut_lse_without_max)
    elif mutant == "dq_scale":
        orig = OA.head_backward

        def hb(q, k, v, do, scale, mask, q_rows=None, k_rows=None, drop=None):
            dq, dk, dv = orig(q, k, v, do, scale, mask, q_rows, k_rows)
            return (None if dq is None else dq / scale), dk, dv
        monkeypatch.setattr(OA, "head_backward", hb)
    elif mutant == "ds_no_d":
        def hb(q, k, v, do, scale, mask, q_rows=None, k_rows=None, drop=None):
            # dS = P * dP: the -D_i term dropped.
            p = OA.probabilities(q, k, scale, mask)
            dp = do @ v.T
            ds = p * dp
            return scale * ds @ k, scale * ds.T @ q, p.T @ do
        monkeypatch.setattr(OA, "head_backward", hb)
    elif mutant == "gqa_index":
        def fwd(q, k, v, scale, *, causal=False, seqlens=None, block_mask=None,
                mask_block=128):
            B, Hq, N, d = q.shape
            Hkv = k.shape[1]
            o = np.zeros((B, Hq, N, v.shape[3]))
            lse = np.zeros((B, Hq, N))
            for b in range(B):
                m = OA.mask_for(b, causal=causal, seqlens=seqlens,
                                block_mask=block_mask, mask_block=mask_block)
                for h in range(Hq):
                    o[b, h], lse[b, h] = OA.head_forward(q[b, h], k[b, h % Hkv],
                                                         v[b, h % Hkv], scale, m)
            return o, lse
        monkeypatch.setattr(oracle, "attention_forward", fwd)
    assert not _pins_pass(), f"mutant {mutant} survived every pin"
