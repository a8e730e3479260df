"""Pins of the oracle's dropout: the Philox4x32-10 generator against its
published known-answer vectors, the keep-mask index mapping against a scalar
brute-force reading of its definition, statistics of the mask, unbiasedness
of the dropped forward (Monte Carlo over seeds), and the dropped backward
against finite differences of the dropped forward. Mutants of the dropout
path must fail at least one pin."""
from __future__ import annotations

import os

import numpy as np
import pytest

import oracle
import oracle.attention as OA
import oracle.philox as OP

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "philox4x32_10_kat.txt")


def _kat():
    out = []
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        lhs, rhs = line.split("->")
        a = [int(x, 16) for x in lhs.split()]
        b = [int(x, 16) for x in rhs.split()]
        out.append((a[:4], a[4:], b))
    return out


def test_philox_known_answer_vectors():
    kat = _kat()
    assert len(kat) == 3
    for ctr, key, want in kat:
        got = OP.philox4x32(np.array([ctr], dtype=np.uint64), key)[0]
        assert [int(x) for x in got] == want


def _philox_scalar(ctr, key):
    """One Philox4x32-10 call with Python ints (a second, loop-free-of-numpy
    reading of the same definition, used only to check index plumbing)."""
    x = [int(c) for c in ctr]
    k0, k1 = int(key[0]), int(key[1])
    for _ in range(10):
        p0 = x[0] * 0xD2511F53
        p1 = x[2] * 0xCD9E8D57
        x = [((p1 >> 32) ^ x[1] ^ k0) & 0xFFFFFFFF, p1 & 0xFFFFFFFF,
             ((p0 >> 32) ^ x[3] ^ k1) & 0xFFFFFFFF, p0 & 0xFFFFFFFF]
        k0 = (k0 + 0x9E3779B9) & 0xFFFFFFFF
        k1 = (k1 + 0xBB67AE85) & 0xFFFFFFFF
    return x


def test_scalar_reading_matches_known_answers():
    for ctr, key, want in _kat():
        assert _philox_scalar(ctr, key) == want


@pytest.mark.parametrize("seed,offset,bh", [(0, 0, 0), (0x0123456789ABCDEF, 7, 5),
                                            (2**64 - 1, 2**32 - 1, 1000)])
def test_uniform_mapping_matches_scalar_definition(seed, offset, bh):
    """u(i, j) = half (j mod 2) of word ((j div 2) mod 4) of
    Philox(counter = (j div 8, i, bh, offset), key = (seed lo, seed hi))."""
    d = OP.Dropout(0.3, seed, offset)
    rows = np.array([0, 1, 2, 77, 1023, 4096])
    cols = np.arange(0, 40)
    u = d.uniforms(bh, rows, cols)
    key = (seed & 0xFFFFFFFF, seed >> 32)
    for a, i in enumerate(rows):
        for c, j in enumerate(cols):
            j = int(j)
            w = _philox_scalar([j // 8, int(i), bh, offset], key)[(j // 2) % 4]
            want = (w >> 16) if j % 2 else (w & 0xFFFF)
            assert int(u[a, c]) == want, (i, j)
    keep = d.keep(bh, rows, cols)
    np.testing.assert_array_equal(keep, u < d.threshold)


def test_keep_threshold_edges():
    assert OP.keep_threshold(0.5) == 32768
    assert OP.keep_threshold(0.1) == 58982            # 58982.4 rounds down
    assert OP.keep_threshold(0.25) == 49152
    assert OP.keep_threshold(1e-6) == 65536           # keeps everything
    assert OP.keep_threshold(0.99999) == 1            # 0.655 rounds up to 1
    for bad in (0.0, 1.0, -0.1, 1.5, 0.999995):
        with pytest.raises(ValueError):
            OP.keep_threshold(bad)
    assert OP.Dropout(0.5).scale == 2.0
    assert OP.Dropout(0.25).scale == 65536.0 / 49152


def test_uniform_statistics():
    """16-bit uniforms: mean and variance of U{0..65535}; adjacent keys (the
    two halves of a word, and neighbouring words) and neighbouring rows are
    not copies of each other; the keep rate is q within 6 sigma."""
    d = OP.Dropout(0.2, seed=12345, offset=3)
    n = 512
    u = d.uniforms(9, np.arange(n), np.arange(n)).astype(np.float64)
    m = u.size
    mean, var = 65535 / 2, (65536**2 - 1) / 12
    assert abs(u.mean() - mean) < 6 * np.sqrt(var / m)
    assert abs(u.var() / var - 1) < 0.02
    for a, b in ((u[:, 0::2], u[:, 1::2]), (u[:, :-2], u[:, 2:]), (u[:, :-8], u[:, 8:]),
                 (u[:-1], u[1:])):
        eq = float((a == b).mean())
        assert eq < 20 / 65536, eq   # about 1/65536 for independent draws
        c = np.corrcoef(a.ravel(), b.ravel())[0, 1]
        assert abs(c) < 6 / np.sqrt(a.size), c
    keep = u < d.threshold
    q = d.threshold / 65536
    assert abs(keep.mean() - q) < 6 * np.sqrt(q * (1 - q) / m)


def test_streams_depend_on_every_counter_word_and_the_key():
    base = OP.Dropout(0.5, seed=1, offset=0)
    rows, cols = np.arange(64), np.arange(64)
    u0 = base.uniforms(0, rows, cols)
    for other in (base.uniforms(1, rows, cols),                       # head
                  OP.Dropout(0.5, seed=1, offset=1).uniforms(0, rows, cols),
                  OP.Dropout(0.5, seed=2, offset=0).uniforms(0, rows, cols),
                  OP.Dropout(0.5, seed=1 + 2**32, offset=0).uniforms(0, rows, cols),
                  base.uniforms(0, rows + 64, cols),                  # row
                  base.uniforms(0, rows, cols + 64)):                 # key group
        assert float((u0 == other).mean()) < 0.01


def rand(*shape, rng):
    return rng.standard_normal(shape)


def test_dropout_forward_is_unbiased():
    """E_seed[O_dropped] = O (Monte Carlo over 3000 seeds, within 6 sigma of
    the sample mean per element); the LSE does not depend on the mask."""
    rng = np.random.default_rng(5)
    B, H, n, d = 1, 1, 12, 3
    q, k, v = rand(B, H, n, d, rng=rng), rand(B, H, n, d, rng=rng), rand(B, H, n, d, rng=rng)
    o_ref, lse_ref = oracle.attention_forward(q, k, v, 0.8, causal=True)
    samples = []
    for s in range(3000):
        o, lse = oracle.attention_forward(q, k, v, 0.8, causal=True,
                                          dropout=OP.Dropout(0.4, seed=s))
        np.testing.assert_array_equal(lse, lse_ref)
        samples.append(o)
    x = np.stack(samples)
    sem = x.std(axis=0) / np.sqrt(len(samples))
    err = np.abs(x.mean(axis=0) - o_ref)
    assert np.all(err <= 6 * sem + 1e-12), float((err / (sem + 1e-30)).max())


def test_dropout_with_identity_values_exposes_the_scaled_mask():
    """V = I (N = d): O = P o Z / q exactly, zero exactly where dropped.
    At p = 0.3, (1 - p) 65536 = 45875.2, so T = 45875 and 1 / q = 65536 / 45875
    (not 1 / 0.7: the realised keep probability is what is undone)."""
    rng = np.random.default_rng(6)
    n = 16
    q, k = rand(1, 1, n, 4, rng=rng), rand(1, 1, n, 4, rng=rng)
    v = np.eye(n)[None, None]
    dr = OP.Dropout(0.3, seed=99, offset=4)
    o, _ = oracle.attention_forward(q, k, v, 0.6, dropout=dr)
    p = OA.probabilities(q[0, 0], k[0, 0], 0.6, OA.MaskSpec())
    keep = dr.uniforms(0, np.arange(n), np.arange(n)) < 45875
    assert 0 < keep.sum() < keep.size
    np.testing.assert_array_equal(o[0, 0] == 0, ~keep)
    np.testing.assert_allclose(o[0, 0], p * keep * (65536 / 45875), rtol=1e-14, atol=0)


def _loss(q, k, v, do, scale, kw):
    o, _ = oracle.attention_forward(q, k, v, scale, **kw)
    return float((o * do).sum())


FD_CASES = [
    dict(dropout=OP.Dropout(0.3, seed=7)),
    dict(causal=True, dropout=OP.Dropout(0.5, seed=8, offset=2)),
    dict(seqlens=np.array([5]), window=(3, 2), dropout=OP.Dropout(0.2, seed=9)),
]


@pytest.mark.parametrize("ci", range(len(FD_CASES)))
@pytest.mark.parametrize("G", [1, 2])
def test_dropout_finite_difference_gradients(ci, G):
    """The dropped backward is the gradient of the dropped forward at a fixed
    mask (central differences, h = 1e-6)."""
    kw = FD_CASES[ci]
    rng = np.random.default_rng(300 + ci + 10 * G)
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
        np.testing.assert_allclose(g, num, atol=5e-7, err_msg=name)


def test_dropout_d_identity():
    """D_i = sum_j P_ij dP_ij equals dO_i . O_i for the dropped O."""
    rng = np.random.default_rng(11)
    n, d = 20, 5
    q, k, v, do = (rand(n, d, rng=rng) for _ in range(4))
    dr = OP.Dropout(0.35, seed=3).head(0)
    m = OA.MaskSpec(causal=True)
    o, _ = OA.head_forward(q, k, v, 0.5, m, drop=dr)
    p = OA.probabilities(q, k, 0.5, m)
    z = dr.keep(np.arange(n), np.arange(n)) * dr.scale
    dp = z * (do @ v.T)
    np.testing.assert_allclose((p * dp).sum(axis=1), (do * o).sum(axis=1), atol=1e-13)


# ---------------------------------------------------------------- mutants

def _pins_pass():
    try:
        test_uniform_mapping_matches_scalar_definition(0x0123456789ABCDEF, 7, 5)
        test_dropout_with_identity_values_exposes_the_scaled_mask()
        test_dropout_finite_difference_gradients(1, 2)
    except (AssertionError, ValueError, IndexError):
        return False
    return True


def _unbiased_passes():
    try:
        test_dropout_forward_is_unbiased()
    except AssertionError:
        return False
    return True


@pytest.mark.parametrize("mutant", ["transposed", "half_order", "no_dp_mask", "scale_1_minus_p"])
def test_dropout_mutants_are_caught(mutant, monkeypatch):
    assert _pins_pass()
    if mutant == "transposed":
        orig = OP.Dropout.keep
        monkeypatch.setattr(OP.Dropout, "keep",
                            lambda self, bh, rows, cols: orig(self, bh, cols, rows).T)
    elif mutant == "half_order":
        orig_u = OP.Dropout.uniforms

        def u(self, bh, rows, cols):
            cols = np.asarray(cols)
            return orig_u(self, bh, rows, cols ^ 1)
        monkeypatch.setattr(OP.Dropout, "uniforms", u)
    elif mutant == "no_dp_mask":
        orig = OA.head_backward

        def hb(q, k, v, do, scale, mask, q_rows=None, k_rows=None, drop=None):
            # dP left unmasked: recompute the pieces without Z on dP.
            if drop is None:
                return orig(q, k, v, do, scale, mask, q_rows, k_rows)
            n = q.shape[0]
            p = OA.probabilities(q, k, scale, mask)
            z = drop.keep(np.arange(n), np.arange(n)) * drop.scale
            dp = do @ v.T
            ds = p * (dp - (p * dp).sum(axis=1)[:, None])
            return scale * ds @ k, scale * ds.T @ q, (p * z).T @ do
        monkeypatch.setattr(OA, "head_backward", hb)
    elif mutant == "scale_1_minus_p":
        monkeypatch.setattr(OP.Dropout, "scale", property(lambda self: 1.0 / (1.0 - self.p)))
    assert not _pins_pass(), f"mutant {mutant} survived every pin"


def test_dropout_placement_mutant_fails_unbiasedness(monkeypatch):
    """Dropping scores before the softmax (instead of probabilities after it)
    is biased, and the Monte-Carlo pin sees it."""
    assert _unbiased_passes()
    orig_hf = OA.head_forward

    def hf(q, k, v, scale, mask, rows=None, drop=None):
        if drop is None:
            return orig_hf(q, k, v, scale, mask, rows)
        rows = np.arange(q.shape[0]) if rows is None else np.asarray(rows)
        s = OA._scores(q[rows], k, scale, mask, rows)
        keep = drop.keep(rows, np.arange(k.shape[0]))
        s = np.where(keep, s, -np.inf)             # mask scores, then softmax
        p, lse = OA._softmax_rows(s)
        return p @ v, lse
    monkeypatch.setattr(OA, "head_forward", hf)
    assert not _unbiased_passes()
