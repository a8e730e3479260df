"""GPU parity of in-kernel dropout.

* The keep mask, bit-exact, as each kernel applies it: with Q = 0 every
  allowed score is 0 and P is uniform; a block mask that is a permutation of
  the 128-key tiles gives each query tile exactly one key tile; then
  - forward: V one-hot (v_j = e_(j mod 128)) makes O[i, c] nonzero exactly
    when key 128 f(qb) + c is kept for row i;
  - dK/dV: dO one-hot makes dV[j, c] nonzero exactly when row
    128 g(kb) + c keeps key j;
  - dQ: K one-hot and dO . v_j = 1 give dQ[i, c] = (scale / q) (1/128)
    (Z_ij - k_i / 128) (k_i the row's kept count), positive exactly when
    kept.
  (d = 64 covers the two 64-column halves of a tile in two launches.)
* Random inputs against the fp64 oracle with the same seed and offset, at the
  bf16 bars, over the mask kinds; determinism; full-size sampled rows.
"""
import numpy as np
import pytest
import torch

import exact_io_aware_29_amd as fa
import oracle
from synth import WORKLOADS, draw, draw_case
from tests.gpu_util import (TOL_BF16_LSE, check_grad, check_lse, check_o, dev, host64,
                            oracle_heads)

pytestmark = pytest.mark.gpu

SEED = 0x0123456789ABCDEF  # both key words nonzero
OFFSET = 7


def _p32(p):
    return float(np.float32(p))


def _perm(nb):
    """Query tile qb sees key tile f(qb) = (3 qb + 1) mod nb (a permutation)."""
    assert np.gcd(3, nb) == 1
    f = (3 * np.arange(nb) + 1) % nb
    bm = np.zeros((nb, nb), dtype=np.uint8)
    bm[np.arange(nb), f] = 1
    return f, bm


def _onehot(n, d, half):
    """[n, d] with row j = e_(j mod 128 - 64 half) when that index lies in
    [0, d), else zero."""
    m = np.zeros((n, d), dtype=np.float32)
    j = np.arange(n)
    c = j % 128 - 64 * half
    ok = (c >= 0) & (c < d)
    m[j[ok], c[ok]] = 1.0
    return m


def check_o_dropped(o, o_ref, drop, o_is_bf16, what):
    """The O bar applied to q O: with dropout O = (1/q) sum_j P_ij Z_ij v_j, a
    sub-convex combination of V rows scaled by the exact 1/q, and the
    accumulation (and its rounding) acts on q O; bf16 output rounding stays
    relative. Without the rescale the absolute bar would tighten by 1/q."""
    q = 1.0 / drop.scale
    return check_o(o * q, o_ref * q, o_is_bf16, what)


def _t(a, dtype):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dtype).cuda()


MASK_CASES = [(64, torch.bfloat16), (128, torch.bfloat16), (64, torch.float32),
              (128, torch.float32)]


@pytest.mark.parametrize("d,dt", MASK_CASES, ids=[f"d{d}-{str(t)[6:]}" for d, t in MASK_CASES])
def test_forward_keep_mask_bit_exact(d, dt):
    B, Hq, Hkv, nb, p = 2, 4, 2, 4, 0.5
    N = 128 * nb
    f, bm = _perm(nb)
    drop = oracle.Dropout(_p32(p), SEED, OFFSET)
    rng = np.random.default_rng(1)
    q = torch.zeros((B, Hq, N, d), dtype=dt, device="cuda")
    k = _t(rng.standard_normal((B, Hkv, N, d)), dt)
    bmt = torch.from_numpy(bm).cuda()
    for half in range(128 // d):
        print(f"forward keep mask d={d} {dt} half={half}", flush=True)
        v = _t(np.broadcast_to(_onehot(N, d, half), (B, Hkv, N, d)), dt)
        o, lse, _ = fa.fa_fwd(q, k, v, scale=0.125, block_mask=bmt, o_dtype=torch.float32,
                              dropout_p=p, dropout_seed=SEED, dropout_offset=OFFSET)
        o = o.cpu().numpy()
        rows = np.arange(N)
        for b in range(B):
            for h in range(Hq):
                keys = 128 * f[rows // 128][:, None] + 64 * half + np.arange(d)[None, :]
                want = np.zeros((N, d), dtype=bool)
                for i in range(N):
                    want[i] = drop.keep(b * Hq + h, [i], keys[i])[0]
                np.testing.assert_array_equal(o[b, h] != 0, want, err_msg=f"b{b} h{h}")
                kept = o[b, h][want]
                np.testing.assert_allclose(kept, drop.scale / 128, rtol=2e-6)
        np.testing.assert_allclose(lse.cpu().numpy(), np.log(128.0), atol=1e-5)


@pytest.mark.parametrize("d", [64, 128])
def test_dkdv_keep_mask_bit_exact(d):
    B, Hq, Hkv, nb, p = 2, 4, 2, 4, 0.3
    N = 128 * nb
    f, bm = _perm(nb)
    finv = np.argsort(f)  # key tile kb is seen by query tile finv[kb]
    drop = oracle.Dropout(_p32(p), SEED, OFFSET)
    rng = np.random.default_rng(2)
    q = torch.zeros((B, Hq, N, d), dtype=torch.bfloat16, device="cuda")
    k = _t(rng.standard_normal((B, Hkv, N, d)), torch.bfloat16)
    v = _t(rng.standard_normal((B, Hkv, N, d)), torch.bfloat16)
    bmt = torch.from_numpy(bm).cuda()
    kw = dict(scale=0.125, block_mask=bmt, dropout_p=p, dropout_seed=SEED, dropout_offset=OFFSET)
    o, lse, _ = fa.fa_fwd(q, k, v, **kw)
    G = Hq // Hkv
    for half in range(128 // d):
        print(f"dK/dV keep mask d={d} half={half}", flush=True)
        do = _t(np.broadcast_to(_onehot(N, d, half), (B, Hq, N, d)), torch.bfloat16)
        _, _, dv, _ = fa.fa_bwd(q, k, v, o, lse, do, **kw)
        dv = dv.float().cpu().numpy()
        keys = np.arange(N)
        for b in range(B):
            for g in range(Hkv):
                # dV sums the group's query heads: count kept over the group.
                cnt = np.zeros((N, d))
                for h in range(g * G, (g + 1) * G):
                    rows = 128 * finv[keys // 128][:, None] + 64 * half + np.arange(d)[None, :]
                    for j in range(N):
                        cnt[j] += drop.keep(b * Hq + h, rows[j], [j])[:, 0]
                got = np.rint(dv[b, g] * 128 / drop.scale)
                np.testing.assert_array_equal(got, cnt, err_msg=f"b{b} g{g}")


@pytest.mark.parametrize("d", [64, 128])
def test_dq_keep_mask_bit_exact(d):
    B, Hq, Hkv, nb, p = 2, 4, 2, 4, 0.5
    N = 128 * nb
    f, bm = _perm(nb)
    drop = oracle.Dropout(_p32(p), SEED, OFFSET)
    q = torch.zeros((B, Hq, N, d), dtype=torch.bfloat16, device="cuda")
    v = torch.full((B, Hkv, N, d), 1.0 / d, dtype=torch.bfloat16, device="cuda")
    do = torch.ones((B, Hq, N, d), dtype=torch.bfloat16, device="cuda")
    bmt = torch.from_numpy(bm).cuda()
    scale = 0.125
    kw = dict(scale=scale, block_mask=bmt, dropout_p=p, dropout_seed=SEED, dropout_offset=OFFSET)
    for half in range(128 // d):
        print(f"dQ keep mask d={d} half={half}", flush=True)
        k = _t(np.broadcast_to(_onehot(N, d, half), (B, Hkv, N, d)), torch.bfloat16)
        o, lse, _ = fa.fa_fwd(q, k, v, o_dtype=torch.float32, **kw)
        dq, _, _, _ = fa.fa_bwd(q, k, v, o, lse, do, **kw)
        dq = dq.float().cpu().numpy()
        rows = np.arange(N)
        for b in range(B):
            for h in range(Hq):
                tile_keys = 128 * f[rows // 128][:, None] + np.arange(128)[None, :]
                keep_tile = np.stack([drop.keep(b * Hq + h, [i], tile_keys[i])[0] for i in rows])
                kcount = keep_tile.sum(axis=1)
                assert np.all((kcount > 0) & (kcount < 128))
                want = keep_tile[:, 64 * half:64 * half + d]
                np.testing.assert_array_equal(dq[b, h] > 0, want, err_msg=f"b{b} h{h}")
                exp = scale * drop.scale / 128 * (want - kcount[:, None] / 128)
                np.testing.assert_allclose(dq[b, h], exp, rtol=1e-2, atol=1e-6)


# (B, Hq, Hkv, N, d, causal, seqlens, block_mask, window, p)
CASES = [
    (1, 2, 2, 300, 64, False, None, None, None, 0.1),
    (2, 4, 2, 257, 128, True, "random", None, None, 0.5),
    (1, 2, 1, 520, 128, True, None, "random", None, 0.25),
    (2, 2, 2, 640, 64, False, None, None, (130, 60), 0.3),
    (1, 1, 1, 1, 64, False, None, None, None, 0.5),
    (2, 4, 4, 384, 128, False, [384, 130], "butterfly", None, 0.9),
    (1, 8, 2, 1024, 64, True, None, None, None, 0.2),
]


def _ids(c):
    B, Hq, Hkv, N, d, causal, sl, bm, win, p = c
    return (f"B{B}H{Hq}/{Hkv}N{N}d{d}{'c' if causal else ''}{'p' if sl is not None else ''}"
            f"{bm or ''}{'w' if win else ''}-p{p}")


@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_dropout_parity_with_oracle(case):
    B, Hq, Hkv, N, d, causal, sl, bm, win, p = case
    inp = draw_case(B, Hq, Hkv, N, d, "bf16", causal=causal, seqlens=sl, block_mask=bm,
                    seed=3 * N + d, window=win)
    print(f"dropout parity {_ids(case)}", flush=True)
    drop = oracle.Dropout(_p32(p), SEED + N, OFFSET + d)
    okw = dict(causal=causal, seqlens=inp.seqlens, block_mask=inp.block_mask, window=win,
               dropout=drop)
    q64, k64, v64 = inp.as_f64("q"), inp.as_f64("k"), inp.as_f64("v")
    o_ref, lse_ref = oracle.attention_forward(q64, k64, v64, inp.scale, **okw)
    dq_ref, dk_ref, dv_ref = oracle.attention_backward(q64, k64, v64, inp.as_f64("do"),
                                                       inp.scale, **okw)
    q, k, v, do = (dev(getattr(inp, n), "bf16") for n in ("q", "k", "v", "do"))
    slt = None if inp.seqlens is None else torch.from_numpy(inp.seqlens).cuda()
    bmt = None if inp.block_mask is None else torch.from_numpy(inp.block_mask).cuda()
    kw = dict(scale=inp.scale, causal=causal, seqlens_k=slt, block_mask=bmt, window=win,
              dropout_p=p, dropout_seed=SEED + N, dropout_offset=OFFSET + d)
    o, lse, _ = fa.fa_fwd(q, k, v, **kw)
    o32, lse32, _ = fa.fa_fwd(q, k, v, o_dtype=torch.float32, **kw)
    dq, dk, dv, _ = fa.fa_bwd(q, k, v, o, lse, do, **kw)
    torch.cuda.synchronize()
    check_o_dropped(host64(o), o_ref, drop, True, "bf16-O")
    check_o_dropped(host64(o32), o_ref, drop, False, "fp32-O")
    check_lse(host64(lse), lse_ref, TOL_BF16_LSE)
    check_grad(host64(dq), dq_ref, "dQ")
    check_grad(host64(dk), dk_ref, "dK")
    check_grad(host64(dv), dv_ref, "dV")
    # deterministic: the same seed and offset regenerate the same mask
    o2, _, _ = fa.fa_fwd(q, k, v, **kw)
    dq2, dk2, dv2, _ = fa.fa_bwd(q, k, v, o, lse, do, **kw)
    torch.cuda.synchronize()
    for a, b_ in ((o, o2), (dq, dq2), (dk, dk2), (dv, dv2)):
        assert torch.equal(a, b_)


def test_fp32_forward_dropout_parity():
    inp = draw_case(2, 2, 1, 300, 128, "fp32", causal=True, seqlens="random", seed=21)
    drop = oracle.Dropout(_p32(0.35), SEED, OFFSET)
    o_ref, lse_ref = oracle.attention_forward(inp.as_f64("q"), inp.as_f64("k"), inp.as_f64("v"),
                                              inp.scale, causal=True, seqlens=inp.seqlens,
                                              dropout=drop)
    q, k, v = (dev(getattr(inp, n), "fp32") for n in ("q", "k", "v"))
    slt = torch.from_numpy(inp.seqlens).cuda()
    o, lse, _ = fa.fa_fwd(q, k, v, scale=inp.scale, causal=True, seqlens_k=slt,
                          dropout_p=0.35, dropout_seed=SEED, dropout_offset=OFFSET)
    torch.cuda.synchronize()
    err = np.abs(host64(o) - o_ref).max()
    assert err <= 1e-5 * max(1.0, np.abs(o_ref).max()), err
    check_lse(host64(lse), lse_ref, 1e-5)


def test_streams_and_degenerate_probabilities():
    """Another seed or offset changes the result; a p whose threshold rounds
    to 65536 keeps everything and equals no dropout bit for bit."""
    inp = draw_case(1, 2, 2, 256, 64, "bf16", seed=5)
    q, k, v = (dev(getattr(inp, n), "bf16") for n in ("q", "k", "v"))
    base, _, _ = fa.fa_fwd(q, k, v, scale=inp.scale)
    tiny, _, _ = fa.fa_fwd(q, k, v, scale=inp.scale, dropout_p=1e-7, dropout_seed=3)
    a, _, _ = fa.fa_fwd(q, k, v, scale=inp.scale, dropout_p=0.5, dropout_seed=3)
    b, _, _ = fa.fa_fwd(q, k, v, scale=inp.scale, dropout_p=0.5, dropout_seed=4)
    c, _, _ = fa.fa_fwd(q, k, v, scale=inp.scale, dropout_p=0.5, dropout_seed=3,
                        dropout_offset=1)
    torch.cuda.synchronize()
    assert torch.equal(base, tiny)
    assert not torch.equal(a, b) and not torch.equal(a, c)
    with pytest.raises(fa.FAError):
        fa.fa_fwd(q, k, v, scale=inp.scale, dropout_p=1.0)


def test_full_size_headline_shape_with_dropout_sampled():
    """B64 H16 N1024 d64 with p = 0.1 in the launch configuration the
    benchmark times: sampled heads against the oracle (all rows of the head
    for O/LSE/dQ, a key sample for dK/dV)."""
    w = WORKLOADS[2]
    inp = draw(w, 2)
    p = 0.1
    q, k, v, do = (dev(getattr(inp, n), "bf16") for n in ("q", "k", "v", "do"))
    kw = dict(scale=inp.scale, dropout_p=p, dropout_seed=SEED, dropout_offset=OFFSET)
    print("full-size dropout B64 H16 N1024 d64", flush=True)
    o, lse, _ = fa.fa_fwd(q, k, v, **kw)
    dq, dk, dv, _ = fa.fa_bwd(q, k, v, o, lse, do, **kw)
    torch.cuda.synchronize()
    drop = oracle.Dropout(_p32(p), SEED, OFFSET)
    heads = [(0, 0), (37, 11), (63, 15)]
    k_rows = np.array([0, 1, 255, 256, 700, 1023])
    ref = oracle_heads(inp, heads, k_rows=k_rows, dropout=drop)
    for (b, h) in heads:
        r = ref[(b, h)]
        check_o_dropped(host64(o[b, h]), r["o"], drop, True, f"O b{b} h{h}")
        check_lse(host64(lse[b, h]), r["lse"], TOL_BF16_LSE)
        check_grad(host64(dq[b, h]), r["dq"], "dQ")
        g = h // (w.heads_q // w.heads_kv)
        kv = ref[(b, g, "kv")]
        check_grad(host64(dk[b, g][k_rows]), kv["dk"], "dK")
        check_grad(host64(dv[b, g][k_rows]), kv["dv"], "dV")
