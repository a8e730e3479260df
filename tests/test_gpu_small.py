"""GPU parity on small problems: every mask kind, both head dims, GQA, ragged
lengths, strided layouts, fp32 forward, tile-visit logs, determinism and the
Q = 0 closed forms. Each case is compared element by element with the full
fp64 oracle."""
import math

import numpy as np
import pytest
import torch

import exact_io_aware_29_amd as fa
import oracle
from synth import bf16_bits_to_f64, butterfly_block_mask, draw_case
from tests.gpu_util import (TOL_BF16_LSE, TOL_FP32_LSE, TOL_FP32_O, check_grad, check_lse,
                            check_o, decode_log, dev, expected_tiles, host64)

pytestmark = pytest.mark.gpu

# (B, Hq, Hkv, N, d, causal, seqlens, block_mask)
CASES = [
    (1, 1, 1, 1, 64, False, None, None),
    (1, 2, 2, 17, 64, False, None, None),
    (2, 2, 1, 127, 128, True, None, None),
    (1, 2, 2, 128, 64, True, None, None),
    (1, 1, 1, 129, 128, False, None, None),
    (2, 4, 2, 300, 64, False, "random", None),
    (2, 4, 1, 300, 128, True, "random", None),
    (3, 2, 2, 257, 64, True, [0, 1, 200], None),
    (1, 2, 2, 640, 64, False, None, "random"),
    (1, 2, 1, 520, 128, True, None, "random"),
    (1, 2, 2, 1024, 64, False, None, "butterfly"),
    (2, 4, 4, 384, 128, True, [384, 130], "butterfly"),
    (1, 8, 2, 256, 128, False, None, None),
    (1, 2, 1, 8300, 128, True, "random", None),   # long rows: the 256-row dQ blocks, ragged
    (1, 1, 1, 8200, 128, False, None, None),
]

# Sliding-window (local) attention: (case as above, (left, right) band).
WINDOW_CASES = [
    ((2, 2, 2, 300, 64, False, None, None), (37, 5)),
    ((1, 4, 2, 520, 128, True, None, None), (100, 0)),
    ((2, 2, 1, 700, 128, True, "random", None), (200, 0)),
    ((1, 2, 2, 640, 64, False, None, "random"), (130, 60)),
    ((1, 2, 2, 257, 64, True, None, None), (0, 0)),
    ((2, 4, 4, 384, 128, False, [384, 130], None), (0, 3)),
    ((1, 2, 1, 8300, 128, True, None, None), (700, 0)),    # long rows: 256-row dQ blocks
]


def _ids(c):
    B, Hq, Hkv, N, d, causal, sl, bm = c
    return f"B{B}H{Hq}/{Hkv}N{N}d{d}{'c' if causal else ''}{'p' if sl is not None else ''}{bm or ''}"


def _run(inp, o_dtype=None, tile_log=True):
    w = inp.workload
    q, k, v = dev(inp.q, w.dtype), dev(inp.k, w.dtype), dev(inp.v, w.dtype)
    sl = None if inp.seqlens is None else torch.from_numpy(inp.seqlens).cuda()
    bm = None if inp.block_mask is None else torch.from_numpy(inp.block_mask).cuda()
    o, lse, log = fa.fa_fwd(q, k, v, scale=inp.scale, causal=w.causal, seqlens_k=sl,
                            block_mask=bm, o_dtype=o_dtype, tile_log=tile_log, window=inp.window)
    return (q, k, v, sl, bm), o, lse, log


def _oracle_full(inp, backward=True):
    w = inp.workload
    kw = dict(causal=w.causal, seqlens=inp.seqlens, block_mask=inp.block_mask,
              window=inp.window)
    q, k, v = inp.as_f64("q"), inp.as_f64("k"), inp.as_f64("v")
    o, lse = oracle.attention_forward(q, k, v, inp.scale, **kw)
    if not backward:
        return o, lse, None
    grads = oracle.attention_backward(q, k, v, inp.as_f64("do"), inp.scale, **kw)
    return o, lse, grads


@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_small_fwd_bwd_bf16(case):
    _check_bf16(case, None)


@pytest.mark.parametrize("case,window", WINDOW_CASES,
                         ids=[f"{_ids(c)}w{w[0]}-{w[1]}" for c, w in WINDOW_CASES])
def test_small_sliding_window_bf16(case, window):
    _check_bf16(case, window)


def _check_bf16(case, window):
    B, Hq, Hkv, N, d, causal, sl, bm = case
    inp = draw_case(B, Hq, Hkv, N, d, "bf16", causal=causal, seqlens=sl, block_mask=bm,
                    seed=N + d + Hq, window=window)
    print(f"case {_ids(case)} window {window}", flush=True)
    o_ref, lse_ref, (dq_ref, dk_ref, dv_ref) = _oracle_full(inp)
    (q, k, v, slt, bmt), o, lse, log = _run(inp)
    torch.cuda.synchronize()
    check_o(host64(o), o_ref, True, "bf16-O")
    check_lse(host64(lse), lse_ref, TOL_BF16_LSE)
    exp_tiles = expected_tiles(B, Hq, N, causal, inp.seqlens, inp.block_mask, window)
    assert np.array_equal(decode_log(log, B, Hq, N), exp_tiles), "forward tile set"

    o32, lse32, _ = _run(inp, o_dtype=torch.float32, tile_log=False)[1:]
    torch.cuda.synchronize()
    check_o(host64(o32), o_ref, False, "fp32-O")

    do = dev(inp.do, "bf16")
    dq, dk, dv, blog = fa.fa_bwd(q, k, v, o, lse, do, scale=inp.scale, causal=causal,
                                 seqlens_k=slt, block_mask=bmt, tile_log=True, window=window)
    torch.cuda.synchronize()
    check_grad(host64(dq), dq_ref, "dQ")
    check_grad(host64(dk), dk_ref, "dK")
    check_grad(host64(dv), dv_ref, "dV")
    half = blog.numel() // 2
    assert np.array_equal(decode_log(blog[:half], B, Hq, N), exp_tiles), "dK/dV tile set"
    assert np.array_equal(decode_log(blog[half:], B, Hq, N), exp_tiles), "dQ tile set"

    # the backward also accepts an fp32 O
    dq2, dk2, dv2, _ = fa.fa_bwd(q, k, v, o32, lse32, do, scale=inp.scale, causal=causal,
                                 seqlens_k=slt, block_mask=bmt, window=window)
    torch.cuda.synchronize()
    check_grad(host64(dq2), dq_ref, "dQ(fp32 O)")
    check_grad(host64(dk2), dk_ref, "dK(fp32 O)")
    check_grad(host64(dv2), dv_ref, "dV(fp32 O)")


FP32_CASES = [
    (1, 1, 1, 1, 64, False, None, None),
    (1, 1, 1, 128, 64, False, None, None),
    (1, 2, 1, 129, 128, True, None, None),
    (2, 2, 2, 300, 64, True, "random", None),
    (1, 2, 2, 384, 128, False, None, "random"),
]


@pytest.mark.parametrize("case", FP32_CASES, ids=_ids)
def test_small_fwd_fp32(case):
    _check_fp32(case, None)


@pytest.mark.parametrize("case,window", [((1, 2, 1, 300, 128, True, None, None), (50, 0)),
                                         ((1, 1, 1, 200, 64, False, "random", None), (7, 90))],
                         ids=["causal-w50", "w7-90pad"])
def test_small_sliding_window_fp32(case, window):
    _check_fp32(case, window)


def _check_fp32(case, window):
    B, Hq, Hkv, N, d, causal, sl, bm = case
    inp = draw_case(B, Hq, Hkv, N, d, "fp32", causal=causal, seqlens=sl, block_mask=bm,
                    seed=3 * N + d, with_do=False, window=window)
    print(f"case {_ids(case)} window {window}", flush=True)
    o_ref, lse_ref, _ = _oracle_full(inp, backward=False)
    _, o, lse, log = _run(inp)
    torch.cuda.synchronize()
    err = np.abs(host64(o) - o_ref).max()
    assert err <= TOL_FP32_O, f"fp32 O max abs err {err:.3g}"
    check_lse(host64(lse), lse_ref, TOL_FP32_LSE)
    assert np.array_equal(decode_log(log, B, Hq, N),
                          expected_tiles(B, Hq, N, causal, inp.seqlens, inp.block_mask, window))


ISOLATED_BWD_CASES = [
    (2, 4, 2, 300, 64, False, "random", None),
    (3, 2, 2, 257, 64, True, [0, 1, 200], None),
    (1, 2, 1, 520, 128, True, None, "random"),
    (2, 4, 4, 384, 128, True, [384, 130], "butterfly"),
]


@pytest.mark.parametrize("case", ISOLATED_BWD_CASES, ids=_ids)
def test_backward_on_the_oracle_forward(case):
    """The backward alone: fed the oracle's O (fp32) and LSE instead of the
    GPU forward's, so its error is measured apart from the forward's. Empty
    rows arrive with LSE = -inf, as the forward would store them."""
    B, Hq, Hkv, N, d, causal, sl, bm = case
    inp = draw_case(B, Hq, Hkv, N, d, "bf16", causal=causal, seqlens=sl, block_mask=bm,
                    seed=7 * N + d)
    print(f"isolated backward {_ids(case)}", flush=True)
    o_ref, lse_ref, (dq_ref, dk_ref, dv_ref) = _oracle_full(inp)
    q, k, v = dev(inp.q, "bf16"), dev(inp.k, "bf16"), dev(inp.v, "bf16")
    do = dev(inp.do, "bf16")
    o = torch.from_numpy(o_ref.astype(np.float32)).cuda()
    lse = torch.from_numpy(lse_ref.astype(np.float32)).cuda()
    slt = None if inp.seqlens is None else torch.from_numpy(inp.seqlens).cuda()
    bmt = None if inp.block_mask is None else torch.from_numpy(inp.block_mask).cuda()
    dq, dk, dv, _ = fa.fa_bwd(q, k, v, o, lse, do, scale=inp.scale, causal=causal,
                              seqlens_k=slt, block_mask=bmt)
    torch.cuda.synchronize()
    for name, g, ref in (("dQ", dq, dq_ref), ("dK", dk, dk_ref), ("dV", dv, dv_ref)):
        r = check_grad(host64(g), ref, name, _ids(case))
        print(f"  {name} relF {r:.2e}", flush=True)


def test_strided_bshd_layout():
    """[B, N, H, d] storage viewed as [B, H, N, d]: strides, not copies."""
    B, H, N, d = 2, 3, 200, 64
    inp = draw_case(B, H, H, N, d, "bf16", causal=True, seed=77)
    o_ref, lse_ref, (dq_ref, dk_ref, dv_ref) = _oracle_full(inp)

    def bshd(x):
        t = dev(np.ascontiguousarray(np.transpose(x, (0, 2, 1, 3))), "bf16")
        return t.permute(0, 2, 1, 3)

    q, k, v, do = bshd(inp.q), bshd(inp.k), bshd(inp.v), bshd(inp.do)
    assert not q.is_contiguous()
    out = torch.empty((B, N, H, d), dtype=torch.bfloat16, device="cuda").permute(0, 2, 1, 3)
    o, lse, _ = fa.fa_fwd(q, k, v, scale=inp.scale, causal=True, out=out)
    dq = torch.empty((B, N, H, d), dtype=torch.bfloat16, device="cuda").permute(0, 2, 1, 3)
    dq, dk, dv, _ = fa.fa_bwd(q, k, v, o, lse, do, scale=inp.scale, causal=True, dq=dq)
    torch.cuda.synchronize()
    check_o(host64(o), o_ref, True)
    check_lse(host64(lse), lse_ref, TOL_BF16_LSE)
    check_grad(host64(dq), dq_ref, "dQ")
    check_grad(host64(dk), dk_ref, "dK")
    check_grad(host64(dv), dv_ref, "dV")


def test_rows_spaced_past_2_gib():
    """Q, K, V and dO rows 4 MiB apart: one head's 600 rows span 2.5 GB, so
    every staged byte offset past row ~512 is beyond 2^31 (and below the
    4 GiB limit). The strided views hold the same values as the dense case,
    whose oracle is cheap."""
    B, Hq, Hkv, N, d = 1, 2, 1, 600, 64
    S = (1 << 21) + 64  # row stride in elements (4 MiB + 128 bytes)
    inp = draw_case(B, Hq, Hkv, N, d, "bf16", causal=True, seed=29)
    print(f"rows {S * 2} bytes apart, span {((N - 1) * S + d) * 2} bytes per head", flush=True)
    o_ref, lse_ref, (dq_ref, dk_ref, dv_ref) = _oracle_full(inp)

    def spread(x, H):
        big = torch.zeros(B * H * N * S, dtype=torch.bfloat16, device="cuda")
        view = big.as_strided((B, H, N, d), (H * N * S, N * S, S, 1))
        view.copy_(dev(x, "bf16"))
        return view

    q, k, v, do = spread(inp.q, Hq), spread(inp.k, Hkv), spread(inp.v, Hkv), spread(inp.do, Hq)
    o, lse, _ = fa.fa_fwd(q, k, v, scale=inp.scale, causal=True)
    dq, dk, dv, _ = fa.fa_bwd(q, k, v, o, lse, do, scale=inp.scale, causal=True)
    torch.cuda.synchronize()
    check_o(host64(o), o_ref, True)
    check_lse(host64(lse), lse_ref, TOL_BF16_LSE)
    check_grad(host64(dq), dq_ref, "dQ")
    check_grad(host64(dk), dk_ref, "dK")
    check_grad(host64(dv), dv_ref, "dV")
    del q, k, v, do


def test_deterministic_bitwise():
    inp = draw_case(2, 4, 2, 700, 128, "bf16", causal=True, seqlens="random", seed=5)
    (q, k, v, sl, bm), o1, l1, _ = _run(inp, tile_log=False)
    _, o2, l2, _ = _run(inp, tile_log=False)
    do = dev(inp.do, "bf16")
    g1 = fa.fa_bwd(q, k, v, o1, l1, do, scale=inp.scale, causal=True, seqlens_k=sl)[:3]
    g2 = fa.fa_bwd(q, k, v, o1, l1, do, scale=inp.scale, causal=True, seqlens_k=sl)[:3]
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)
    for a, b in zip(g1, g2):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("kind", ["plain", "causal", "padding", "butterfly", "gqa-causal-pad"])
def test_zero_query_closed_form_on_gpu(kind):
    """Q = 0 makes every allowed score 0: LSE_i = ln(count_i) and O_i is the mean
    of V over the allowed keys. Checks the masks and the GQA head mapping."""
    B, Hq, Hkv, N, d = 2, 4, 4, 1024, 64
    causal, sl, bm = False, None, None
    if kind == "causal":
        causal = True
    elif kind == "padding":
        sl = [1000, 3]
    elif kind == "butterfly":
        bm = butterfly_block_mask(8)
    elif kind == "gqa-causal-pad":
        Hkv, causal, sl, d = 1, True, [513, 1024], 128
    inp = draw_case(B, Hq, Hkv, N, d, "bf16", causal=causal, seqlens=sl, block_mask=bm, seed=9)
    inp.q[:] = 0
    _, o, lse, _ = _run(inp, o_dtype=torch.float32, tile_log=False)
    torch.cuda.synchronize()
    o, lse = host64(o), host64(lse)
    G = Hq // Hkv
    for b in range(B):
        L = N if sl is None else sl[b]
        for h in range(Hq):
            v = bf16_bits_to_f64(inp.v[b, h // G])
            i = np.arange(N)
            cnt = np.full(N, L)
            if causal:
                cnt = np.minimum(i + 1, L)
            if bm is not None:
                cnt = bm.sum(axis=1)[i // 128] * 128
            np.testing.assert_allclose(lse[b, h], np.log(cnt), atol=1e-5)
            if causal or sl is not None:
                csum = np.cumsum(v, axis=0)
                last = np.minimum(i, L - 1) if causal else np.full(N, L - 1)
                mean = csum[last] / cnt[:, None]
            elif bm is not None:
                blk = v.reshape(N // 128, 128, d).sum(axis=1)
                mean = (bm.astype(float) @ blk)[i // 128] / cnt[:, None]
            else:
                mean = np.tile(v.mean(axis=0), (N, 1))
            np.testing.assert_allclose(o[b, h], mean, atol=1e-4)


def test_fully_masked_rows_give_zero_and_neg_inf():
    """Block-mask rows with no present block: O = 0, LSE = -inf, and no
    gradient flows from them."""
    N = 384
    bm = np.array([[0, 0, 0], [1, 1, 0], [0, 1, 1]], dtype=np.uint8)
    inp = draw_case(1, 2, 2, N, 64, "bf16", block_mask=bm, seed=21)
    o_ref, lse_ref, (dq_ref, dk_ref, dv_ref) = _oracle_full(inp)
    (q, k, v, sl, bmt), o, lse, _ = _run(inp, tile_log=False)
    dq, dk, dv, _ = fa.fa_bwd(q, k, v, o, lse, dev(inp.do, "bf16"), scale=inp.scale,
                              block_mask=bmt)
    torch.cuda.synchronize()
    assert torch.all(o[:, :, :128] == 0)
    assert torch.all(torch.isneginf(lse[:, :, :128]))
    assert torch.all(dq[:, :, :128] == 0)
    check_o(host64(o), o_ref, True)
    check_grad(host64(dk), dk_ref, "dK")
    check_grad(host64(dv), dv_ref, "dV")


def test_invalid_arguments_raise_before_launch():
    q = torch.zeros((1, 2, 64, 96), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(fa.FAError, match="head_dim"):
        fa.fa_fwd(q, q, q)
    q = torch.zeros((1, 3, 64, 64), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((1, 2, 64, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(fa.FAError, match="multiple"):
        fa.fa_fwd(q, k, k)
    with pytest.raises(fa.FAError, match="scale"):
        fa.fa_fwd(q, q, q, scale=-1.0)
    x = torch.zeros((1, 1, 64, 64), dtype=torch.float32, device="cuda")
    o, lse, _ = fa.fa_fwd(x, x, x)
    with pytest.raises(fa.FAError, match="bf16"):
        fa.fa_bwd(x, x, x, o, lse, x)
