"""Key rows at or past a batch entry's valid length, and memory past the
last row of a head, are never read: filling them with NaN and infinities
must leave every output bit for bit as it is with finite values there (the
keys are masked, so they must contribute exactly nothing: Report section
3.2, masking inside the fused kernel). The finite-padding results are
themselves checked against the oracle by the parity suites."""
import numpy as np
import pytest
import torch

import exact_io_aware_29_amd as fa
import oracle
from synth import draw_case
from tests.gpu_util import check_grad, check_lse, check_o, dev, host64, TOL_BF16_LSE

pytestmark = pytest.mark.gpu

BAD = (float("nan"), float("inf"), float("-inf"))


def _embed(x: torch.Tensor, fill: float, tail_rows: int = 256) -> torch.Tensor:
    """x [B, H, N, d] copied into storage whose remaining elements (the
    `tail_rows` rows after the last head) hold `fill`; a view of the same
    shape and strides as a contiguous tensor."""
    B, H, N, d = x.shape
    store = torch.full(((B * H * N + tail_rows) * d,), fill, dtype=x.dtype, device=x.device)
    view = store[: B * H * N * d].view(B, H, N, d)
    view.copy_(x)
    return view


def _poison_keys(x: torch.Tensor, seqlens, n_bad: int) -> torch.Tensor:
    """Key rows at or past seqlens[b] set to NaN / +inf / -inf in turn."""
    y = x.clone()
    for b, L in enumerate(seqlens):
        for r in range(n_bad):
            y[b, :, int(L) + r::n_bad, :] = BAD[r]
    return y


@pytest.mark.parametrize("d,causal,N", [(64, False, 300), (128, True, 300), (64, True, 1000),
                                        (128, False, 129)])
def test_padded_keys_and_tail_memory_hold_nan(d, causal, N):
    B, Hq, Hkv = 3, 4, 2
    seqlens = [N, (N * 2) // 3 + 1, 1]
    inp = draw_case(B, Hq, Hkv, N, d, "bf16", causal=causal, seqlens=seqlens, seed=N + d)
    print(f"nan padding d={d} causal={causal} N={N}", flush=True)
    sl = torch.tensor(seqlens, dtype=torch.int32, device="cuda")
    q, k, v, do = (dev(getattr(inp, n), "bf16") for n in ("q", "k", "v", "do"))

    def run(q, k, v, do):
        o, lse, _ = fa.fa_fwd(q, k, v, scale=inp.scale, causal=causal, seqlens_k=sl)
        g = fa.fa_bwd(q, k, v, o, lse, do, scale=inp.scale, causal=causal, seqlens_k=sl)[:3]
        o32, lse32, _ = fa.fa_fwd(q, k, v, scale=inp.scale, causal=causal, seqlens_k=sl,
                                  o_dtype=torch.float32)
        torch.cuda.synchronize()
        return [o, lse, *g, o32, lse32]

    ref = run(q, k, v, do)
    kb = _embed(_poison_keys(k, seqlens, 3), float("nan"))
    vb = _embed(_poison_keys(v, seqlens, 3), float("inf"))
    qb, dob = _embed(q, float("nan")), _embed(do, float("-inf"))
    got = run(qb, kb, vb, dob)
    names = ["O", "LSE", "dQ", "dK", "dV", "O(fp32)", "LSE(fp32 O)"]
    for name, a, b in zip(names, ref, got):
        assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                           b.view(torch.int16) if b.dtype == torch.bfloat16 else b), name
    # padded keys get exactly zero gradients
    dk, dv = got[3], got[4]
    for b, L in enumerate(seqlens):
        assert torch.all(dk[b, :, L:] == 0) and torch.all(dv[b, :, L:] == 0)
    # and the finite run agrees with the oracle
    kw = dict(causal=causal, seqlens=inp.seqlens)
    qq, kk, vv = inp.as_f64("q"), inp.as_f64("k"), inp.as_f64("v")
    o_ref, lse_ref = oracle.attention_forward(qq, kk, vv, inp.scale, **kw)
    dq_ref, dk_ref, dv_ref = oracle.attention_backward(qq, kk, vv, inp.as_f64("do"), inp.scale,
                                                       **kw)
    check_o(host64(got[0]), o_ref, True)
    check_lse(host64(got[1]), lse_ref, TOL_BF16_LSE)
    check_grad(host64(got[2]), dq_ref, "dQ")
    check_grad(host64(got[3]), dk_ref, "dK")
    check_grad(host64(got[4]), dv_ref, "dV")


def test_fp8_forward_ignores_nan_padding():
    B, Hq, Hkv, N, d = 2, 4, 4, 300, 128
    seqlens = [211, 300]
    inp = draw_case(B, Hq, Hkv, N, d, "bf16", causal=True, seqlens=seqlens, seed=41)
    sl = torch.tensor(seqlens, dtype=torch.int32, device="cuda")
    q, k, v = (dev(getattr(inp, n), "bf16").to(torch.float8_e4m3fn) for n in ("q", "k", "v"))
    o1, l1, _ = fa.fa_fwd(q, k, v, scale=inp.scale, causal=True, seqlens_k=sl)

    def poison(x):
        # e4m3 (E4M3FN) code 0x7F is NaN; the bytes are written as uint8
        y = x.view(torch.uint8).clone()
        for b, L in enumerate(seqlens):
            y[b, :, L:] = 0x7F
        store = torch.full(((B * Hq * N + 256) * d,), 0x7F, dtype=torch.uint8, device="cuda")
        view = store[: B * Hq * N * d].view(B, Hq, N, d)
        view.copy_(y)
        return view.view(torch.float8_e4m3fn)

    o2, l2, _ = fa.fa_fwd(q, poison(k), poison(v), scale=inp.scale, causal=True, seqlens_k=sl)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)


def test_decode_ignores_nan_past_the_cache_length():
    B, Hq, Hkv, N, d = 3, 8, 2, 1000, 128
    seqlens = [1000, 517, 64]
    inp = draw_case(B, Hkv, Hkv, N, d, "bf16", seed=43, with_do=False)
    k, v = dev(inp.k, "bf16"), dev(inp.v, "bf16")
    q = torch.randn((B, Hq, 1, d), generator=torch.Generator().manual_seed(5)).to(
        torch.bfloat16).cuda()
    sl = torch.tensor(seqlens, dtype=torch.int32, device="cuda")
    o1, l1 = fa.fa_decode(q, k, v, seqlens_k=sl)
    kb = _embed(_poison_keys(k, seqlens, 3), float("nan"))
    vb = _embed(_poison_keys(v, seqlens, 3), float("nan"))
    o2, l2 = fa.fa_decode(q, kb, vb, seqlens_k=sl)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)


def test_overlapping_rows_raise():
    """A dO expanded from one row (row stride 0) is rejected before launch:
    rows past N would otherwise read real rows where zeros are meant."""
    inp = draw_case(1, 2, 2, 300, 64, "bf16", seed=3)
    q, k, v = (dev(getattr(inp, n), "bf16") for n in ("q", "k", "v"))
    o, lse, _ = fa.fa_fwd(q, k, v, scale=inp.scale)
    do = torch.ones((1, 1, 1, 64), dtype=torch.bfloat16, device="cuda").expand(1, 2, 300, 64)
    with pytest.raises(fa.FAError, match="row stride"):
        fa.fa_bwd(q, k, v, o, lse, do, scale=inp.scale)
    with pytest.raises(fa.FAError, match="row stride"):
        fa.fa_fwd(q, do, v, scale=inp.scale)
