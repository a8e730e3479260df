"""GPU checks of the FP8 (e4m3) forward.

* Parity against the fp64 oracle of the decoded, descaled inputs under the
  per-element bound derived from the kernel's one rounding (P~ to e4m3):
  tests/fp8_bound.py. Every mask kind, both head dims, GQA, ragged lengths,
  non-unit descales; LSE at the bf16 bar; the tile-visit set equals the mask.
* Q = 0: every allowed score is 0, P~ = 1 exactly in e4m3, and O must be the
  mean of the allowed V rows to fp32 precision -- the V^T operand mapping
  with no quantisation slack.
* The two FP8 workload shapes at full size, sampled heads.
"""
import numpy as np
import pytest
import torch

import exact_io_aware_29_amd as fa
import oracle
import oracle.attention as OA
from synth import WORKLOADS, draw, draw_case
from tests.fp8_bound import fp8_o_bound
from tests.gpu_util import TOL_BF16_LSE, check_lse, decode_log, expected_tiles, host64

pytestmark = pytest.mark.gpu


def _dev8(codes):
    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).cuda()


def _run(inp, o_dtype=torch.bfloat16, tile_log=False):
    w = inp.workload
    q, k, v = _dev8(inp.q), _dev8(inp.k), _dev8(inp.v)
    sl = None if inp.seqlens is None else torch.from_numpy(inp.seqlens).cuda()
    bm = None if inp.block_mask is None else torch.from_numpy(inp.block_mask).cuda()
    return fa.fa_fwd(q, k, v, scale=inp.scale, causal=w.causal, seqlens_k=sl, block_mask=bm,
                     o_dtype=o_dtype, tile_log=tile_log, window=inp.window,
                     descale=inp.descale)


def _check_heads(inp, o, lse, heads, rows=None, what=""):
    """O of the selected (b, h) heads within the derived bound (plus the
    bf16 rounding of O when it is stored in bf16), LSE at the bf16 bar."""
    w = inp.workload
    G = w.heads_q // w.heads_kv
    o = host64(o)
    lse = host64(lse)
    worst = 0.0
    for (b, h) in heads:
        m = OA.mask_for(b, causal=w.causal, seqlens=inp.seqlens, block_mask=inp.block_mask,
                        window=inp.window)
        q = inp.as_f64("q", (b, h))
        k = inp.as_f64("k", (b, h // G))
        v = inp.as_f64("v", (b, h // G))
        r = np.arange(w.seqlen) if rows is None else np.asarray(rows)
        o_ref, lse_ref = oracle.head_forward(q, k, v, inp.scale, m, rows=r)
        p = OA.probabilities(q, k, inp.scale, m, rows=r)
        allowed = m.allowed(r, np.arange(w.seqlen))
        bound = fp8_o_bound(p, v, allowed) + 2.0 ** -9 * np.abs(o_ref) + 1e-5 * (1 + np.abs(o_ref))
        err = np.abs(o[b, h][r] - o_ref)
        bad = err > bound
        assert not bad.any(), (f"{what} b{b} h{h}: {int(bad.sum())} elements beyond the bound, "
                               f"worst err {err.max():.3g} vs bound {bound[np.unravel_index(np.argmax(err - bound), err.shape)]:.3g}")
        worst = max(worst, float((err / bound).max()))
        check_lse(lse[b, h][r], lse_ref, TOL_BF16_LSE, f"{what} b{b} h{h}")
    return worst


# (B, Hq, Hkv, N, d, causal, seqlens, block_mask, window, descale)
CASES = [
    (1, 1, 1, 1, 64, False, None, None, None, (1.0, 1.0, 1.0)),
    (1, 2, 2, 17, 64, False, None, None, None, (0.5, 0.25, 2.0)),
    (2, 2, 1, 127, 128, True, None, None, None, (1.0, 1.0, 1.0)),
    (1, 2, 2, 300, 64, True, "random", None, None, (0.0625, 0.0625, 0.0625)),
    (2, 4, 2, 257, 128, False, [0, 200], None, None, (0.125, 0.5, 0.25)),
    (1, 2, 1, 520, 128, True, None, "random", None, (1.0, 1.0, 1.0)),
    (1, 2, 2, 1024, 64, False, None, "butterfly", None, (0.25, 0.25, 1.0)),
    (2, 2, 2, 640, 64, False, None, None, (130, 60), (1.0, 0.5, 1.0)),
    (1, 4, 2, 700, 128, True, None, None, (200, 0), (0.0625, 0.0625, 0.0625)),
]


def _ids(c):
    B, Hq, Hkv, N, d, causal, sl, bm, win, ds = c
    return (f"B{B}H{Hq}/{Hkv}N{N}d{d}{'c' if causal else ''}{'p' if sl is not None else ''}"
            f"{bm or ''}{'w' if win else ''}-ds{ds[0]:g}/{ds[1]:g}/{ds[2]:g}")


@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_fp8_forward_within_derived_bound(case):
    B, Hq, Hkv, N, d, causal, sl, bm, win, ds = case
    inp = draw_case(B, Hq, Hkv, N, d, "fp8", causal=causal, seqlens=sl, block_mask=bm,
                    seed=5 * N + d, with_do=False, window=win, descale=ds)
    print(f"fp8 forward {_ids(case)}", flush=True)
    o, lse, log = _run(inp, tile_log=True)
    o32, lse32, _ = _run(inp, o_dtype=torch.float32)
    torch.cuda.synchronize()
    heads = [(b, h) for b in range(B) for h in range(Hq)]
    _check_heads(inp, o, lse, heads, what="bf16-O")
    _check_heads(inp, o32, lse32, heads, what="fp32-O")
    exp_tiles = expected_tiles(B, Hq, N, causal, inp.seqlens, inp.block_mask, win)
    assert np.array_equal(decode_log(log, B, Hq, N), exp_tiles), "forward tile set"
    # deterministic
    o2, _, _ = _run(inp)
    torch.cuda.synchronize()
    assert torch.equal(o, o2)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_fp8_zero_query_is_the_exact_mean_of_v(d, causal):
    """Q = 0: P~ = 1 for every allowed key (exact in e4m3), so O is the mean
    of the allowed V rows up to fp32 accumulation."""
    B, Hq, Hkv, N = 2, 4, 2, 333
    inp = draw_case(B, Hq, Hkv, N, d, "fp8", causal=causal, seqlens=[333, 150], seed=d,
                    with_do=False, descale=(1.0, 0.5, 0.25))
    inp.q[...] = 0
    o, lse, _ = _run(inp, o_dtype=torch.float32)
    torch.cuda.synchronize()
    o = host64(o)
    lse = host64(lse)
    G = Hq // Hkv
    for b in range(B):
        L = int(inp.seqlens[b])
        for h in range(Hq):
            v = inp.as_f64("v", (b, h // G))
            for i in (0, 1, 77, 149, 150, 332):
                n = min(i + 1, L) if causal else L
                want = v[:n].mean(axis=0)
                np.testing.assert_allclose(o[b, h, i], want, rtol=1e-5, atol=1e-6,
                                           err_msg=f"b{b} h{h} row{i}")
                assert abs(lse[b, h, i] - np.log(n)) < 1e-5


@pytest.mark.parametrize("wid", [10, 11])
def test_fp8_workloads_full_size_sampled(wid):
    w = WORKLOADS[wid]
    inp = draw(w, wid)
    print(f"fp8 workload {wid}: {w.describe()}", flush=True)
    o, lse, _ = _run(inp)
    torch.cuda.synchronize()
    heads = [(0, 0), (w.batch - 1, w.heads_q - 1), (w.batch // 2, 5)]
    rows = np.unique(np.concatenate([np.arange(0, w.seqlen, 97), [w.seqlen - 1]]))
    worst = _check_heads(inp, o, lse, heads, rows=rows, what=f"w{wid}")
    print(f"w{wid}: worst err / bound = {worst:.3f}", flush=True)
