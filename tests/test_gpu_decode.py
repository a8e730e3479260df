"""GPU parity of decode attention (one query row per head against a key/
value cache, keys split across workgroups and merged) against the fp64
oracle: small cases spanning splits, GQA groups of more than 16 heads,
ragged and empty caches, and the full-size decode workload on sampled
heads."""
import numpy as np
import pytest
import torch

import exact_io_aware_29_amd as fa
import oracle
from synth import WORKLOADS, draw, draw_case
from tests.gpu_util import TOL_BF16_LSE, check_lse, check_o, dev, host64

pytestmark = pytest.mark.gpu

# (B, Hq, Hkv, N cache, d, cache lengths)
CASES = [
    (1, 1, 1, 1, 64, None),
    (2, 4, 2, 300, 64, "random"),
    (3, 8, 1, 1000, 128, [1000, 1, 0]),
    (1, 32, 1, 777, 128, None),
    (2, 16, 4, 5000, 128, "random"),
    (4, 8, 8, 40000, 64, None),
    (1, 20, 4, 2049, 128, [1987]),
]


def _ids(c):
    B, Hq, Hkv, N, d, sl = c
    return f"B{B}H{Hq}/{Hkv}N{N}d{d}{'p' if sl is not None else ''}"


def _decode_inputs(inp):
    """The last query row of each head of a drawn case is the decoded row."""
    q = np.ascontiguousarray(inp.q[:, :, -1:, :])
    return q


@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_decode_small(case):
    B, Hq, Hkv, N, d, sl = case
    inp = draw_case(B, Hq, Hkv, N, d, "bf16", seqlens=sl, seed=N + Hq, with_do=False)
    print(f"decode case {_ids(case)}", flush=True)
    qbits = _decode_inputs(inp)
    q, k, v = dev(qbits, "bf16"), dev(inp.k, "bf16"), dev(inp.v, "bf16")
    slt = None if inp.seqlens is None else torch.from_numpy(inp.seqlens).cuda()
    o, lse = fa.fa_decode(q, k, v, scale=inp.scale, seqlens_k=slt)
    o32, lse32 = fa.fa_decode(q, k, v, scale=inp.scale, seqlens_k=slt, o_dtype=torch.float32)
    torch.cuda.synchronize()
    q64 = inp.as_f64("q")[:, :, -1, :]
    o_ref, lse_ref = oracle.attention_decode(q64, inp.as_f64("k"), inp.as_f64("v"), inp.scale,
                                             seqlens=inp.seqlens)
    check_o(host64(o)[:, :, 0], o_ref, True, "decode O")
    check_o(host64(o32)[:, :, 0], o_ref, False, "decode O fp32")
    check_lse(host64(lse), lse_ref, TOL_BF16_LSE, "decode")
    check_lse(host64(lse32), lse_ref, TOL_BF16_LSE, "decode fp32-O")
    empty = lse_ref == -np.inf
    assert not host64(o)[:, :, 0][empty].any(), "an empty cache gives O = 0"


def test_decode_workload7_full_size():
    w = WORKLOADS[7]
    print(f"workload 7: {w.describe()}", flush=True)
    inp = draw(w, 7)
    q, k, v = dev(inp.q, "bf16"), dev(inp.k, "bf16"), dev(inp.v, "bf16")
    slt = torch.from_numpy(inp.seqlens).cuda()
    o, lse = fa.fa_decode(q, k, v, scale=inp.scale, seqlens_k=slt)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
    # oracle on sampled (batch, head) pairs: the shortest and longest caches
    bs = [int(np.argmin(inp.seqlens)), int(np.argmax(inp.seqlens)), 5]
    for b in bs:
        q64 = inp.as_f64("q", (slice(b, b + 1),))[:, :, 0, :]
        o_ref, lse_ref = oracle.attention_decode(q64, inp.as_f64("k", (slice(b, b + 1),)),
                                                 inp.as_f64("v", (slice(b, b + 1),)), inp.scale,
                                                 seqlens=inp.seqlens[b:b + 1])
        check_o(host64(o[b:b + 1])[:, :, 0], o_ref, True, f"decode b{b}")
        check_lse(host64(lse[b:b + 1]), lse_ref, TOL_BF16_LSE, f"decode b{b}")


def test_decode_cache_past_2_gib_per_head():
    """A cache whose K (and V) rows of one head span 2.3 GB, past every 31-bit
    byte offset and below the 4 GiB limit, with ragged lengths. Q = 0 makes
    every allowed probability equal, so O is the mean of V over the cached
    keys and LSE = ln(L): a closed form at any size (the mean is summed on
    the GPU in fp64, in chunks)."""
    B, Hq, Hkv, N, d = 2, 4, 1, 9_000_000, 128
    lens = [N - 7, N // 2 + 3]
    print(f"decode B{B} H{Hq}/{Hkv} N{N} d{d} lens {lens}", flush=True)
    g = torch.Generator(device="cuda").manual_seed(11)
    k = torch.randn((B, Hkv, N, d), generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    v = torch.randn((B, Hkv, N, d), generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    q = torch.zeros((B, Hq, 1, d), device="cuda", dtype=torch.bfloat16)
    slt = torch.tensor(lens, dtype=torch.int32, device="cuda")
    o32, lse32 = fa.fa_decode(q, k, v, scale=d ** -0.5, seqlens_k=slt, o_dtype=torch.float32)
    o, lse = fa.fa_decode(q, k, v, scale=d ** -0.5, seqlens_k=slt)
    torch.cuda.synchronize()
    for b, L in enumerate(lens):
        acc = torch.zeros(d, dtype=torch.float64, device="cuda")
        for r0 in range(0, L, 1 << 20):
            acc += v[b, 0, r0:min(L, r0 + (1 << 20))].to(torch.float64).sum(dim=0)
        mean = (acc / L).cpu().numpy()
        for h in range(Hq):
            err32 = np.abs(host64(o32[b, h, 0]) - mean).max()
            assert err32 <= 2e-5, f"b{b} h{h} fp32 O err {err32:.3g}"
            err = np.abs(host64(o[b, h, 0]) - mean)
            assert (err <= 1e-5 + 2.0 ** -9 * np.abs(mean)).all(), f"b{b} h{h} bf16 O err {err.max():.3g}"
            for name, l in (("fp32-O", lse32), ("bf16-O", lse)):
                e = abs(float(l[b, h]) - np.log(L))
                assert e <= 1e-5, f"b{b} h{h} {name} LSE err {e:.3g}"
    del k, v
