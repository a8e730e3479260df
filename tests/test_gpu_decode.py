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
