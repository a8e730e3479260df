"""fa_bwd_noalloc through the C ABI: the backward with the library's fixed
device array as workspace must give exactly fa_bwd's results (same kernels,
same inputs), on two calls in a row, the second smaller than the first (the
array keeps the first call's row vectors, which the second must not use)."""
import ctypes

import numpy as np
import pytest
import torch

import exact_io_aware_29_amd as fa
from exact_io_aware_29_amd import _abi
from synth import draw_case
from tests.gpu_util import dev

pytestmark = pytest.mark.gpu


def _strides(t):
    return _abi.Strides(t.stride(0), t.stride(1), t.stride(2))


def _ptr(t):
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _noalloc_via_abi(inp, q, k, v, o, lse, do, sl, causal, log_words):
    w = inp.workload
    p = fa.make_params(batch=w.batch, heads_q=w.heads_q, heads_kv=w.heads_kv, seqlen=w.seqlen,
                       head_dim=w.head_dim, scale=inp.scale, causal=causal,
                       seqlens_k=0 if sl is None else sl.data_ptr(), o_dtype=_abi.FA_BF16)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    log = torch.zeros(2 * log_words, dtype=torch.int32, device="cuda")
    lib = fa.library()
    st = lib.fa_bwd_noalloc(ctypes.byref(p), _ptr(q), _strides(q), _ptr(k), _strides(k), _ptr(v),
                            _strides(v), _ptr(o), _strides(o), _ptr(do), _strides(do), _ptr(lse),
                            _ptr(dq), _strides(dq), _ptr(dk), _strides(dk), _ptr(dv),
                            _strides(dv), _ptr(log), None,
                            ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, (st, lib.fa_last_error_detail().decode())
    return dq, dk, dv, log


def _case(B, Hq, Hkv, N, d, causal, seqlens, seed):
    inp = draw_case(B, Hq, Hkv, N, d, "bf16", causal=causal, seqlens=seqlens, seed=seed)
    print(f"noalloc B{B} H{Hq}/{Hkv} N{N} d{d} causal={causal}", flush=True)
    q, k, v, do = (dev(getattr(inp, n), "bf16") for n in ("q", "k", "v", "do"))
    sl = None if inp.seqlens is None else torch.from_numpy(inp.seqlens).cuda()
    o, lse, _ = fa.fa_fwd(q, k, v, scale=inp.scale, causal=causal, seqlens_k=sl)
    ref = fa.fa_bwd(q, k, v, o, lse, do, scale=inp.scale, causal=causal, seqlens_k=sl,
                    tile_log=True)
    got = _noalloc_via_abi(inp, q, k, v, o, lse, do, sl, causal, ref[3].numel() // 2)
    torch.cuda.synchronize()
    for name, a, b in zip(("dQ", "dK", "dV", "tile log"), ref, got):
        assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                           b.view(torch.int16) if b.dtype == torch.bfloat16 else b), name
    assert all(torch.isfinite(g.float()).all() for g in got[:3])


def test_noalloc_matches_fa_bwd_on_two_calls_in_a_row():
    # the first call fills the array with 2 * 3 * 8 * 1000 row values ...
    _case(3, 8, 2, 1000, 128, True, "random", 11)
    # ... the second, smaller one must write and read only its own
    _case(1, 2, 1, 300, 64, False, [211], 12)


def test_noalloc_rejects_a_problem_beyond_its_array():
    rows = _abi.FA_NOALLOC_WORKSPACE_BYTES // 8 + 1  # batch * heads * seqlen one row too many
    q = torch.zeros((1, 1, 64, 64), dtype=torch.bfloat16, device="cuda")
    # shapes are not touched: validation fails before any launch
    p = fa.make_params(batch=1, heads_q=1, heads_kv=1, seqlen=rows, head_dim=64)
    s = _abi.Strides(rows * 64, rows * 64, 64)
    lib = fa.library()
    x = _ptr(q)
    st = lib.fa_bwd_noalloc(ctypes.byref(p), x, s, x, s, x, s, x, s, x, s, x, x, s, x, s, x, s,
                            None, None, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == _abi.FA_ERR_WORKSPACE, (st, lib.fa_last_error_detail().decode())
