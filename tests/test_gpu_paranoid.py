"""The debug build with extra barriers (libfa_paranoid.so: a workgroup
barrier before every refill of an LDS stage, and a full wait plus barrier
right after it) must give results bit-identical to the release build, which
overlaps each refill with the reads of the other stage (Report section 3.2:
K_j and V_j are staged tile by tile). A read that the release build let run
ahead of a refill it depends on, or a refill that overwrote a stage still
being read, would show here as a difference. The timeline build
(libfa_timeline.so), which only adds timestamp stores, is held to the same
bar on the paths that carry the stamps."""
import contextlib
import os

import numpy as np
import pytest
import torch

import exact_io_aware_29_amd as fa
from exact_io_aware_29_amd import _abi
from synth import draw_case
from tests.gpu_util import dev

pytestmark = pytest.mark.gpu


@contextlib.contextmanager
def _variant(path):
    """Route the binding's calls to another build for the duration."""
    saved = _abi.load()
    _abi._lib = _abi.load_variant(path)
    try:
        yield
    finally:
        _abi._lib = saved


def _paranoid():
    return _variant(_abi.PARANOID_LIB_PATH)


def _bits(t):
    return t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)


# (B, Hq, Hkv, N, d, causal, seqlens, block_mask, window, dropout_p)
CASES = [
    (2, 4, 2, 300, 128, True, "random", None, None, 0.0),     # causal pairs, padding
    (1, 2, 2, 257, 64, False, None, None, None, 0.0),          # lean one-block kernels
    (1, 2, 2, 640, 64, False, None, "random", None, 0.0),      # block-mask scan
    (1, 4, 2, 520, 128, True, None, None, (100, 0), 0.0),      # sliding window
    (2, 2, 1, 300, 64, True, [300, 77], None, None, 0.2),      # dropout
    (1, 2, 2, 700, 128, False, "random", "butterfly", None, 0.0),
    (1, 2, 2, 333, 128, False, "random", None, None, 0.0),    # lean one-block, d=128
    (1, 4, 2, 520, 64, True, None, None, None, 0.0),           # lean causal pairs, d=64
    (1, 2, 1, 8300, 128, True, "random", None, None, 0.0),    # long rows: 256-row dQ blocks
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"B{c[0]}H{c[1]}/{c[2]}N{c[3]}d{c[4]}"
                         f"{'c' if c[5] else ''}{'p' if c[6] is not None else ''}{c[7] or ''}"
                         f"{'w' if c[8] else ''}{'drop' if c[9] else ''}")
def test_paranoid_build_is_bit_identical(case):
    _compare_with(_abi.PARANOID_LIB_PATH, case)


# The timeline build's stamps sit in the 16x16x32 kernels: their paths.
TIMELINE_CASES = [CASES[0], CASES[3], CASES[6], CASES[7], CASES[8]]


@pytest.mark.parametrize("case", TIMELINE_CASES, ids=lambda c: f"B{c[0]}H{c[1]}/{c[2]}N{c[3]}d{c[4]}"
                         f"{'c' if c[5] else ''}{'w' if c[8] else ''}")
def test_timeline_build_is_bit_identical(case):
    """libfa_timeline.so only adds stores of timestamps: its results equal
    the release build's bit for bit."""
    _compare_with(_abi.TIMELINE_LIB_PATH, case)


def _compare_with(path, case):
    B, Hq, Hkv, N, d, causal, sl, bm, window, p = case
    print(f"{os.path.basename(path)} vs release {case}", flush=True)
    inp = draw_case(B, Hq, Hkv, N, d, "bf16", causal=causal, seqlens=sl, block_mask=bm,
                    seed=N + 3 * d, window=window)
    q, k, v, do = (dev(getattr(inp, n), "bf16") for n in ("q", "k", "v", "do"))
    slt = None if inp.seqlens is None else torch.from_numpy(inp.seqlens).cuda()
    bmt = None if inp.block_mask is None else torch.from_numpy(inp.block_mask).cuda()
    kw = dict(scale=inp.scale, causal=causal, seqlens_k=slt, block_mask=bmt, window=window,
              dropout_p=p, dropout_seed=0x5EED, dropout_offset=3)

    def run():
        o, lse, flog = fa.fa_fwd(q, k, v, tile_log=True, **kw)
        o32, lse32, _ = fa.fa_fwd(q, k, v, o_dtype=torch.float32, **kw)
        dq, dk, dv, blog = fa.fa_bwd(q, k, v, o, lse, do, tile_log=True, **kw)
        torch.cuda.synchronize()
        return [o, lse, flog, o32, lse32, dq, dk, dv, blog]

    rel = run()
    with _variant(path):
        par = run()
    names = ["O", "LSE", "fwd tiles", "O fp32", "LSE (fp32 O)", "dQ", "dK", "dV", "bwd tiles"]
    for name, a, b in zip(names, rel, par):
        assert torch.equal(_bits(a), _bits(b)), name


def test_paranoid_build_fp8_and_decode():
    B, Hq, Hkv, N, d = 2, 4, 2, 300, 128
    inp = draw_case(B, Hq, Hkv, N, d, "bf16", causal=True, seqlens=[211, 300], seed=19)
    q, k, v = (dev(getattr(inp, n), "bf16") for n in ("q", "k", "v"))
    sl = torch.from_numpy(inp.seqlens).cuda()
    q8, k8, v8 = (x.to(torch.float8_e4m3fn) for x in (q, k, v))
    qd = q[:, :, :1].contiguous()

    def run():
        o8, l8, _ = fa.fa_fwd(q8, k8, v8, scale=inp.scale, causal=True, seqlens_k=sl)
        od, ld = fa.fa_decode(qd, k, v, scale=inp.scale, seqlens_k=sl)
        torch.cuda.synchronize()
        return [o8, l8, od, ld]

    rel = run()
    with _paranoid():
        par = run()
    for name, a, b in zip(["O fp8", "LSE fp8", "O decode", "LSE decode"], rel, par):
        assert torch.equal(_bits(a), _bits(b)), name
