"""The C-ABI library on a machine without a GPU: it loads, exports every
function include/fa.h declares, and rejects invalid calls on the host before
any HIP call (fake, never dereferenced pointer values are used)."""
import ctypes
import math
import os
import re

import pytest

import torch

import exact_io_aware_29_amd as fa
from exact_io_aware_29_amd import _abi

# Every call below must be rejected by host-side validation; the pointer
# values are fake. Where a GPU is visible these host checks are left to the
# GPU suite, which exercises validation with real device buffers.
no_gpu_only = pytest.mark.skipif(torch.cuda.device_count() > 0,
                                 reason="fake-pointer ABI checks run on GPU-less hosts only")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(?:int|size_t|const char\*)\s+(fa_\w+)\s*\(", text)))


def exported_symbols():
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", _abi.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    return sorted({l.split()[-1] for l in out.splitlines() if " T " in l and "fa_" in l})


def test_library_exports_every_declared_function():
    declared = header_functions()
    assert declared == sorted(_abi.SIGNATURES), "binding signatures out of date with fa.h"
    exported = [s for s in exported_symbols() if s.startswith("fa_")]
    assert exported == declared
    lib = fa.library()
    for name in declared:
        assert hasattr(lib, name)


def test_status_codes_match_header():
    text = open(HEADER).read()
    codes = dict((n, int(v)) for n, v in re.findall(r"(FA_\w+)\s*=\s*(-?\d+)", text))
    for name in ("FA_OK", "FA_ERR_NULL", "FA_ERR_SHAPE", "FA_ERR_DTYPE", "FA_ERR_HEADDIM",
                 "FA_ERR_GQA", "FA_ERR_STRIDE", "FA_ERR_ALIGN", "FA_ERR_WORKSPACE",
                 "FA_ERR_HIP", "FA_ERR_MASK", "FA_ERR_SCALE", "FA_ERR_DROPOUT", "FA_BF16",
                 "FA_FP32", "FA_FP8_E4M3"):
        assert codes[name] == getattr(_abi, name), name
    msgs = {fa.fa_strerror(c) for c in _abi.STATUS_CODES}
    assert len(msgs) == len(_abi.STATUS_CODES)
    assert fa.fa_strerror(12345) == "unknown status"


def _params(**kw):
    base = dict(batch=2, heads_q=4, heads_kv=2, seqlen=300, head_dim=64)
    base.update(kw)
    return fa.make_params(**base)


def _strides(p, heads=None, eb=2, d=None):
    d = d or p.head_dim
    h = heads or p.heads_q
    return _abi.Strides(h * p.seqlen * d, p.seqlen * d, d)


P16, P32, P48, P64, P80 = (ctypes.c_void_p(x) for x in (0x1000, 0x2000, 0x3000, 0x4000, 0x5000))


def _fwd(p, q=P16, k=P32, v=P48, o=P64, lse=P80, sq=None, sk=None, so=None, log=None):
    lib = fa.library()
    sq = sq or _strides(p)
    sk = sk or _strides(p, p.heads_kv)
    so = so or _strides(p)
    st = lib.fa_fwd(ctypes.byref(p), q, sq, k, sk, v, sk, o, so, lse, log, None)
    return st, lib.fa_last_error_detail().decode()


@no_gpu_only
@pytest.mark.parametrize("mut,code", [
    (dict(head_dim=96), _abi.FA_ERR_HEADDIM),
    (dict(head_dim=256), _abi.FA_ERR_HEADDIM),
    (dict(heads_q=3), _abi.FA_ERR_GQA),
    (dict(batch=0), _abi.FA_ERR_SHAPE),
    (dict(seqlen=0), _abi.FA_ERR_SHAPE),
    (dict(seqlen=-5), _abi.FA_ERR_SHAPE),
    (dict(scale=0.0), _abi.FA_ERR_SCALE),
    (dict(scale=-0.5), _abi.FA_ERR_SCALE),
    (dict(scale=math.inf), _abi.FA_ERR_SCALE),
    (dict(scale=math.nan), _abi.FA_ERR_SCALE),
    (dict(dtype=7), _abi.FA_ERR_DTYPE),
    (dict(dtype=_abi.FA_FP32, o_dtype=_abi.FA_BF16), _abi.FA_ERR_DTYPE),
    (dict(block_mask=0x9000, block_mask_ld=2), _abi.FA_ERR_MASK),
    (dict(block_mask=0x9000, block_mask_ld=(1 << 24) + 16), _abi.FA_ERR_MASK),
    (dict(window=(-1, 4)), _abi.FA_ERR_MASK),
    (dict(window=(3, -2)), _abi.FA_ERR_MASK),
    (dict(dropout_p=1.0), _abi.FA_ERR_DROPOUT),
    (dict(dropout_p=-0.1), _abi.FA_ERR_DROPOUT),
    (dict(dropout_p=math.nan), _abi.FA_ERR_DROPOUT),
    (dict(dropout_p=0.999995), _abi.FA_ERR_DROPOUT),  # T = round(0.33) = 0
    (dict(dtype=_abi.FA_FP8_E4M3, o_dtype=_abi.FA_BF16, descale=(1.0, 0.0, 1.0)),
     _abi.FA_ERR_SCALE),
    (dict(dtype=_abi.FA_FP8_E4M3, o_dtype=_abi.FA_BF16, descale=(1.0, 1.0, math.inf)),
     _abi.FA_ERR_SCALE),
    (dict(dtype=_abi.FA_FP8_E4M3, o_dtype=_abi.FA_FP8_E4M3), _abi.FA_ERR_DTYPE),
    (dict(dtype=_abi.FA_FP8_E4M3, o_dtype=_abi.FA_BF16, dropout_p=0.1), _abi.FA_ERR_DROPOUT),
    (dict(batch=1 << 20, heads_q=1 << 10, heads_kv=1 << 10, seqlen=1 << 20), _abi.FA_ERR_SHAPE),
])
def test_fwd_rejects_bad_params(mut, code):
    st, detail = _fwd(_params(**mut))
    assert st == code, (st, detail)
    assert detail


@no_gpu_only
def test_head_span_over_4_gib_is_rejected():
    """Staged tensors are addressed per head through a 32-bit buffer extent:
    (seqlen - 1) * row stride + head_dim elements must stay below 4 GiB."""
    # contiguous d=128 rows: 2^24 + 1 rows of 256 bytes span just over 4 GiB
    p = _params(batch=1, heads_q=1, heads_kv=1, seqlen=(1 << 24) + 1, head_dim=128)
    st, detail = _fwd(p)
    assert st == _abi.FA_ERR_SHAPE and "4 GiB" in detail, (st, detail)
    # 2^24 - 1 rows stay inside: the span check passes (what follows needs a GPU)
    p = _params(batch=1, heads_q=1, heads_kv=1, seqlen=(1 << 24) - 1, head_dim=128)
    assert _fwd(p)[0] != _abi.FA_ERR_SHAPE
    # a short sequence with a huge row stride
    p = _params()
    wide = _abi.Strides(0, 0, 1 << 26)
    st, detail = _fwd(p, sk=wide)
    assert st == _abi.FA_ERR_SHAPE and "k:" in detail, (st, detail)
    # the backward also stages Q and dO
    lib = fa.library()
    s = _strides(p)
    skv = _strides(p, p.heads_kv)
    st = lib.fa_bwd(ctypes.byref(p), P16, wide, P32, skv, P48, skv, P64, s, P80, s,
                    ctypes.c_void_p(0x6000), P16, s, P32, skv, P48, skv,
                    ctypes.c_void_p(0x8000), 1 << 30, None, None, None)
    assert st == _abi.FA_ERR_SHAPE, (st, lib.fa_last_error_detail().decode())


@no_gpu_only
def test_tile_rounded_rows_bound_the_span():
    """Tiles cover whole 128-row blocks: a tail tile addresses rows up to
    ceil(N/128)*128 - 1, and their 32-bit byte offsets must not wrap past
    4 GiB back into the buffer (rows past N must read as zeros)."""
    MiB = 1 << 20
    # forward, d=64, N=41, K row stride 100 MiB: the 41 valid rows span
    # 40 * 100 MiB + 128 B < 4 GiB, but rows 41..127 of the tile do not fit
    p = _params(batch=1, heads_q=1, heads_kv=1, seqlen=41, head_dim=64)
    assert 40 * 100 * MiB + 128 < 1 << 32
    wide = _abi.Strides(0, 0, 100 * MiB // 2)
    st, detail = _fwd(p, sk=wide)
    assert st == _abi.FA_ERR_SHAPE and "k:" in detail and "128-row" in detail, (st, detail)
    st, detail = _fwd(p, sk=_abi.Strides(0, 0, 64), sq=_abi.Strides(0, 0, 64))
    assert st != _abi.FA_ERR_SHAPE, detail
    # backward, d=64, N=100, Q row stride 41 MiB (the dK/dV kernel stages Q)
    p = _params(batch=1, heads_q=1, heads_kv=1, seqlen=100, head_dim=64)
    assert 99 * 41 * MiB + 128 < 1 << 32
    lib = fa.library()
    s = _abi.Strides(0, 0, 64)
    q41 = _abi.Strides(0, 0, 41 * MiB // 2)
    for pos in range(2):  # Q, then dO
        args = [s, s]
        args[pos] = q41
        st = lib.fa_bwd(ctypes.byref(p), P16, args[0], P32, s, P48, s, P64, s, P80, args[1],
                        ctypes.c_void_p(0x6000), P16, s, P32, s, P48, s,
                        ctypes.c_void_p(0x8000), 1 << 30, None, None, None)
        detail = lib.fa_last_error_detail().decode()
        assert st == _abi.FA_ERR_SHAPE and "128-row" in detail, (pos, st, detail)
    # the largest stride that still fits: 127 rows * stride + 128 B <= 4 GiB
    ok = ((1 << 32) - 128) // 127 // 16 * 16
    p = _params(batch=1, heads_q=1, heads_kv=1, seqlen=41, head_dim=64)
    assert _fwd(p, sk=_abi.Strides(0, 0, ok // 2))[0] != _abi.FA_ERR_SHAPE
    assert _fwd(p, sk=_abi.Strides(0, 0, ok // 2 + 8))[0] == _abi.FA_ERR_SHAPE


@no_gpu_only
def test_overlapping_rows_are_rejected():
    """A row stride below head_dim (e.g. a tensor expanded from one row) is
    FA_ERR_STRIDE for every [B][H][N][d] tensor of fa_fwd and fa_bwd: rows
    past N would otherwise read real rows where the kernels expect zeros."""
    p = _params()
    for key in ("sq", "sk", "so"):
        for row in (0, 8, 56):
            st, detail = _fwd(p, **{key: _abi.Strides(64, 64, row)})
            assert st == _abi.FA_ERR_STRIDE and "below head_dim" in detail, (key, row, st, detail)
    lib = fa.library()
    s, skv = _strides(p), _strides(p, p.heads_kv)
    zero = _abi.Strides(0, 0, 0)
    for pos in range(9):  # q, k, v, o, dout, dq, dk, dv in order (pos 8: none)
        st_args = [s, skv, skv, s, s, s, skv, skv]
        if pos < 8:
            st_args[pos] = zero
        st = lib.fa_bwd(ctypes.byref(p), P16, st_args[0], P32, st_args[1], P48, st_args[2],
                        P64, st_args[3], P80, st_args[4], ctypes.c_void_p(0x6000),
                        P16, st_args[5], P32, st_args[6], P48, st_args[7],
                        ctypes.c_void_p(0x8000), 1 << 30, None, None, None)
        if pos < 8:
            assert st == _abi.FA_ERR_STRIDE, (pos, st, lib.fa_last_error_detail().decode())
        else:
            assert st not in (_abi.FA_ERR_STRIDE, _abi.FA_ERR_SHAPE), st
    # decode: K and V rows must not overlap; q and o (row 0 only) are exempt
    pd = _params(heads_q=4, heads_kv=2, seqlen=300)
    one = _abi.Strides(4 * 64, 64, 0)
    st = lib.fa_decode(ctypes.byref(pd), P16, one, P32, zero, P48, skv, P64, one, P80,
                       ctypes.c_void_p(0x8000), 1 << 30, None)
    assert st == _abi.FA_ERR_STRIDE, (st, lib.fa_last_error_detail().decode())
    st = lib.fa_decode(ctypes.byref(pd), P16, one, P32, skv, P48, skv, P64, one, P80,
                       ctypes.c_void_p(0x8000), 1 << 30, None)
    assert st not in (_abi.FA_ERR_STRIDE, _abi.FA_ERR_SHAPE), st


@no_gpu_only
def test_fwd_rejects_bad_pointers_and_strides():
    p = _params()
    assert _fwd(p, q=ctypes.c_void_p(0))[0] == _abi.FA_ERR_NULL
    assert _fwd(p, lse=ctypes.c_void_p(0))[0] == _abi.FA_ERR_NULL
    assert _fwd(p, k=ctypes.c_void_p(0x1008))[0] == _abi.FA_ERR_ALIGN
    assert _fwd(p, o=ctypes.c_void_p(0x1004))[0] == _abi.FA_ERR_ALIGN
    assert _fwd(p, lse=ctypes.c_void_p(0x1002))[0] == _abi.FA_ERR_ALIGN
    assert _fwd(p, log=ctypes.c_void_p(0x1001))[0] == _abi.FA_ERR_ALIGN
    bad = _abi.Strides(1, 1, 1)
    assert _fwd(p, sq=bad)[0] == _abi.FA_ERR_STRIDE
    neg = _abi.Strides(-64, 64, 64)
    assert _fwd(p, sk=neg)[0] == _abi.FA_ERR_STRIDE
    # bf16 strides must be multiples of 8 elements (16 bytes)
    assert _fwd(_params(), sq=_abi.Strides(4, 4, 68))[0] == _abi.FA_ERR_STRIDE


@no_gpu_only
def test_bwd_validation():
    lib = fa.library()
    p = _params()
    s, skv = _strides(p), _strides(p, p.heads_kv)
    need = fa.fa_bwd_workspace_size(p)
    assert need == 2 * (2 * 4 * 300) * 4  # D and the base-2 LSE

    def call(p=p, ws=ctypes.c_void_p(0x7000), nbytes=need, ev=None):
        return lib.fa_bwd(ctypes.byref(p), P16, s, P32, skv, P48, skv, P64, s, P80, s,
                          ctypes.c_void_p(0x6000), P16, s, P32, skv, P48, skv, ws, nbytes,
                          None, ev, None)

    assert call(ws=ctypes.c_void_p(0)) == _abi.FA_ERR_WORKSPACE
    assert call(nbytes=need - 1) == _abi.FA_ERR_WORKSPACE
    assert call(ws=ctypes.c_void_p(0x7008)) == _abi.FA_ERR_ALIGN
    p32 = _params(dtype=_abi.FA_FP32, o_dtype=_abi.FA_FP32)
    assert call(p=p32) == _abi.FA_ERR_DTYPE
    ev = (ctypes.c_void_p * 3)(1, None, 3)
    assert call(ev=ctypes.cast(ev, ctypes.c_void_p)) == _abi.FA_ERR_NULL
    assert "stage_events" in lib.fa_last_error_detail().decode()


@no_gpu_only
def test_bwd_noalloc_rejects_problems_beyond_its_array():
    """fa_bwd_noalloc's workspace is the library's fixed array: a problem
    whose two row vectors need more than FA_NOALLOC_WORKSPACE_BYTES is
    FA_ERR_WORKSPACE, decided on the host before any HIP call."""
    lib = fa.library()
    assert _abi.FA_NOALLOC_WORKSPACE_BYTES == 32 << 20
    rows_max = _abi.FA_NOALLOC_WORKSPACE_BYTES // 8  # two fp32 values per row
    for seqlen, ok in ((rows_max // 16, True), (rows_max // 16 + 1, False)):
        p = _params(batch=1, heads_q=16, heads_kv=16, seqlen=seqlen)
        s = _strides(p)
        st = lib.fa_bwd_noalloc(ctypes.byref(p), P16, s, P32, s, P48, s, P64, s, P80, s,
                                ctypes.c_void_p(0x6000), P16, s, P32, s, P48, s, None, None, None)
        detail = lib.fa_last_error_detail().decode()
        if ok:
            assert st != _abi.FA_ERR_WORKSPACE, (seqlen, st, detail)
        else:
            assert st == _abi.FA_ERR_WORKSPACE and "fixed array" in detail, (seqlen, st, detail)
    # the other checks are fa_bwd's
    p = _params()
    s = _strides(p)
    st = lib.fa_bwd_noalloc(ctypes.byref(p), P16, s, P32, _abi.Strides(0, 0, 0), P48, s, P64, s,
                            P80, s, ctypes.c_void_p(0x6000), P16, s, P32, s, P48, s, None, None,
                            None)
    assert st == _abi.FA_ERR_STRIDE


def test_size_queries():
    p = _params(seqlen=4097)
    nlb = 33
    assert fa.fa_tile_log_words(p) == 2 * 4 * nlb * 2
    # two fp32 row vectors (D and the base-2 LSE) of B * Hq * N entries
    assert fa.fa_bwd_workspace_size(p) == 2 * (2 * 4 * 4097) * 4
    assert fa.fa_tile_log_words(_params(head_dim=80)) == 0
    assert fa.fa_bwd_workspace_size(_params(heads_q=3)) == 0


def test_params_struct_window_fields():
    """A zero-initialised fa_params has no window; make_params fills the flag
    and both widths."""
    z = _abi.Params()
    assert z.window == 0
    p = _params(window=(12, 0))
    assert (p.window, p.window_left, p.window_right) == (1, 12, 0)
    assert _params().window == 0


def test_params_struct_dropout_fields():
    """A zero-initialised fa_params has no dropout; make_params stores p as
    float32, the 64-bit seed and the 32-bit offset."""
    z = _abi.Params()
    assert z.dropout_p == 0.0 and z.dropout_seed == 0 and z.dropout_offset == 0
    p = _params(dropout_p=0.1, dropout_seed=2**64 - 1, dropout_offset=2**32 - 1)
    assert p.dropout_p == ctypes.c_float(0.1).value
    assert (p.dropout_seed, p.dropout_offset) == (2**64 - 1, 2**32 - 1)


def test_struct_layout_matches_the_c_header(tmp_path):
    """Field offsets and sizes of the ctypes mirrors equal those the C
    compiler gives include/fa.h."""
    import subprocess
    fields = [f for f, _ in _abi.Params._fields_]
    src = ['#include <stddef.h>', '#include <stdio.h>', '#include "fa.h"', "int main(void) {",
           '  printf("%zu\\n", sizeof(fa_params));',
           '  printf("%zu\\n", sizeof(fa_strides));']
    src += [f'  printf("%zu\\n", offsetof(fa_params, {f}));' for f in fields]
    src += ["  return 0;", "}"]
    c = tmp_path / "layout.c"
    c.write_text("\n".join(src) + "\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), str(c), "-o", str(exe)],
                   check=True)
    vals = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True,
                                           check=True).stdout.split()]
    assert vals[0] == ctypes.sizeof(_abi.Params)
    assert vals[1] == ctypes.sizeof(_abi.Strides)
    for f, off in zip(fields, vals[2:]):
        assert getattr(_abi.Params, f).offset == off, f


@no_gpu_only
def test_decode_rejects_dropout_window_and_mask():
    lib = fa.library()

    def call(**kw):
        p = _params(heads_q=8, heads_kv=2, **kw)
        sq = _abi.Strides(8 * 64, 64, 64)
        skv = _strides(p, p.heads_kv)
        st = lib.fa_decode(ctypes.byref(p), P16, sq, P32, skv, P48, skv, P64, sq, P80,
                           ctypes.c_void_p(0x7000), 1 << 30, None)
        return st
    assert call(dropout_p=0.1) == _abi.FA_ERR_DROPOUT
    assert call(window=(4, 0)) == _abi.FA_ERR_MASK
    assert call(dtype=_abi.FA_FP32, o_dtype=_abi.FA_FP32) == _abi.FA_ERR_DTYPE


@no_gpu_only
def test_fp8_is_forward_only():
    """The backward and decode reject FP8 inputs; FP8 strides are in bytes
    (multiples of 16)."""
    lib = fa.library()
    p = _params(dtype=_abi.FA_FP8_E4M3, o_dtype=_abi.FA_BF16)
    s8 = _abi.Strides(4 * 300 * 64, 300 * 64, 64)
    assert _fwd(p, sq=_abi.Strides(4 * 300 * 72, 300 * 72, 72))[0] == _abi.FA_ERR_STRIDE
    s, skv = _strides(p), _strides(p, p.heads_kv)
    st = lib.fa_bwd(ctypes.byref(p), P16, s8, P32, s8, P48, s8, P64, s, P80, s8,
                    ctypes.c_void_p(0x6000), P16, s8, P32, s8, P48, s8, ctypes.c_void_p(0x7000),
                    1 << 30, None, None, None)
    assert st == _abi.FA_ERR_DTYPE
