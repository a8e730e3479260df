"""GPU parity for block-mask scans that cross many 64-block windows.

The kernels find the next present block of a mask row (forward, dQ) or
column (dK/dV) 64 blocks at a time. Here N = 200 * 128 - 37 (a ragged tail
and 200 mask blocks, so four windows), the mask pitch is wider than the
mask, and the mask has present blocks on window edges (0, 63, 64, 127,
128, 191, 192, 199), a row whose only block lies 169 blocks from its
diagonal, an empty row and an empty column; GQA with two query heads per
key/value head, both head dims, with and without the causal mask (causal
launches take query or key blocks in pairs). The visited-tile logs must
equal the mask exactly; O, LSE and dQ on sampled rows and dK/dV on sampled
key rows are compared with the fp64 oracle; rows without an allowed key
must give O = 0 and LSE = -inf, and keys no query sees zero gradients."""
import numpy as np
import pytest
import torch

import exact_io_aware_29_amd as fa
from synth import draw_case
from tests.gpu_util import (TOL_BF16_LSE, check_grad, check_lse, check_o, decode_log, dev,
                            expected_tiles, host64, oracle_heads)

pytestmark = pytest.mark.gpu

NB = 200
N = NB * 128 - 37
EDGES = [0, 63, 64, 127, 128, 191, 192, 199]
EMPTY_ROW, GAP_ROW, EMPTY_COL = 70, 30, 150


def mask() -> np.ndarray:
    rng = np.random.default_rng(2025)
    bm = (rng.random((NB, NB)) < 0.02).astype(np.uint8)
    np.fill_diagonal(bm, 1)
    bm[::7][:, EDGES] = 1
    bm[EMPTY_ROW, :] = 0
    bm[GAP_ROW, :] = 0
    bm[GAP_ROW, NB - 1] = 1
    bm[:, EMPTY_COL] = 0
    return bm


def _rows(blocks, step):
    r = np.concatenate([np.arange(b * 128, min(N, b * 128 + 128), step) for b in blocks])
    return np.unique(np.concatenate([r, [N - 1]]))


@pytest.mark.parametrize("d,causal", [(64, False), (64, True), (128, False), (128, True)])
def test_mask_scan_across_windows(d, causal):
    print(f"mask scan N{N} d{d} causal={causal}", flush=True)
    bm = mask()
    inp = draw_case(1, 2, 1, N, d, causal=causal, block_mask=bm, seed=d + causal)
    q, k, v, do = (dev(inp.q, "bf16"), dev(inp.k, "bf16"), dev(inp.v, "bf16"),
                   dev(inp.do, "bf16"))
    wide = torch.zeros((NB, 256), dtype=torch.uint8)
    wide[:, :NB] = torch.from_numpy(bm)
    bmd = wide.cuda()[:, :NB]  # pitch 256 bytes, wider than the mask
    kw = dict(scale=inp.scale, causal=causal, block_mask=bmd)
    o, lse, flog = fa.fa_fwd(q, k, v, tile_log=True, **kw)
    dq, dk, dv, blog = fa.fa_bwd(q, k, v, o, lse, do, tile_log=True, **kw)
    torch.cuda.synchronize()

    exp = expected_tiles(1, 2, N, causal, None, bm)
    assert np.array_equal(decode_log(flog, 1, 2, N), exp), "forward tiles"
    half = blog.numel() // 2
    assert np.array_equal(decode_log(blog[:half], 1, 2, N), exp), "dQ tiles"
    assert np.array_equal(decode_log(blog[half:], 1, 2, N), exp), "dK/dV tiles"

    # Rows of the empty mask row (and, under the causal mask, of the row
    # whose only block is above the diagonal) see no key.
    empty = [EMPTY_ROW] + ([GAP_ROW] if causal else [])
    for blk in empty:
        r = slice(blk * 128, blk * 128 + 128)
        assert torch.all(o[0, :, r] == 0) and torch.all(torch.isneginf(lse[0, :, r]))
        assert torch.all(dq[0, :, r] == 0)
    c = slice(EMPTY_COL * 128, EMPTY_COL * 128 + 128)
    assert torch.all(dk[0, :, c] == 0) and torch.all(dv[0, :, c] == 0)

    q_rows = _rows([0, GAP_ROW, 63, 64, 127, 128, 191, 192, NB - 1], 9)
    k_rows = _rows([0, 63, 64, 128, NB - 1], 5)
    ref = oracle_heads(inp, [(0, 0), (0, 1)], q_rows=q_rows, k_rows=k_rows)
    for h in (0, 1):
        r = ref[(0, h)]
        fin = np.isfinite(r["lse"])
        check_o(host64(o[0, h])[q_rows], r["o"], True, f"h{h}")
        check_lse(host64(lse[0, h])[q_rows][fin], r["lse"][fin], TOL_BF16_LSE, f"h{h}")
        check_grad(host64(dq[0, h])[q_rows], r["dq"], "dQ", f"h{h}")
    kv = ref[(0, 0, "kv")]
    check_grad(host64(dk[0, 0])[k_rows], kv["dk"], "dK")
    check_grad(host64(dv[0, 0])[k_rows], kv["dv"], "dV")


@pytest.mark.parametrize("d,causal", [(64, False), (128, True)])
def test_fp8_forward_mask_scan_across_windows(d, causal):
    """The FP8 forward walks the same mask rows: its visited tiles must equal
    the mask exactly, and rows of the empty mask row must give O = 0 and
    LSE = -inf (values of visited rows are covered by the FP8 parity tests)."""
    print(f"fp8 mask scan N{N} d{d} causal={causal}", flush=True)
    bm = mask()
    g = torch.Generator(device="cpu").manual_seed(d)
    q, k, v = (torch.randn((1, 2 if i == 0 else 1, N, d), generator=g).to(torch.float8_e4m3fn)
               .cuda() for i in range(3))
    o, lse, flog = fa.fa_fwd(q, k, v, causal=causal, block_mask=torch.from_numpy(bm).cuda(),
                             tile_log=True)
    torch.cuda.synchronize()
    assert np.array_equal(decode_log(flog, 1, 2, N), expected_tiles(1, 2, N, causal, None, bm))
    r = slice(EMPTY_ROW * 128, EMPTY_ROW * 128 + 128)
    assert torch.all(o[0, :, r].float() == 0) and torch.all(torch.isneginf(lse[0, :, r]))
    assert torch.isfinite(o.float()).all()
