"""Host-side work/traffic accounting, pinned to the pages' worked example and
to brute-force counts of the mask definitions."""
import json
import os

import numpy as np
import pytest

from exact_io_aware_29_amd import accounting as acc
from synth import WORKLOADS, butterfly_block_mask, draw
from tests import brute

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_score_matrix_size_worked_example():
    """The bowenzhou.top tutorial's exercise 1: 32 heads, sequence 32K, bf16
    (2 bytes): the N x N score matrix needs 32 * 32K * 32K * 2 bytes, about
    64 GB, more than one 80 GB card can spare."""
    g = json.load(open(os.path.join(GOLDEN, "score_matrix_size.json")))
    assert acc.score_matrix_bytes(g["heads"], g["seqlen"], g["bytes_per_element"]) == g["bytes"]
    assert acc.score_matrix_bytes(32, 32 * 1024, 2) == 64 * 2 ** 30


@pytest.mark.parametrize("N,causal,L,bm", [
    (37, False, None, None), (37, True, None, None), (37, True, 20, None),
    (40, False, 13, None), (48, True, None, "butterfly"), (33, False, 30, "random"),
])
def test_pair_counts_match_brute_force(N, causal, L, bm):
    block = 8
    nb = -(-N // block)
    mask = None
    if bm == "butterfly":
        mask = butterfly_block_mask(8)[:nb, :nb]
    elif bm == "random":
        rng = np.random.default_rng(1)
        mask = (rng.random((nb, nb)) < 0.5).astype(np.uint8)
    ours = acc.allowed_pairs_per_row(N, causal=causal, seqlen_k=L, block_mask=mask, block=block)
    ref = [sum(brute.allowed(i, j, causal, L, mask, block) for j in range(N)) for i in range(N)]
    assert list(ours) == ref


@pytest.mark.parametrize("N,causal,L,win", [
    (37, False, None, (3, 2)), (37, True, None, (5, 0)), (40, True, 31, (9, 4)),
    (29, False, 20, (0, 0)), (33, False, None, (40, 40)),
])
def test_window_pair_counts_and_tiles_match_brute_force(N, causal, L, win):
    block = 8
    ours = acc.allowed_pairs_per_row(N, causal=causal, seqlen_k=L, block=block, window=win)
    ref = [sum(brute.allowed(i, j, causal, L, None, block, win) for j in range(N))
           for i in range(N)]
    assert list(ours) == ref
    nb = -(-N // block)
    tiles = acc.tile_map(N, causal=causal, seqlen_k=L, block=block, window=win)
    for a in range(nb):
        for c in range(nb):
            any_pair = any(brute.allowed(i, j, causal, L, None, block, win)
                           for i in range(a * block, min(N, a * block + block))
                           for j in range(c * block, min(N, c * block + block)))
            assert tiles[a, c] == any_pair, (a, c)


def test_workload_flop_counts():
    """Forward = 4 d pairs; backward = 10 d pairs (five products)."""
    w2 = WORKLOADS[2]
    pairs = acc.allowed_pairs(w2.batch, w2.heads_q, w2.seqlen)
    assert pairs == 64 * 16 * 1024 * 1024
    f = acc.flops(pairs, 64)
    assert f["fwd"] == 274877906944 and f["fwd_bwd"] == 962072674304
    assert f["bwd_dkdv"] + f["bwd_dq"] == f["bwd"]
    w5 = WORKLOADS[5]
    p5 = acc.allowed_pairs(1, 8, 65536, block_mask=butterfly_block_mask(512))
    assert p5 == 8 * 65536 * 1280
    assert acc.visited_tiles(1, 8, 65536, block_mask=butterfly_block_mask(512)) == 8 * 5120
    # causal with padding: L(L+1)/2 + (N - L) L per (b, h)
    for L in (2048, 3000, 4096):
        assert acc.allowed_pairs(1, 1, 4096, causal=True, seqlens=[L]) == L * (L + 1) // 2 + (4096 - L) * L


def test_byte_models_order():
    w = WORKLOADS[2]
    tiles = acc.visited_tiles(w.batch, w.heads_q, w.seqlen)
    m = acc.bytes_models(w.batch, w.heads_q, w.heads_kv, w.seqlen, w.head_dim, 2, tiles=tiles)
    assert m["fwd_compulsory"] < m["fwd_tile_model"] < m["fwd_alg0"]
    assert m["bwd_compulsory"] < m["bwd_tile_model"] < m["bwd_alg0"]
    # compulsory forward = Q, K, V read + O written (bf16) + LSE (fp32)
    assert m["fwd_compulsory"] == 4 * 64 * 16 * 1024 * 64 * 2 + 64 * 16 * 1024 * 4


def test_decode_bytes():
    """K and V rows of each cache read once (bf16), q read and o written
    (bf16), LSE written (fp32)."""
    n = acc.decode_bytes(2, 8, 2, 128, [100, 0])
    assert n == 100 * 2 * 128 * 2 * 2 + 2 * 8 * 128 * 2 * 2 + 2 * 8 * 4
