"""Checks of the seeded input generator (no attention arithmetic involved)."""
import numpy as np
import torch

from synth import (MASK_BLOCK, WORKLOADS, bf16_bits_to_f64, butterfly_block_mask,
                   draw, draw_case, f32_to_bf16_bits)


def test_bf16_rounding_matches_torch():
    """Round-to-nearest-even agrees with torch's float32 -> bfloat16 cast,
    including exact ties and values near powers of two."""
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(100000).astype(np.float32) * 10,
        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 255.5, 0.0, -0.0,
                  1e-30, 3.0e38], dtype=np.float32),
    ])
    ours = f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    back = bf16_bits_to_f64(ours)
    np.testing.assert_array_equal(back, torch.from_numpy(ours.view(np.int16)).view(
        torch.bfloat16).to(torch.float64).numpy())


def test_butterfly_pattern():
    bm = butterfly_block_mask(512)
    assert bm.shape == (512, 512)
    assert np.array_equal(bm, bm.T)
    assert np.all(np.diag(bm) == 1)
    assert np.all(bm.sum(axis=1) == 10)  # diagonal + 9 partners i ^ 2^k
    assert bm.sum() == 5120
    i = 37
    partners = sorted([i] + [i ^ (1 << k) for k in range(9)])
    assert list(np.nonzero(bm[i])[0]) == partners


def test_draws_are_deterministic_and_ordered():
    w = WORKLOADS[3]
    small = type(w)("t", 2, 2, 2, 64, 8, "bf16", causal=True, pad_range=(10, 20))
    a = draw(small, 3)
    b = draw(small, 3)
    for name in ("q", "k", "v", "do", "seqlens"):
        np.testing.assert_array_equal(getattr(a, name), getattr(b, name))
    assert a.seqlens.dtype == np.int32 and np.all((a.seqlens >= 10) & (a.seqlens <= 20))
    # draw order: Q first from the same stream
    rng = np.random.default_rng(3)
    q0 = f32_to_bf16_bits(rng.standard_normal((2, 2, 64, 8), dtype=np.float32))
    np.testing.assert_array_equal(a.q, q0)


def test_workload_table():
    assert WORKLOADS[2].describe() == "B64 Hq16 Hkv16 N1024 d64 bf16 fwd+bwd"
    assert WORKLOADS[4].group == 4
    assert WORKLOADS[1].dtype == "fp32" and not WORKLOADS[1].backward
    assert abs(WORKLOADS[3].scale - 0.08838834764831845) < 1e-8
    assert MASK_BLOCK == 128


def test_draw_case_masks():
    c = draw_case(2, 2, 1, 300, 8, seqlens="random", block_mask="random", seed=5)
    assert c.seqlens.shape == (2,) and c.block_mask.shape == (3, 3)
    assert np.all(np.diag(c.block_mask) == 1)


def test_fp8_workloads_encode_scaled_draws():
    """fp8 inputs are e4m3 codes of x / descale; the logical value
    descale * decode(code) is within half an e4m3 unit of the fp32 draw."""
    w = WORKLOADS[10]
    assert w.dtype == "fp8" and not w.backward and w.descale == (0.0625, 0.0625, 0.0625)
    assert "fp8" in w.describe() and "descale" in w.describe()
    small = type(w)("t", 1, 2, 2, 64, 64, "fp8", backward=False, descale=(0.25, 0.5, 2.0))
    inp = draw(small, 9)
    assert inp.q.dtype == np.uint8 and inp.descale == (0.25, 0.5, 2.0)
    rng = np.random.default_rng(9)
    x = rng.standard_normal((1, 2, 64, 64), dtype=np.float32).astype(np.float64)
    got = inp.as_f64("q")
    # half a unit: 2^-4 relative (normal range) or 2^-10 * descale absolute
    assert np.all(np.abs(got - x) <= np.maximum(2.0 ** -4 * np.abs(x), 2.0 ** -10 * 0.25) + 1e-15)
