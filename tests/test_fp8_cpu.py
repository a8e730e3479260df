"""CPU pins of the FP8 pieces: the e4m3 codec of the input generator against
torch's float8_e4m3fn (exhaustive decode, random and edge encodes), and the
FP8 forward's error bound against a CPU model of the kernel's quantization
of P~ (lagged running maximum, nearest and truncating e4m3 rounding)."""
import numpy as np
import torch

import oracle
import oracle.attention as OA
from synth import e4m3_bits_to_f64, f32_to_e4m3_bits, draw_case
from tests.fp8_bound import fp8_o_bound


def test_e4m3_decode_every_code_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = e4m3_bits_to_f64(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    np.testing.assert_array_equal(np.isnan(ours), np.isnan(ref))
    fin = ~np.isnan(ref)
    np.testing.assert_array_equal(ours[fin], ref[fin])
    assert ours[0x7E] == 448 and ours[0x01] == 2.0 ** -9 and ours[0x08] == 2.0 ** -6
    assert np.isnan(ours[0x7F]) and np.isnan(ours[0xFF])


def test_e4m3_encode_matches_torch_and_saturates():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(100000) * np.exp2(rng.integers(-14, 9, 100000))
    x = np.concatenate([x, [448.0, -448.0, 447.9, 2.0 ** -10, 3 * 2.0 ** -10, 0.0, -0.0,
                            1.0625, 1.1875, 2.0 ** -6, 2.0 ** -6 * (1 - 1 / 16), 240.0, 232.0]])
    x = x[np.abs(x) <= 448].astype(np.float32)
    ours = f32_to_e4m3_bits(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(ours, ref)
    assert f32_to_e4m3_bits(np.array([1e4, -600.0]))[0] == 0x7E
    assert f32_to_e4m3_bits(np.array([1e4, -600.0]))[1] == 0xFE
    # decode(encode(x)) is the nearest finite e4m3 value
    finite = e4m3_bits_to_f64(np.arange(256, dtype=np.uint8))
    finite = np.unique(finite[~np.isnan(finite)])
    y = x[:2000].astype(np.float64)
    nearest = finite[np.abs(finite[None, :] - y[:, None]).argmin(axis=1)]
    np.testing.assert_array_equal(np.abs(e4m3_bits_to_f64(ours[:2000]) - y),
                                  np.abs(nearest - y))


def _quantize(x, mode):
    if mode == "nearest":
        return e4m3_bits_to_f64(f32_to_e4m3_bits(x))
    # truncation toward zero to the e4m3 grid (a worst-case rounding mode)
    finite = e4m3_bits_to_f64(np.arange(0, 0x7F, dtype=np.uint8))
    idx = np.searchsorted(finite, x, side="right") - 1
    return finite[np.clip(idx, 0, None)]


def test_fp8_bound_covers_a_cpu_model_of_the_kernel():
    inp = draw_case(1, 2, 1, 200, 64, "fp8", causal=True, seqlens=[150], seed=4,
                    with_do=False, descale=(0.25, 0.5, 0.125))
    q, k, v = inp.as_f64("q"), inp.as_f64("k"), inp.as_f64("v")
    o_ref, _ = oracle.attention_forward(q, k, v, inp.scale, causal=True, seqlens=inp.seqlens)
    m = OA.mask_for(0, causal=True, seqlens=inp.seqlens)
    rows = np.arange(200)
    for h in range(2):
        p = OA.probabilities(q[0, h], k[0, 0], inp.scale, m)
        allowed = m.allowed(rows, rows)
        bound = fp8_o_bound(p, v[0, 0], allowed)
        s = inp.scale * (q[0, h] @ k[0, 0].T) / np.log(2.0)   # log2 units
        s = np.where(allowed, s, -np.inf)
        mx = s.max(axis=1, keepdims=True)
        for lag in (0.0, 3.7, 8.0):
            for mode in ("nearest", "truncate"):
                pt = np.exp2(s - (mx - lag))                    # P~ in [0, 2^lag]
                l = pt.sum(axis=1, keepdims=True)
                o = (_quantize(pt, mode) @ v[0, 0]) / l
                err = np.abs(o - o_ref[0, h])
                assert np.all(err <= bound + 1e-12), (h, lag, mode, float((err - bound).max()))
                if mode == "truncate":
                    # the bound is not vacuous: it is within a small factor of
                    # what a worst-case rounding reaches
                    assert err.max() > 0.05 * bound.max()
