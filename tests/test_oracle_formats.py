"""Pins of the oracle's number formats (oracle/formats.py).

Checked against torch's own bfloat16 / float8_e4m3fn dtypes (library
routines independent of the oracle) and against exact-rational brute force."""
import numpy as np
import pytest
import torch

from oracle import formats as F
from tests._exact import E4M3_TABLE, e4m3_nearest_code, mx_block_exact


def test_bf16_decode_exhaustive_matches_torch():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ours = F.bf16_decode(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan].view(np.uint64), ref[~nan].view(np.uint64))  # bitwise, keeps -0


def test_e4m3_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = F.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert list(np.nonzero(nan)[0]) == [0x7F, 0xFF]
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan].view(np.uint64), ref[~nan].view(np.uint64))
    assert F.e4m3_decode(0x7E) == 448.0 and F.e4m3_decode(0x08) == 2.0 ** -6
    assert F.e4m3_decode(0x01) == 2.0 ** -9


def test_e4m3_roundtrip_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    assert np.array_equal(F.e4m3_encode(F.e4m3_decode(codes)), codes)


def test_e4m3_midpoints_round_to_even_code():
    vals = [v for v, _ in E4M3_TABLE]
    codes = [c for _, c in E4M3_TABLE]
    for i in range(len(vals) - 1):
        mid = float((vals[i] + vals[i + 1]) / 2)
        want = codes[i] if codes[i] % 2 == 0 else codes[i + 1]
        assert F.e4m3_encode(mid) == want, (mid, codes[i], codes[i + 1])
        assert F.e4m3_encode(-mid) == want | 0x80


def test_e4m3_saturation_and_signed_zero():
    for v in (448.0, 448.0001, 463.99, 464.0, 480.0, 1e30):
        assert F.e4m3_encode(v) == 0x7E
        assert F.e4m3_encode(-v) == 0xFE
    assert F.e4m3_encode(0.0) == 0x00
    assert F.e4m3_encode(-0.0) == 0x80
    assert F.e4m3_encode(2.0 ** -10) == 0x00        # half the smallest subnormal: tie to even 0
    assert F.e4m3_encode(2.0 ** -10 * 1.0001) == 0x01
    with pytest.raises(ValueError):
        F.e4m3_encode(np.nan)


def test_e4m3_encode_random_vs_bruteforce_and_torch():
    rng = np.random.default_rng(1)
    v = np.concatenate([rng.standard_normal(4000) * s for s in (1e-3, 0.05, 1, 30, 200)])
    v = v[np.abs(v) < 440]
    ours = F.e4m3_encode(v)
    brute = np.array([e4m3_nearest_code(float(x)) for x in v], dtype=np.uint8)
    assert np.array_equal(ours, brute)
    # torch's RNE cast agrees wherever it does not overflow
    tor = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, tor)


def test_e8m0_decode():
    c = np.arange(255, dtype=np.uint8)
    assert np.array_equal(F.e8m0_decode(c), np.exp2(np.arange(255) - 127.0))
    assert np.isnan(F.e8m0_decode(255))
    assert F.e8m0_decode(127) == 1.0


def test_mx_quantize_matches_exact_quantizer():
    rng = np.random.default_rng(7)
    blocks = []
    for scale in (1e-6, 0.02, 1.0, 3.0, 1e4):
        blocks.append(rng.standard_normal((40, 32)) * scale)
    b = np.concatenate(blocks)
    # exact powers of two, values at the saturation edge, zero block, one-hot block
    b[0] = 0.0
    b[1] = 0.0
    b[1, 5] = -2.0 ** 10
    b[2, :] = 2.0 ** 3
    b[3] = np.linspace(-1, 1, 32) * (2.0 ** 9 - 1)        # max just below a power of two
    b[4] = np.linspace(-1, 1, 32) * 1.99999 * 2.0 ** 5    # values that saturate to 448 * 2^s
    codes, scales = F.mx_quantize(b)
    for r in range(b.shape[0]):
        want_codes, want_scale = mx_block_exact(b[r].tolist())
        assert scales[r, 0] == want_scale, r
        assert list(codes[r]) == want_codes, r


def test_mx_quantize_invariants():
    rng = np.random.default_rng(3)
    v = rng.standard_normal((64, 256)) * 0.7
    codes, scales = F.mx_quantize(v)
    s = scales.astype(np.int64) - 127
    deq = F.mx_dequantize(codes, scales)
    blocks = np.abs(v.reshape(64, 8, 32))
    # the block max lands in the top E4M3 binade [256, 448] after scaling
    top = blocks.max(-1) / np.exp2(s)
    assert np.all((top >= 256) & (top < 512))
    # error at most half a step of the element's binade (saturated ones excepted)
    err = np.abs(deq - v).reshape(64, 8, 32)
    binade = np.floor(np.log2(np.maximum(blocks / np.exp2(s)[..., None], 2.0 ** -6)))
    half_step = np.exp2(binade - 4) * np.exp2(s)[..., None]
    sat = blocks / np.exp2(s)[..., None] > 448
    assert np.all(err[~sat] <= half_step[~sat] * (1 + 1e-12))
    # scaling a block by 2^j moves the scale code by j and keeps every code
    c2, s2 = F.mx_quantize(v * 2.0 ** 5)
    assert np.array_equal(c2, codes)
    assert np.array_equal(s2.astype(int) - scales.astype(int), np.full(scales.shape, 5))


def test_bf16_round_matches_torch_on_float32_inputs():
    # torch's float32 -> bfloat16 cast (round to nearest even) is an independent
    # routine; on float32 inputs one rounding from float64 equals it
    rng = np.random.default_rng(11)
    mag = rng.standard_normal(40000) * np.exp2(rng.integers(-140, 120, 40000).astype(np.float64))
    ties = (rng.integers(0, 1 << 16, 2000).astype(np.uint32) << 16 | 0x8000).view(np.float32)
    subn = (rng.integers(1, 1 << 23, 2000).astype(np.uint32)).view(np.float32)   # float32 subnormals
    v = np.concatenate([mag.astype(np.float32), ties, subn, -ties, np.float32([0.0, -0.0])])
    v = v[np.isfinite(v)]
    ours = F.bf16_round(v.astype(np.float64))
    ref = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(ours, ref)


def test_bf16_round_fixes_bf16_values_and_bounds_error():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    vals = F.bf16_decode(bits)
    vals = vals[np.isfinite(vals)]
    assert np.array_equal(F.bf16_round(vals), vals)            # BF16 values are fixed points
    rng = np.random.default_rng(12)
    v = rng.standard_normal(100000) * np.exp2(rng.integers(-100, 100, 100000).astype(np.float64))
    r = F.bf16_round(v)
    # unit roundoff of an 8-bit significand: |r - v| <= 2^-8 |v|
    assert np.all(np.abs(r - v) <= np.abs(v) * 2.0 ** -8 * (1 + 1e-15))
    assert np.array_equal(F.bf16_round(r), r)
