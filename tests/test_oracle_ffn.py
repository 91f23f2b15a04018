"""Pins of the oracle's layer (oracle/moe.py: moe_forward).

* mpmath brute force at 50 digits on tiny shapes (scalar loops, its own
  routing by sorting, its own BF16 / E4M3 decode and exact MX quantizer);
* identical experts reduce the layer to one dense SwiGLU FFN (torch float64,
  torch.nn.functional.silu);
* k = E equals the softmax-weighted dense mixture over all experts;
* expert relabelling gives a bit-identical output; doubling W_down doubles it.
"""
from fractions import Fraction

import mpmath
import numpy as np
import pytest
import torch

from oracle import formats as F
from oracle import moe_forward, route
from tests._exact import bf16_bits_to_float, mx_block_exact

mpmath.mp.dps = 50


def _bf16_bits(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)


def _rand_layer(rng, T, H, I, E, xs=1.0, ws=0.3):
    x = _bf16_bits(rng.standard_normal((T, H)) * xs)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    wgu = _bf16_bits(rng.standard_normal((E, 2 * I, H)) * ws)
    wd = _bf16_bits(rng.standard_normal((E, H, I)) * ws)
    return x, logits, wgu, wd


def _mp_silu(z):
    return z / (1 + mpmath.exp(-z))


def _mp_layer(xv, logits, gate_up, down, k, quant=None):
    """Scalar-loop layer at 50 digits.  xv[t][h], gate_up[e][n][h], down[e][d][n]
    are Python floats (already decoded); quant(list)->list re-quantizes a row."""
    T, H = len(xv), len(xv[0])
    E = len(gate_up)
    I = len(gate_up[0]) // 2
    outs = []
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-Fraction(float(logits[t][e])), e))[:k]
        ls = [mpmath.mpf(float(logits[t][e])) for e in order]
        ex = [mpmath.exp(v - ls[0]) for v in ls]
        den = mpmath.fsum(ex)
        xt = xv[t] if quant is None else quant(xv[t])
        out = [mpmath.mpf(0)] * H
        for j, e in enumerate(order):
            a = []
            for n in range(I):
                g = mpmath.fsum(mpmath.mpf(gate_up[e][n][h]) * xt[h] for h in range(H))
                u = mpmath.fsum(mpmath.mpf(gate_up[e][I + n][h]) * xt[h] for h in range(H))
                a.append(_mp_silu(g) * u)
            if quant is not None:
                a = quant([float(v) for v in a])   # a rounded to float64 first (< 2^-53 rel)
            wj = ex[j] / den
            for d in range(H):
                y = mpmath.fsum(mpmath.mpf(down[e][d][n]) * a[n] for n in range(I))
                out[d] += wj * y
        outs.append([float(v) for v in out])
    return np.array(outs)


def test_bf16_layer_matches_mpmath_bruteforce():
    rng = np.random.default_rng(11)
    T, H, I, E, k = 3, 8, 4, 4, 2
    x, logits, wgu, wd = _rand_layer(rng, T, H, I, E)
    dec = np.vectorize(bf16_bits_to_float)
    ref = _mp_layer(dec(x).tolist(), logits.tolist(), dec(wgu).tolist(), dec(wd).tolist(), k)
    got = moe_forward(x, logits, wgu, wd, k)
    assert np.max(np.abs(got - ref)) <= 1e-13 * np.max(np.abs(ref))


def _mx_quant_row(row):
    out = []
    for b in range(0, len(row), 32):
        codes, sc = mx_block_exact(row[b:b + 32])
        s = 2.0 ** (sc - 127)
        for c in codes:
            t = torch.tensor([c], dtype=torch.uint8).view(torch.float8_e4m3fn).double().item()
            out.append(mpmath.mpf(t) * s)
    return out


def test_mxfp8_layer_matches_mpmath_bruteforce():
    rng = np.random.default_rng(12)
    T, H, I, E, k = 2, 32, 32, 3, 2
    x = _bf16_bits(rng.standard_normal((T, H)))
    logits = rng.standard_normal((T, E)).astype(np.float32)
    wgu_codes = rng.integers(0, 0x7E, (E, 2 * I, H), dtype=np.uint8) | \
        (rng.integers(0, 2, (E, 2 * I, H), dtype=np.uint8) << 7)
    wd_codes = rng.integers(0, 0x7E, (E, H, I), dtype=np.uint8) | \
        (rng.integers(0, 2, (E, H, I), dtype=np.uint8) << 7)
    wgu_sc = rng.integers(118, 124, (E, 2 * I, H // 32), dtype=np.uint8)
    wd_sc = rng.integers(118, 124, (E, H, I // 32), dtype=np.uint8)

    def dec(codes, sc):
        v = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
        return (v.reshape(codes.shape[:-1] + (-1, 32)) *
                np.exp2(sc.astype(np.float64) - 127)[..., None]).reshape(codes.shape)

    xv = np.vectorize(bf16_bits_to_float)(x)
    ref = _mp_layer(xv.tolist(), logits.tolist(), dec(wgu_codes, wgu_sc).tolist(),
                    dec(wd_codes, wd_sc).tolist(), k, quant=_mx_quant_row)
    got = moe_forward(x, logits, wgu_codes, wd_codes, k, dtype="mxfp8",
                      w_gate_up_scales=wgu_sc, w_down_scales=wd_sc)
    assert np.max(np.abs(got - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_identical_experts_reduce_to_dense_swiglu():
    rng = np.random.default_rng(13)
    T, H, I, E, k = 9, 64, 48, 6, 3
    x, logits, wgu, wd = _rand_layer(rng, T, H, I, E, ws=0.1)
    wgu[:] = wgu[0]
    wd[:] = wd[0]
    got = moe_forward(x, logits, wgu, wd, k)
    xt = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).double()
    wg = torch.from_numpy(wgu[0].view(np.int16)).view(torch.bfloat16).double()
    wdn = torch.from_numpy(wd[0].view(np.int16)).view(torch.bfloat16).double()
    dense = (torch.nn.functional.silu(xt @ wg[:I].T) * (xt @ wg[I:].T)) @ wdn.T
    dense = dense.numpy()
    assert np.max(np.abs(got - dense)) <= 1e-13 * np.max(np.abs(dense))


def test_k_equals_E_is_dense_softmax_mixture():
    rng = np.random.default_rng(14)
    T, H, I, E = 7, 32, 24, 5
    x, logits, wgu, wd = _rand_layer(rng, T, H, I, E, ws=0.2)
    got = moe_forward(x, logits, wgu, wd, E)
    xt = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).double()
    wg = torch.from_numpy(wgu.view(np.int16)).view(torch.bfloat16).double()
    wdn = torch.from_numpy(wd.view(np.int16)).view(torch.bfloat16).double()
    p = torch.softmax(torch.from_numpy(logits).double(), dim=-1)          # [T, E]
    g = torch.einsum("th,enh->ten", xt, wg[:, :I])
    u = torch.einsum("th,enh->ten", xt, wg[:, I:])
    y = torch.einsum("ten,edn->ted", torch.nn.functional.silu(g) * u, wdn)
    dense = torch.einsum("te,ted->td", p, y).numpy()
    assert np.max(np.abs(got - dense)) <= 1e-13 * np.max(np.abs(dense))


def test_relabelling_bitwise_and_down_scaling():
    rng = np.random.default_rng(15)
    T, H, I, E, k = 16, 32, 16, 8, 3
    x, logits, wgu, wd = _rand_layer(rng, T, H, I, E)
    out = moe_forward(x, logits, wgu, wd, k)
    perm = rng.permutation(E)
    out2 = moe_forward(x, logits[:, perm], wgu[perm], wd[perm], k)
    assert np.array_equal(out.view(np.uint64), out2.view(np.uint64))
    wd2 = _bf16_bits(torch.from_numpy(wd.view(np.int16)).view(torch.bfloat16).float().numpy() * 2)
    out3 = moe_forward(x, logits, wgu, wd2, k)
    assert np.array_equal(out3, 2 * out)


def test_token_subset_equals_full_rows():
    rng = np.random.default_rng(16)
    T, H, I, E, k = 12, 32, 16, 6, 2
    x, logits, wgu, wd = _rand_layer(rng, T, H, I, E)
    full = moe_forward(x, logits, wgu, wd, k)
    sub = moe_forward(x, logits, wgu, wd, k, tokens=[3, 0, 11])
    assert np.array_equal(sub, full[[3, 0, 11]])
    out, inter = moe_forward(x, logits, wgu, wd, k, return_intermediates=True)
    idx, w = route(logits, k)
    assert np.array_equal(inter["idx"], idx) and np.array_equal(out, full)


def test_callable_weights_match_arrays():
    rng = np.random.default_rng(17)
    x, logits, wgu, wd = _rand_layer(rng, 5, 32, 16, 4)
    a = moe_forward(x, logits, wgu, wd, 2)
    b = moe_forward(x, logits, lambda e: wgu[e], lambda e: wd[e], 2)
    assert np.array_equal(a, b)


def test_shape_mismatch_rejected():
    rng = np.random.default_rng(18)
    x, logits, wgu, wd = _rand_layer(rng, 2, 32, 16, 4)
    with pytest.raises(ValueError):
        moe_forward(x, logits, wgu, wd[:, :, :8], 2)


def _mx_exact(rng, shape):
    """Values whose MX quantization is exact: E4M3 codes times one power of two
    per block of 32 along the last axis, each block holding a +-256 (so the
    block rule recovers the same scale).  Returns (codes, scales, float64)."""
    *lead, K = shape
    codes = rng.integers(0, 0x7F, size=shape).astype(np.uint8)     # finite, positive
    codes |= (rng.integers(0, 2, size=shape).astype(np.uint8) << 7)  # random sign
    blk = codes.reshape(*lead, K // 32, 32)
    blk[..., 0] = 0x78 | (blk[..., 0] & 0x80)                       # +-256 = 1.0 * 2^8
    blk[..., 1:] = np.where((blk[..., 1:] & 0x7F) > 0x78, blk[..., 1:] & 0x80, blk[..., 1:])
    codes = blk.reshape(shape)
    scales = rng.integers(118, 126, size=(*lead, K // 32)).astype(np.uint8)
    vals = F.mx_dequantize(codes, scales)
    return codes, scales, vals


def test_h_round_mxfp8_equals_mxfp8_mode_on_mx_exact_inputs():
    # with x and the weights already exactly MX-representable, the MXFP8 mode
    # (which re-quantizes x and a) and the BF16 mode with a quantized by h_round
    # perform the same float64 arithmetic
    rng = np.random.default_rng(21)
    T, H, I, E, k = 5, 64, 64, 4, 2
    _, _, xv = _mx_exact(rng, (T, H))
    gc, gs, gv = _mx_exact(rng, (E, 2 * I, H))
    dc, ds, dv = _mx_exact(rng, (E, H, I))
    logits = rng.standard_normal((T, E)).astype(np.float32)
    a = moe_forward(_bf16_bits(xv), logits, gc, dc, k, dtype="mxfp8",
                    w_gate_up_scales=gs, w_down_scales=ds)
    b = moe_forward(_bf16_bits(xv), logits, _bf16_bits(gv), _bf16_bits(dv), k, h_round="mxfp8")
    assert np.array_equal(a, b)


def test_h_round_bf16_rounds_the_activations_once():
    rng = np.random.default_rng(22)
    x, logits, wgu, wd = _rand_layer(rng, 4, 64, 32, 6)
    exact, ie = moe_forward(x, logits, wgu, wd, 3, return_intermediates=True)
    rounded, ir = moe_forward(x, logits, wgu, wd, 3, h_round="bf16", return_intermediates=True)
    assert np.array_equal(ir["a"], F.bf16_round(ie["a"]))
    # the output moves by at most the rounding of a, carried through the down projection
    dv = F.bf16_decode(wd)
    bound = np.zeros_like(exact)
    for t in range(4):
        for j in range(3):
            e = ie["idx"][t, j]
            bound[t] += ie["w"][t, j] * (np.abs(dv[e]) @ (np.abs(ie["a"][t, j]) * 2.0 ** -8))
    assert np.all(np.abs(rounded - exact) <= bound * (1 + 1e-9) + 1e-300)
    with pytest.raises(ValueError):
        moe_forward(x, logits, wgu, wd, 3, h_round="fp8")
