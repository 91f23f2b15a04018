"""Pins of the oracle's MXFP8 backward (oracle/backward.py: moe_backward_mxfp8).

* Structure: with its quantizer replaced by the identity it is the FP64
  backward (moe_backward, dtype "f64") of the same decoded inputs, whose own
  pins are finite differences and autograd.
* Axes and rounding: a 50-digit mpmath scalar-loop brute force of the reading,
  quantizing every operand with the exact rational MX quantizer of
  tests/_exact.py (nearest E4M3 value found by search, the scale by stepping
  powers of two) along the stated axis: H for dh, 2I for dx, the expert's
  routed pairs (token order, blocks of 32 from the first) for both weight
  gradients.
* Special cases: zero output gradient, k = 1 (no logit gradient), an expert no
  token routes to (zero weight gradients), token / expert subsets.
"""
from fractions import Fraction

import mpmath
import numpy as np
import pytest
import torch

from oracle import formats as F
from oracle import moe_backward, moe_backward_mxfp8, route
from tests._exact import E4M3_TABLE, mx_block_exact

mpmath.mp.dps = 50

_E4M3_EXACT = {code: v for v, code in E4M3_TABLE}


def _dec_code(c):
    """E4M3 code -> Fraction, from the exact table."""
    v = _E4M3_EXACT[c & 0x7F]
    return -v if c & 0x80 else v


def _bf16_bits(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)


def _mx_weights(rng, E, R, K, std):
    w = rng.standard_normal((E, R, K)) * std
    codes, scales = F.mx_quantize(w)
    return codes, scales


def _case(seed, T=5, H=32, I=32, E=3, k=2):
    rng = np.random.default_rng(seed)
    x = _bf16_bits(rng.standard_normal((T, H)))
    dout = _bf16_bits(rng.standard_normal((T, H)))
    logits = rng.standard_normal((T, E)).astype(np.float32)
    wgu, wgus = _mx_weights(rng, E, 2 * I, H, 0.3)
    wd, wds = _mx_weights(rng, E, H, I, 0.3)
    return x, logits, wgu, wgus, wd, wds, dout, k


def test_identity_quantizer_is_the_fp64_backward():
    x, logits, wgu, wgus, wd, wds, dout, k = _case(1, T=7, H=64, I=32, E=4, k=2)
    got = moe_backward_mxfp8(x, logits, wgu, wgus, wd, wds, dout, k, quant=lambda m: m)
    want = moe_backward(F.bf16_decode(x), logits, F.mx_dequantize(wgu, wgus),
                        F.mx_dequantize(wd, wds), F.bf16_decode(dout), k, dtype="f64")
    for key in ("dx", "d_topk_w", "dlogits", "dw_gate_up", "dw_down"):
        ref = want[key]
        assert np.allclose(got[key], ref, rtol=1e-12, atol=1e-12 * max(1.0, np.abs(ref).max())), key


def _mp(v):
    return mpmath.mpf(v) if not isinstance(v, Fraction) else mpmath.mpf(v.numerator) / v.denominator


def _frac(v):
    """mpmath value -> exact Fraction (its binary expansion at 50 digits)."""
    sign, man, exp, _ = mpmath.mpf(v)._mpf_          # value = (-1)^sign * man * 2^exp
    m = -int(man) if sign else int(man)
    return Fraction(m) * (Fraction(2) ** exp) if exp >= 0 else Fraction(m, 2 ** (-exp))


def _q(vec):
    """Exact MX round trip of a list of mpmath values (length a multiple of 32)."""
    out = []
    for b in range(0, len(vec), 32):
        blk = [_frac(v) for v in vec[b:b + 32]]
        codes, sc = mx_block_exact(blk)
        scale = Fraction(2) ** (sc - 127)
        out += [_mp(_dec_code(c) * scale) for c in codes]
    return out


def _q_pairs(vec):
    """Along a pair axis: zero-pad to a multiple of 32, quantize, drop the pad."""
    n = len(vec)
    pad = (-n) % 32
    return _q(list(vec) + [mpmath.mpf(0)] * pad)[:n]


def _brute(x, logits, wgu, wgus, wd, wds, dout, k):
    T, H = x.shape
    E = wgu.shape[0]
    I = wgu.shape[1] // 2
    xv = [[_mp(F.bf16_decode(x[t, h])) for h in range(H)] for t in range(T)]
    dv = [[_mp(F.bf16_decode(dout[t, h])) for h in range(H)] for t in range(T)]

    def wdec(codes, scales, e, r, c):
        return _mp(_dec_code(int(codes[e, r, c])) * Fraction(2) ** (int(scales[e, r, c // 32]) - 127))
    Wgu = [[[wdec(wgu, wgus, e, r, c) for c in range(H)] for r in range(2 * I)] for e in range(E)]
    Wd = [[[wdec(wd, wds, e, r, c) for c in range(I)] for r in range(H)] for e in range(E)]
    # routing: order by (logit desc, index asc), renormalised softmax
    sel, wts = [], []
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-Fraction(float(logits[t][e])), e))[:k]
        ls = [mpmath.mpf(float(logits[t][e])) for e in order]
        ex = [mpmath.exp(v - ls[0]) for v in ls]
        den = mpmath.fsum(ex)
        sel.append(order)
        wts.append([v / den for v in ex])
    xq = [_q(row) for row in xv]
    dq = [_q(row) for row in dv]
    dx = [[mpmath.mpf(0)] * H for _ in range(T)]
    dtw = [[mpmath.mpf(0)] * k for _ in range(T)]
    dWd = [[[mpmath.mpf(0)] * I for _ in range(H)] for _ in range(E)]
    dWgu = [[[mpmath.mpf(0)] * H for _ in range(2 * I)] for _ in range(E)]
    sig = lambda z: 1 / (1 + mpmath.exp(-z))
    for e in range(E):
        pairs = [(t, j) for t in range(T) for j in range(k) if sel[t][j] == e]   # token order
        if not pairs:
            continue
        WdTq = [_q([Wd[e][h][i] for h in range(H)]) for i in range(I)]          # column i along H
        WguTq = [_q([Wgu[e][c][h] for c in range(2 * I)]) for h in range(H)]     # column h along 2I
        A, DGU, DY, X = [], [], [], []
        for (t, j) in pairs:
            g = [mpmath.fsum(Wgu[e][n][h] * xq[t][h] for h in range(H)) for n in range(I)]
            u = [mpmath.fsum(Wgu[e][I + n][h] * xq[t][h] for h in range(H)) for n in range(I)]
            a = [g[n] * sig(g[n]) * u[n] for n in range(I)]
            dh = [mpmath.fsum(dq[t][h] * WdTq[i][h] for h in range(H)) for i in range(I)]
            w = wts[t][j]
            dg = [w * dh[n] * u[n] * sig(g[n]) * (1 + g[n] * (1 - sig(g[n]))) for n in range(I)]
            du = [w * dh[n] * g[n] * sig(g[n]) for n in range(I)]
            dgu = dg + du
            dtw[t][j] = mpmath.fsum(a[n] * dh[n] for n in range(I))
            dgq = _q(dgu)
            for h in range(H):
                dx[t][h] += mpmath.fsum(dgq[c] * WguTq[h][c] for c in range(2 * I))
            A.append(a)
            DGU.append(dgu)
            DY.append([w * dv[t][h] for h in range(H)])
            X.append(xv[t])
        qa = [_q_pairs([A[p][i] for p in range(len(pairs))]) for i in range(I)]
        qdy = [_q_pairs([DY[p][h] for p in range(len(pairs))]) for h in range(H)]
        qdgu = [_q_pairs([DGU[p][c] for p in range(len(pairs))]) for c in range(2 * I)]
        qx = [_q_pairs([X[p][h] for p in range(len(pairs))]) for h in range(H)]
        for h in range(H):
            for i in range(I):
                dWd[e][h][i] = mpmath.fsum(qdy[h][p] * qa[i][p] for p in range(len(pairs)))
        for c in range(2 * I):
            for h in range(H):
                dWgu[e][c][h] = mpmath.fsum(qdgu[c][p] * qx[h][p] for p in range(len(pairs)))
    dl = [[mpmath.mpf(0)] * E for _ in range(T)]
    for t in range(T):
        s = mpmath.fsum(wts[t][j] * dtw[t][j] for j in range(k))
        for j in range(k):
            dl[t][sel[t][j]] = wts[t][j] * (dtw[t][j] - s)
    f = lambda m: np.array(m, dtype=np.float64)
    return {"dx": f(dx), "d_topk_w": f(dtw), "dlogits": f(dl), "dw_gate_up": f(dWgu),
            "dw_down": f(dWd)}


@pytest.mark.parametrize("seed,k", [(2, 2), (3, 1)])
def test_brute_force_mpmath(seed, k):
    x, logits, wgu, wgus, wd, wds, dout, _ = _case(seed, T=4, H=32, I=32, E=3, k=k)
    got = moe_backward_mxfp8(x, logits, wgu, wgus, wd, wds, dout, k)
    want = _brute(x, logits, wgu, wgus, wd, wds, dout, k)
    for key in ("dx", "d_topk_w", "dlogits", "dw_gate_up", "dw_down"):
        ref = want[key]
        scale = max(1e-30, np.abs(ref).max())
        assert np.max(np.abs(got[key] - ref)) <= 1e-12 * scale, key


def test_special_cases():
    x, logits, wgu, wgus, wd, wds, dout, k = _case(4, T=6, H=32, I=32, E=5, k=2)
    # zero output gradient: every gradient is exactly zero
    z = moe_backward_mxfp8(x, logits, wgu, wgus, wd, wds, np.zeros_like(dout), k)
    for key in ("dx", "d_topk_w", "dlogits", "dw_gate_up", "dw_down"):
        assert not np.any(z[key]), key
    # an expert no token routes to has zero weight gradients
    lg = logits.copy()
    lg[:, 4] = -50.0
    r = moe_backward_mxfp8(x, lg, wgu, wgus, wd, wds, dout, k)
    assert not np.any(r["dw_gate_up"][4]) and not np.any(r["dw_down"][4])
    # k = 1: the weight is 1 for any logit, so the logits get no gradient
    r1 = moe_backward_mxfp8(x, logits, wgu, wgus, wd, wds, dout, 1)
    assert not np.any(r1["dlogits"])
    # subsets equal the full result
    full = moe_backward_mxfp8(x, logits, wgu, wgus, wd, wds, dout, k)
    sub = moe_backward_mxfp8(x, logits, wgu, wgus, wd, wds, dout, k, tokens=[1, 4],
                             experts=[0, 3])
    for key in ("dx", "d_topk_w", "dlogits"):
        assert np.allclose(sub[key], full[key][[1, 4]], rtol=1e-14, atol=1e-300), key
    for key in ("dw_gate_up", "dw_down"):
        assert np.allclose(sub[key], full[key][[0, 3]], rtol=1e-14, atol=1e-300), key


def test_close_to_the_unquantized_backward():
    # information, with a loose bar: MX quantization of every operand moves the
    # gradients by a few percent relative L2
    x, logits, wgu, wgus, wd, wds, dout, k = _case(5, T=64, H=64, I=64, E=4, k=2)
    mx = moe_backward_mxfp8(x, logits, wgu, wgus, wd, wds, dout, k)
    ex = moe_backward(F.bf16_decode(x), logits, F.mx_dequantize(wgu, wgus),
                      F.mx_dequantize(wd, wds), F.bf16_decode(dout), k, dtype="f64")
    for key in ("dx", "dw_gate_up", "dw_down"):
        rl = np.linalg.norm(mx[key] - ex[key]) / np.linalg.norm(ex[key])
        assert 1e-3 < rl < 0.15, (key, rl)
