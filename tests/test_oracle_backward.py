"""Pins of the oracle's backward pass (oracle/backward.py: moe_backward).

Each check is a different route to the same derivative:
* central finite differences of the forward oracle (float64 mode), along
  random directions and entry by entry, for x, W_gate_up and W_down;
* central finite differences in the router logits (FP32 logits moved by an
  exact step of 2^-10 that keeps the top-k selection);
* torch.autograd in float64 on the layer written with torch operations;
* special cases: k = 1 (weights constant, zero logit gradient), zero dout,
  an expert nobody routes to, and subsets equal to the full result.
"""
import numpy as np
import pytest
import torch

from oracle import moe_backward, moe_forward, route
from oracle.formats import bf16_decode


def _layer(rng, T=6, H=16, I=8, E=5, ws=0.4):
    x = rng.standard_normal((T, H))
    logits = rng.standard_normal((T, E)).astype(np.float32)
    wgu = rng.standard_normal((E, 2 * I, H)) * ws
    wd = rng.standard_normal((E, H, I)) * ws
    dout = rng.standard_normal((T, H))
    return x, logits, wgu, wd, dout


def _loss(x, logits, wgu, wd, dout, k):
    return float(np.sum(dout * moe_forward(x, logits, wgu, wd, k, dtype="f64")))


@pytest.mark.parametrize("k", [1, 2, 3])
def test_directional_finite_differences(k):
    rng = np.random.default_rng(10 + k)
    x, logits, wgu, wd, dout = _layer(rng)
    g = moe_backward(x, logits, wgu, wd, dout, k, dtype="f64")
    eps = 1e-6
    for name, base, grad in (("x", x, g["dx"]), ("w_gate_up", wgu, g["dw_gate_up"]),
                             ("w_down", wd, g["dw_down"])):
        v = rng.standard_normal(base.shape)
        args = {"x": x, "w_gate_up": wgu, "w_down": wd}
        args_p = dict(args, **{name: base + eps * v})
        args_m = dict(args, **{name: base - eps * v})
        fd = (_loss(args_p["x"], logits, args_p["w_gate_up"], args_p["w_down"], dout, k)
              - _loss(args_m["x"], logits, args_m["w_gate_up"], args_m["w_down"], dout, k)) / (2 * eps)
        an = float(np.sum(grad * v))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, fd, an)


def test_entrywise_finite_differences():
    rng = np.random.default_rng(3)
    k = 2
    x, logits, wgu, wd, dout = _layer(rng, T=4, H=8, I=4, E=3)
    g = moe_backward(x, logits, wgu, wd, dout, k, dtype="f64")
    eps = 1e-6
    idx, _ = route(logits, k)
    used = sorted(set(idx.ravel().tolist()))
    for name, base, grad in (("x", x, g["dx"]), ("w_gate_up", wgu, g["dw_gate_up"]),
                             ("w_down", wd, g["dw_down"])):
        cells = [tuple(int(rng.integers(0, n)) for n in base.shape) for _ in range(6)]
        if name != "x":                               # include cells of used experts
            cells += [(used[0],) + tuple(int(rng.integers(0, n)) for n in base.shape[1:])]
        for c in cells:
            d = np.zeros_like(base)
            d[c] = eps
            args = {"x": x, "w_gate_up": wgu, "w_down": wd}
            p = dict(args, **{name: base + d})
            m = dict(args, **{name: base - d})
            fd = (_loss(p["x"], logits, p["w_gate_up"], p["w_down"], dout, k)
                  - _loss(m["x"], logits, m["w_gate_up"], m["w_down"], dout, k)) / (2 * eps)
            assert abs(fd - grad[c]) <= 1e-6 * max(1.0, abs(grad[c])), (name, c, fd, grad[c])


def test_logit_gradient_finite_differences():
    rng = np.random.default_rng(5)
    T, E, k = 3, 6, 3
    x, _, wgu, wd, dout = _layer(rng, T=T, H=8, I=4, E=E)
    # well separated logits (gaps of 0.25), so a step of 2^-10 keeps the selection
    logits = np.stack([rng.permutation(E) * 0.25 for _ in range(T)]).astype(np.float32)
    g = moe_backward(x, logits, wgu, wd, dout, k, dtype="f64")
    step = np.float32(2.0 ** -10)                     # exact in FP32 for |l| < 2^13
    for t in range(T):
        for e in range(E):
            lp = logits.copy()
            lm = logits.copy()
            lp[t, e] += step
            lm[t, e] -= step
            assert float(lp[t, e]) - float(lm[t, e]) == 2 * float(step)
            fd = (_loss(x, lp, wgu, wd, dout, k) - _loss(x, lm, wgu, wd, dout, k)) / (2 * float(step))
            an = g["dlogits"][t, e]
            assert abs(fd - an) <= 1e-5 * max(1.0, abs(an)), (t, e, fd, an)
        # softmax over the selection: shifting all selected logits changes nothing
        assert abs(np.sum(g["dlogits"][t])) <= 1e-12 * max(1.0, np.max(np.abs(g["dlogits"][t])))


def _torch_layer(x, logits, wgu, wd, k):
    """The layer in torch float64 operations (selection from the oracle's route,
    held fixed), for torch.autograd."""
    idx, _ = route(logits.detach().numpy().astype(np.float32), k)
    idx_t = torch.as_tensor(idx)
    sel = torch.gather(logits, 1, idx_t)
    w = torch.softmax(sel, dim=1)
    I = wgu.shape[1] // 2
    out = torch.zeros_like(x)
    for t in range(x.shape[0]):
        for j in range(k):
            e = int(idx[t, j])
            g = wgu[e, :I] @ x[t]
            u = wgu[e, I:] @ x[t]
            a = torch.nn.functional.silu(g) * u
            out[t] = out[t] + w[t, j] * (wd[e] @ a)
    return out


@pytest.mark.parametrize("k", [1, 2, 4])
def test_matches_torch_autograd(k):
    rng = np.random.default_rng(20 + k)
    x, logits, wgu, wd, dout = _layer(rng, T=5, H=12, I=6, E=6)
    g = moe_backward(x, logits, wgu, wd, dout, k, dtype="f64")
    xt = torch.tensor(x, requires_grad=True)
    lt = torch.tensor(logits.astype(np.float64), requires_grad=True)
    wgt = torch.tensor(wgu, requires_grad=True)
    wdt = torch.tensor(wd, requires_grad=True)
    out = _torch_layer(xt, lt, wgt, wdt, k)
    (out * torch.tensor(dout)).sum().backward()
    for mine, ref in ((g["dx"], xt.grad), (g["dw_gate_up"], wgt.grad), (g["dw_down"], wdt.grad),
                      (g["dlogits"], lt.grad)):
        ref = ref.numpy()
        assert np.max(np.abs(mine - ref)) <= 1e-12 * max(1.0, np.max(np.abs(ref)))


def test_special_cases():
    rng = np.random.default_rng(7)
    x, logits, wgu, wd, dout = _layer(rng, T=5, H=8, I=4, E=6)
    # k = 1: the routing weight is 1 whatever the logits, so no logit gradient
    g1 = moe_backward(x, logits, wgu, wd, dout, 1, dtype="f64")
    assert np.all(g1["dlogits"] == 0.0)
    # zero output gradient: every gradient is zero
    g0 = moe_backward(x, logits, wgu, wd, np.zeros_like(dout), 2, dtype="f64")
    for key in ("dx", "dw_gate_up", "dw_down", "d_topk_w", "dlogits"):
        assert np.all(g0[key] == 0.0)
    # experts nobody routes to get zero weight gradients
    logits2 = logits.copy()
    logits2[:, 5] = -50.0
    g2 = moe_backward(x, logits2, wgu, wd, dout, 2, dtype="f64")
    assert np.all(g2["dw_gate_up"][5] == 0.0) and np.all(g2["dw_down"][5] == 0.0)


def test_subsets_equal_full_result():
    rng = np.random.default_rng(9)
    x, logits, wgu, wd, dout = _layer(rng, T=8, H=8, I=4, E=5)
    full = moe_backward(x, logits, wgu, wd, dout, 2, dtype="f64")
    tok = np.array([6, 1, 3])
    exps = np.array([4, 0])
    sub = moe_backward(x, logits, wgu, wd, dout, 2, dtype="f64", tokens=tok, experts=exps)
    # equal up to the rounding order of the BLAS products (fewer rows)
    for key, sel in (("dx", tok), ("d_topk_w", tok), ("dlogits", tok), ("dw_gate_up", exps),
                     ("dw_down", exps)):
        assert np.allclose(sub[key], full[key][sel], rtol=0, atol=1e-13), key


def test_bf16_inputs_decode_to_the_f64_layer():
    rng = np.random.default_rng(11)
    T, H, I, E, k = 4, 8, 4, 3, 2

    def bits(a):
        return torch.from_numpy(np.asarray(a, dtype=np.float32)).to(torch.bfloat16) \
            .view(torch.int16).numpy().view(np.uint16)
    x = bits(rng.standard_normal((T, H)))
    logits = rng.standard_normal((T, E)).astype(np.float32)
    wgu = bits(rng.standard_normal((E, 2 * I, H)) * 0.4)
    wd = bits(rng.standard_normal((E, H, I)) * 0.4)
    dout = bits(rng.standard_normal((T, H)))
    gb = moe_backward(x, logits, wgu, wd, dout, k, dtype="bf16")
    gf = moe_backward(bf16_decode(x), logits, bf16_decode(wgu), bf16_decode(wd),
                      bf16_decode(dout), k, dtype="f64")
    for key in ("dx", "dw_gate_up", "dw_down", "d_topk_w", "dlogits"):
        assert np.array_equal(gb[key], gf[key])
