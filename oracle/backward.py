"""Backward pass of the routed MoE FFN layer, written out in float64.

TEST INFRASTRUCTURE ONLY (see the package header).

The Mixture-of-Kittens summary measures the layer's backward pass beside its
forward pass, in BF16 and in MXFP8 ("What is 2.37x measured against"), and
says that its backward walks the dispatch/combine ring in reverse ("Where pull
was faster than push").  The pages give no formulas for it; the gradient of
the layer defined in ``moe.py`` is fixed by calculus, and this module writes
it out.  Readings (also listed in the design notes of the repository):

  B1  the gradient is that of the exact layer (``moe_forward`` with
      h_round="exact"), of the scalar L = sum(dout * out) for a given output
      gradient dout [T, H]; the top-k selection is held fixed (it is piecewise
      constant in the logits), so gradients reach the selected logits only,
      through the renormalised softmax weights.
  B2  results: dx [T, H], dW_gate_up [E, 2I, H], dW_down [E, H, I], the
      gradient of the routing weights d_topk_w [T, k] (slot order) and of the
      router logits dlogits [T, E].

With a = silu(g) * u, y = W_down[e] a and out[t] = sum_j w_j y_j, for each
routed pair (t, j) -> e:
    dy       = w_j * dout[t]
    dw_j     = dout[t] . y_j
    da       = W_down[e]^T dy
    dg       = da * u * silu'(g),   du = da * silu(g)
    dx[t]   += W_gate[e]^T dg + W_up[e]^T du
    dW_down[e]    += dy a^T
    dW_gate_up[e] += [dg; du] x[t]^T
and, for the softmax over the k selected logits, dl_m = w_m (dw_m - sum_j w_j dw_j)
for a selected expert m, 0 for the others.
"""
from __future__ import annotations

from typing import Optional

import numpy as np

from .formats import bf16_decode, mx_dequantize, mx_quantize
from .moe import _expert_matrix, route, silu


def sigmoid(z: np.ndarray) -> np.ndarray:
    """1 / (1 + e^-z), evaluated without overflow for either sign."""
    z = np.asarray(z, dtype=np.float64)
    out = np.empty_like(z)
    pos = z >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-z[pos]))
    ez = np.exp(z[~pos])
    out[~pos] = ez / (1.0 + ez)
    return out


def silu_grad(z: np.ndarray) -> np.ndarray:
    """d/dz [z sigmoid(z)] = s (1 + z (1 - s)), s = sigmoid(z)."""
    s = sigmoid(z)
    return s * (1.0 + np.asarray(z, dtype=np.float64) * (1.0 - s))


def moe_backward(x, logits, w_gate_up, w_down, dout, k: int, dtype: str = "bf16",
                 tokens=None, experts=None):
    """Gradients of L = sum(dout * moe_forward(...)) (readings B1, B2).

    x, logits, w_gate_up, w_down, k: as for ``moe_forward`` (dtype "bf16":
    BF16 bit patterns, weights may be callables e -> [R, K]; dtype "f64":
    float64 values).  dout [T, H]: BF16 bits ("bf16") or float64 ("f64").
    tokens: optional token ids; dx, d_topk_w and dlogits are returned for
        these rows only (each depends on its own token alone).
    experts: optional expert ids; dW_gate_up and dW_down are returned for these
        experts only, stacked in the given order (each depends on every token
        routed to that expert).
    Returns a dict with dx, d_topk_w, dlogits (rows of ``tokens``), dw_gate_up,
    dw_down (rows of ``experts``), and the routing idx, w of all tokens."""
    if dtype not in ("bf16", "f64"):
        raise ValueError(dtype)
    fdt = np.float64 if dtype == "f64" else np.uint16
    x = np.asarray(x, dtype=fdt)
    xf = x if dtype == "f64" else bf16_decode(x)
    dof = np.asarray(dout, dtype=fdt)
    dof = dof if dtype == "f64" else bf16_decode(dof)
    T, H = xf.shape
    if dof.shape != (T, H):
        raise ValueError("dout must be [T, H]")
    idx, w = route(logits, k)
    E = np.asarray(logits).shape[1]

    tok = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)
    exps = np.arange(E) if experts is None else np.asarray(experts, dtype=np.int64)
    tpos = np.full(T, -1, dtype=np.int64)
    tpos[tok] = np.arange(tok.size)
    want_e = np.zeros(E, dtype=bool)
    want_e[exps] = True

    n = tok.size
    dx = np.zeros((n, H), dtype=np.float64)
    dtw = np.zeros((n, k), dtype=np.float64)
    dwgu = None
    dwd = None

    touched = set(int(e) for e in np.unique(idx[tok])) | set(int(e) for e in exps)
    for e in sorted(touched):
        rows, slots = np.nonzero(idx == e)           # every (t, j) routed to e
        if not want_e[e]:                            # only the pairs of the asked tokens
            keep = tpos[rows] >= 0
            rows, slots = rows[keep], slots[keep]
        wgu = _expert_matrix(w_gate_up, e, dtype)    # [2I, H]
        wd = _expert_matrix(w_down, e, dtype)        # [H, I]
        I = wgu.shape[0] // 2
        if dwgu is None:
            dwgu = np.zeros((exps.size, 2 * I, H), dtype=np.float64)
            dwd = np.zeros((exps.size, H, I), dtype=np.float64)
        if rows.size == 0:
            continue                                 # an asked expert nobody routed to
        xe = xf[rows]
        g = xe @ wgu[:I].T
        u = xe @ wgu[I:].T
        a = silu(g) * u
        y = a @ wd.T
        dy = w[rows, slots][:, None] * dof[rows]     # dL/dy per pair
        dw_pair = np.sum(dof[rows] * y, axis=1)      # dL/dw per pair
        da = dy @ wd
        dg = da * u * silu_grad(g)
        du = da * silu(g)
        dgu = np.concatenate([dg, du], axis=1)       # [n_e, 2I]
        if want_e[e]:
            for q in np.nonzero(exps == e)[0]:
                dwd[q] = dy.T @ a
                dwgu[q] = dgu.T @ xe
        sel = tpos[rows] >= 0
        np.add.at(dx, tpos[rows[sel]], dgu[sel] @ wgu)
        dtw[tpos[rows[sel]], slots[sel]] = dw_pair[sel]

    wt = w[tok]
    dl = np.zeros((n, E), dtype=np.float64)
    s = np.sum(wt * dtw, axis=1, keepdims=True)
    np.put_along_axis(dl, idx[tok], wt * (dtw - s), axis=1)
    if dwgu is None:                                 # no expert touched: shapes from the weights
        I = _expert_matrix(w_gate_up, 0, dtype).shape[0] // 2
        dwgu = np.zeros((exps.size, 2 * I, H), dtype=np.float64)
        dwd = np.zeros((exps.size, H, I), dtype=np.float64)
    return {"dx": dx, "d_topk_w": dtw, "dlogits": dl, "dw_gate_up": dwgu, "dw_down": dwd,
            "idx": idx, "w": w}


def _mx_round_trip(m: np.ndarray) -> np.ndarray:
    """MX quantization of a matrix along its last axis, decoded back (exact)."""
    return mx_dequantize(*mx_quantize(m))


def _along_pairs(m: np.ndarray, quant) -> np.ndarray:
    """Quantize an [n, C] matrix along its first (routed-pair) axis: the pairs
    form blocks of 32 from the first one, the last block zero-padded."""
    n, C = m.shape
    pad = (-n) % 32
    mt = np.concatenate([m.T, np.zeros((C, pad))], axis=1) if pad else m.T
    return quant(mt)[:, :n]                      # [C, n]


def moe_backward_mxfp8(x, logits, w_gate_up, w_gate_up_scales, w_down, w_down_scales, dout,
                       k: int, tokens=None, experts=None, quant=None):
    """Backward pass of the MXFP8 layer (readings B1, B2 and BQ).

    BQ (the pages give the MXFP8 backward's speed only): the gradients are those
    of the layer of ``moe_forward(dtype="mxfp8")`` with its FP64 pre-activations
    g, u = W_gate_up[e] q(x) (weights decoded, x MX-quantized along H), and each
    matrix product of the backward takes both operands MX-quantized along that
    product's own reduction axis (blocks of 32), from these values:
      dh        = q_H(dout[t]) . q_H(W_down[e] columns)          (reduction over H)
      da        = w * dh;  dg = da * u * silu'(g);  du = da * silu(g)
      dx[t]    += q_2I([dg; du]) . q_2I(W_gate_up[e] columns)    (over 2I)
      dW_down[e]    = q_P(w dout)^T q_P(a)     a = silu(g) * u   (over e's pairs)
      dW_gate_up[e] = q_P([dg; du])^T q_P(x)                     (over e's pairs)
      d_topk_w[t, j] = a . dh   (the routing weight's gradient dout . y, formed
                                 from the same product dh)
    q_P quantizes along the expert's routed pairs in token order, blocks of 32
    from its first pair, the last block zero-padded.  The weights' decoded MX
    values, x and dout (BF16) and the unquantized a and [dg; du] are the values
    quantized; x's forward quantization along H is used only for g and u.

    x, dout [T, H] BF16 bits; logits [T, E] FP32; w_gate_up [E, 2I, H] and
    w_down [E, H, I] E4M3 codes with E8M0 scales [.., K/32] (arrays or callables
    e -> one expert's matrix).  tokens / experts as for ``moe_backward``.
    ``quant`` replaces the MX round trip along the last axis (a test hook)."""
    q = _mx_round_trip if quant is None else quant
    xb = bf16_decode(np.asarray(x, dtype=np.uint16))
    dof = bf16_decode(np.asarray(dout, dtype=np.uint16))
    T, H = xb.shape
    if dof.shape != (T, H):
        raise ValueError("dout must be [T, H]")
    idx, w = route(logits, k)
    E = np.asarray(logits).shape[1]

    tok = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)
    exps = np.arange(E) if experts is None else np.asarray(experts, dtype=np.int64)
    tpos = np.full(T, -1, dtype=np.int64)
    tpos[tok] = np.arange(tok.size)
    want_e = np.zeros(E, dtype=bool)
    want_e[exps] = True
    n = tok.size
    dx = np.zeros((n, H), dtype=np.float64)
    dtw = np.zeros((n, k), dtype=np.float64)
    dwgu = dwd = None

    touched = set(int(e) for e in np.unique(idx[tok])) | set(int(e) for e in exps)
    for e in sorted(touched):
        rows, slots = np.nonzero(idx == e)       # every (t, j) routed to e, tokens ascending
        wgu = _expert_matrix(w_gate_up, e, "mxfp8", w_gate_up_scales)   # [2I, H]
        wd = _expert_matrix(w_down, e, "mxfp8", w_down_scales)          # [H, I]
        I = wgu.shape[0] // 2
        if dwgu is None:
            dwgu = np.zeros((exps.size, 2 * I, H), dtype=np.float64)
            dwd = np.zeros((exps.size, H, I), dtype=np.float64)
        if rows.size == 0:
            continue
        if not want_e[e]:                        # only the pairs of the asked tokens
            keep = tpos[rows] >= 0
            rows, slots = rows[keep], slots[keep]
        xq = q(xb[rows])                         # the forward's x, along H (row by row)
        g = xq @ wgu[:I].T
        u = xq @ wgu[I:].T
        a = silu(g) * u
        wp = w[rows, slots][:, None]
        dh = q(dof[rows]) @ q(wd.T).T            # [n_e, I], reduction over H
        da = wp * dh
        dgu = np.concatenate([da * u * silu_grad(g), da * silu(g)], axis=1)   # [n_e, 2I]
        dtw_pair = np.sum(a * dh, axis=1)
        if want_e[e]:
            dy = wp * dof[rows]                  # [n_e, H]
            for qq in np.nonzero(exps == e)[0]:
                dwd[qq] = _along_pairs(dy, q) @ _along_pairs(a, q).T
                dwgu[qq] = _along_pairs(dgu, q) @ _along_pairs(xb[rows], q).T
        sel = tpos[rows] >= 0
        dxe = q(dgu[sel]) @ q(wgu.T).T          # [n_sel, H], reduction over 2I
        np.add.at(dx, tpos[rows[sel]], dxe)
        dtw[tpos[rows[sel]], slots[sel]] = dtw_pair[sel]

    wt = w[tok]
    dl = np.zeros((n, E), dtype=np.float64)
    s = np.sum(wt * dtw, axis=1, keepdims=True)
    np.put_along_axis(dl, idx[tok], wt * (dtw - s), axis=1)
    if dwgu is None:
        I = _expert_matrix(w_gate_up, 0, "mxfp8", w_gate_up_scales).shape[0] // 2
        dwgu = np.zeros((exps.size, 2 * I, H), dtype=np.float64)
        dwd = np.zeros((exps.size, H, I), dtype=np.float64)
    return {"dx": dx, "d_topk_w": dtw, "dlogits": dl, "dw_gate_up": dwgu, "dw_down": dwd,
            "idx": idx, "w": w}


__all__ = ["sigmoid", "silu_grad", "moe_backward", "moe_backward_mxfp8"]
