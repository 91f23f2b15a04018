"""The routed MoE FFN layer, written out in float64.

What the layer computes (warp-decode article, "Background" and "Key points";
Mixture-of-Kittens summary, "What is 2.37x measured against"):
for every token, route to k experts, run each routed expert's gated FFN
(gate/up projection, gated activation, down projection), and sum the routed
experts' outputs with their routing weights into the token's output.

Readings taken where the pages are silent (each one also listed in the design
notes of the repository):
  R1  selection is on the FP32 router logits: experts are ordered by (logit
      descending, expert index ascending) and the first k are kept; slot j of
      a token is the j-th expert in that order.  +0 and -0 compare equal, so
      they tie and the lower index wins.  Non-finite logits are rejected.
  R2  routing weights are softmax over the selected logits, i.e. softmax over
      all E followed by renormalisation over the k selected ("renormalised
      top-k"): w_j = exp(l_j - l_0) / sum_i exp(l_i - l_0).
  F1  w_gate_up[e] is [2I, H]: rows [0, I) are the gate projection, rows
      [I, 2I) the up projection ("gate_up" kernel name, warp-decode article).
  F2  the gated activation is SwiGLU: a = silu(g) * u, silu(z) = z / (1 + e^-z)
      ("Qwen-3 style", warp-decode article, "Key points").
  F3  w_down[e] is [H, I]; y = w_down[e] @ a.
  C   out[t] = sum_j w_j * y[t, j] in slot order; no rounding anywhere (the
      GPU rounds its FP32 result to BF16 once, at the end).
  Q   MXFP8 mode: both operands of both projections are MX-quantized: the
      weights arrive as E4M3 + E8M0 codes and are decoded exactly; x is
      quantized along H and a along I with the rule in ``formats``.  No
      capacity limit, no token dropping, no shared expert.
"""
from __future__ import annotations

from typing import Optional, Sequence, Union

import numpy as np

from .formats import bf16_decode, bf16_round, mx_dequantize, mx_quantize

ArrayLike = Union[np.ndarray, Sequence]


def route(logits: ArrayLike, k: int):
    """Top-k selection (R1) and renormalised softmax weights (R2).

    logits: [T, E] float32 (converted exactly to float64).
    Returns (idx int64 [T, k], w float64 [T, k]) in slot order."""
    l32 = np.asarray(logits, dtype=np.float32)
    if l32.ndim != 2:
        raise ValueError("logits must be [T, E]")
    T, E = l32.shape
    if not 1 <= k <= E:
        raise ValueError(f"k={k} outside [1, E={E}]")
    if not np.all(np.isfinite(l32)):
        raise ValueError("route: non-finite logit")
    l = l32.astype(np.float64)
    experts = np.broadcast_to(np.arange(E), (T, E))
    # np.lexsort sorts by the last key first: primary -l ascending (= l
    # descending), secondary expert index ascending.  -0.0 == +0.0 ties.
    order = np.lexsort((experts, -l), axis=-1)
    idx = order[:, :k].astype(np.int64)
    sel = np.take_along_axis(l, idx, axis=1)
    ex = np.exp(sel - sel[:, :1])
    w = ex / ex.sum(axis=1, keepdims=True)
    return idx, w


def silu(z: np.ndarray) -> np.ndarray:
    """z * sigmoid(z), evaluated without overflow for either sign."""
    z = np.asarray(z, dtype=np.float64)
    out = np.empty_like(z)
    pos = z >= 0
    out[pos] = z[pos] / (1.0 + np.exp(-z[pos]))
    ez = np.exp(z[~pos])
    out[~pos] = z[~pos] * ez / (1.0 + ez)
    return out


def _expert_matrix(w, e: int, dtype: str, scales=None) -> np.ndarray:
    """Decode one expert's weight matrix to float64.

    ``w`` is either an array [E, R, K] or a callable e -> array [R, K] (lets a
    caller fetch only the experts it needs)."""
    we = w(e) if callable(w) else np.asarray(w[e])
    if dtype == "f64":
        return np.asarray(we, dtype=np.float64)
    if dtype == "bf16":
        return bf16_decode(we)
    se = scales(e) if callable(scales) else np.asarray(scales[e])
    return mx_dequantize(we, se)


def moe_forward(x, logits, w_gate_up, w_down, k: int, dtype: str = "bf16",
                w_gate_up_scales=None, w_down_scales=None,
                tokens: Optional[ArrayLike] = None,
                return_intermediates: bool = False, h_round: str = "exact"):
    """The whole layer in float64.

    x           [T, H] uint16 BF16 bit patterns
    logits      [T, E] float32
    w_gate_up   [E, 2I, H] uint16 BF16 bits, or uint8 E4M3 codes (dtype="mxfp8")
                with w_gate_up_scales [E, 2I, H/32] uint8 E8M0; either may be a
                callable e -> that expert's [2I, H] matrix
    w_down      [E, H, I] likewise (scales [E, H, I/32])
    tokens      optional subset of token ids: only those rows are computed
                (every token's output depends on that token alone)
    h_round     rounding of the gated activations a before the down projection,
                for the accuracy comparison the warp-decode article draws
                ("Comparison": no quantized intermediate activations): "exact"
                (none, the default), "bf16" (round to nearest even), "mxfp8"
                (E4M3 + E8M0 blocks of 32 along I, the MXFP8 mode's rule).  In
                MXFP8 mode a is always MX-quantized and h_round must be "exact".
    dtype "f64" takes x and the weights as float64 values (no decoding): the
    real-valued layer, for derivative checks by finite differences.
    Returns out [n_tokens, H] float64, or (out, dict) with the routing, the
    per-slot pre-activations gu [n, k, 2I] (gate then up), activations
    a [n, k, I] and expert outputs y [n, k, H]."""
    if dtype not in ("bf16", "mxfp8", "f64"):
        raise ValueError(dtype)
    if h_round not in ("exact", "bf16", "mxfp8") or (dtype == "mxfp8" and h_round != "exact"):
        raise ValueError(h_round)
    x = np.asarray(x, dtype=np.float64 if dtype == "f64" else np.uint16)
    logits = np.asarray(logits, dtype=np.float32)
    if tokens is not None:
        tokens = np.asarray(tokens, dtype=np.int64)
        x = x[tokens]
        logits = logits[tokens]
    T, H = x.shape
    idx, w = route(logits, k)

    xf = x if dtype == "f64" else bf16_decode(x)
    if dtype == "mxfp8":
        xf = mx_dequantize(*mx_quantize(xf))

    a_all: Optional[np.ndarray] = None
    gu_all: Optional[np.ndarray] = None
    y = np.zeros((T, k, H), dtype=np.float64)
    for e in np.unique(idx):
        rows, slots = np.nonzero(idx == e)           # every (t, j) routed to e
        wgu = _expert_matrix(w_gate_up, int(e), dtype, w_gate_up_scales)   # [2I, H]
        wd = _expert_matrix(w_down, int(e), dtype, w_down_scales)          # [H, I]
        I = wgu.shape[0] // 2
        if wgu.shape != (2 * I, H) or wd.shape != (H, I):
            raise ValueError("weight shapes do not match x")
        xe = xf[rows]                                # [n_e, H]
        g = xe @ wgu[:I].T                           # gate projection
        u = xe @ wgu[I:].T                           # up projection
        a = silu(g) * u                              # SwiGLU
        if dtype == "mxfp8" or h_round == "mxfp8":
            a = mx_dequantize(*mx_quantize(a))
        elif h_round == "bf16":
            a = bf16_round(a)
        y[rows, slots] = a @ wd.T                    # down projection
        if return_intermediates:
            if a_all is None:
                a_all = np.zeros((T, k, I), dtype=np.float64)
                gu_all = np.zeros((T, k, 2 * I), dtype=np.float64)
            a_all[rows, slots] = a
            gu_all[rows, slots, :I] = g
            gu_all[rows, slots, I:] = u

    out = np.zeros((T, H), dtype=np.float64)
    for j in range(k):                               # combine in slot order
        out += w[:, j:j + 1] * y[:, j, :]
    if return_intermediates:
        return out, {"idx": idx, "w": w, "gu": gu_all, "a": a_all, "y": y}
    return out


def rel_l2(got, ref) -> float:
    """||got - ref||_2 / ||ref||_2 over the whole tensor, in float64."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.linalg.norm((got - ref).ravel()) / np.linalg.norm(ref.ravel()))


def max_abs_ratio(got, ref) -> float:
    """max |got - ref| / max |ref|."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.max(np.abs(got - ref)) / np.max(np.abs(ref)))


__all__ = ["route", "silu", "moe_forward", "rel_l2", "max_abs_ratio"]
