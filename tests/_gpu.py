"""Helpers shared by the GPU parity tests: move data to the oracle, run it, compare."""
import concurrent.futures as cf
from collections import OrderedDict

import numpy as np
import torch

from oracle import formats as F
from oracle import moe_backward, moe_forward, route
from oracle.moe import max_abs_ratio, rel_l2

BF16_REL_L2 = 5e-3          # relative L2 bound for BF16 outputs
BF16_MAX_ABS = 1e-2         # max |got - ref| <= this * max |ref|
MXFP8_REL_L2 = 3e-2         # relative L2 bound for MXFP8 outputs (quantization-aware oracle)
W_ABS = 1e-6                # routing weights: FP32 path vs FP64 oracle


def bits(t: torch.Tensor) -> np.ndarray:
    """BF16 tensor (any device) -> numpy uint16 bit patterns."""
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def u8(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().cpu().numpy()


class Fetch:
    """Callable e -> one expert's weights as numpy, copied from the GPU on demand."""

    def __init__(self, t: torch.Tensor):
        self.t = t

    def __call__(self, e):
        w = self.t[int(e)]
        return bits(w) if w.dtype == torch.bfloat16 else u8(w)


_POOL = None


def _pool():
    global _POOL
    if _POOL is None:
        _POOL = cf.ThreadPoolExecutor(max_workers=8)
    return _POOL


class Decoded:
    """Callable e -> one expert's weight matrix as float64, decoded by the
    oracle's own codecs (BF16, or E4M3 codes times E8M0 block scales) in
    worker threads a few experts ahead of the oracle's requests.  `order` is
    the order the oracle asks for experts in (ascending ids); each matrix is
    dropped once handed over, so at most `window` are held at a time.  The
    values are exactly those the oracle's own decoding of the same expert
    gives (checked on the CPU by tests/test_gpu_helpers.py)."""

    def __init__(self, w: torch.Tensor, scales: torch.Tensor = None, order=(), window=12):
        self.w, self.s = w, scales
        self.order = [int(e) for e in order]
        self.pos = 0
        self.window = window
        self.fut = OrderedDict()

    def _decode(self, e):
        we = self.w[e]
        if self.s is None:
            return F.bf16_decode(bits(we))
        return F.mx_dequantize(u8(we), u8(self.s[e]))

    def _fill(self):
        while len(self.fut) < self.window and self.pos < len(self.order):
            e = self.order[self.pos]
            self.pos += 1
            if e not in self.fut:
                self.fut[e] = _pool().submit(self._decode, e)

    def __call__(self, e):
        e = int(e)
        self._fill()
        f = self.fut.pop(e, None)
        m = f.result() if f is not None else self._decode(e)
        self._fill()
        return m


def oracle(d, tokens=None, return_intermediates=False):
    """Run the FP64 oracle on a workload dict (tensors may live on the GPU),
    for every token or for the listed ones.

    The oracle runs in its float64-input mode on inputs decoded by its own
    codecs: x from BF16 (and, for MXFP8 workloads, MX-quantized along H as
    its MXFP8 mode does), the experts' weights from BF16 or E4M3 + E8M0 by
    `Decoded`, and the activations MX-quantized along I (h_round="mxfp8") for
    MXFP8.  That is the same computation as its "bf16" / "mxfp8" modes, with
    the weight decoding done ahead in threads."""
    cfg = d["cfg"]
    logits = d["logits"].detach().cpu().numpy()
    xb = bits(d["x"])
    if tokens is not None:
        tokens = np.asarray(tokens, dtype=np.int64)
        xb, logits = xb[tokens], logits[tokens]
    x = F.bf16_decode(xb)
    h_round = "exact"
    sg = sd = None
    if cfg.dtype == "mxfp8":
        x = F.mx_dequantize(*F.mx_quantize(x))
        h_round = "mxfp8"
        sg, sd = d["w_gate_up_scales"], d["w_down_scales"]
    order = np.unique(route(logits, cfg.k)[0])
    return moe_forward(x, logits, Decoded(d["w_gate_up"], sg, order),
                       Decoded(d["w_down"], sd, order), cfg.k, dtype="f64", h_round=h_round,
                       return_intermediates=return_intermediates)


def oracle_backward(d, dout: torch.Tensor, tokens=None, experts=None):
    """The FP64 backward oracle on a BF16 workload dict, in its float64-input
    mode on inputs decoded by its own BF16 codec (weights decoded ahead in
    threads by `Decoded`): the same computation as its "bf16" mode."""
    cfg = d["cfg"]
    logits = d["logits"].detach().cpu().numpy()
    idx, _ = route(logits, cfg.k)
    tok = np.arange(cfg.T) if tokens is None else np.asarray(tokens, dtype=np.int64)
    exps = np.arange(cfg.E) if experts is None else np.asarray(experts, dtype=np.int64)
    order = sorted(set(np.unique(idx[tok]).tolist()) | set(exps.tolist()))
    return moe_backward(F.bf16_decode(bits(d["x"])), logits, Decoded(d["w_gate_up"], None, order),
                        Decoded(d["w_down"], None, order), F.bf16_decode(bits(dout)), cfg.k,
                        dtype="f64", tokens=tokens, experts=experts)


def sample_tokens(logits: np.ndarray, k: int, n: int, seed: int, tile_rows=(64, 128, 256),
                  n_focus: int = 6):
    """At least n token ids (ascending) for a sampled parity check of a full-size
    batch.  The grouped kernels take each expert's routed rows in token order
    and cut them into M-tiles of one of `tile_rows`; the sample holds, for the
    most- and the least-loaded expert and n_focus others: the expert's first and
    last token, and the first and a middle token of its last (ragged) M-tile at
    every tile height; random tokens fill up the rest."""
    idx, _ = route(logits, k)
    T = idx.shape[0]
    E = logits.shape[1]
    counts = np.bincount(idx.ravel(), minlength=E)
    used = np.nonzero(counts)[0]
    rng = np.random.default_rng(seed)
    heavy = int(used[np.argmax(counts[used])])
    light = int(used[np.argmin(counts[used])])
    others = [int(e) for e in rng.permutation(used) if e not in (heavy, light)][:n_focus]
    pick = set()
    for e in [heavy, light] + others:
        toks = np.nonzero((idx == e).any(axis=1))[0]
        c = toks.size
        pick.update((int(toks[0]), int(toks[-1])))
        for bm in tile_rows:
            last = (c - 1) // bm * bm
            pick.update((int(toks[last]), int(toks[(last + c - 1) // 2])))
    rest = [t for t in rng.permutation(T) if int(t) not in pick]
    pick.update(int(t) for t in rest[:max(0, n - len(pick))])
    return np.array(sorted(pick), dtype=np.int64), {"heavy": heavy, "light": light,
                                                    "counts": counts}


def to_f64(out: torch.Tensor) -> np.ndarray:
    return out.detach().cpu().double().numpy()


def check_bf16(got: torch.Tensor, ref: np.ndarray, what: str = ""):
    g = to_f64(got)
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    rl, ma = rel_l2(g, ref), max_abs_ratio(g, ref)
    print(f"[parity] {what}: rel_l2={rl:.3e} max_abs/max={ma:.3e}", flush=True)
    assert rl <= BF16_REL_L2, f"{what}: rel_l2 {rl:.3e} > {BF16_REL_L2}"
    assert ma <= BF16_MAX_ABS, f"{what}: max-abs ratio {ma:.3e} > {BF16_MAX_ABS}"
    return rl, ma
